// tree_draft_build: the candidate tree of each sequence, grown from the draft
// model's top-K rows.
//
// At every expansion the context's top-K probabilities are truncated by
// cumulative mass (kept in descending order until the kept mass reaches
// 1 - prune_ratio, then renormalised by it; page "端侧大模型推测解码草稿模型动态剪枝策略：
// 详解基于重要性采样的树形验证并行加速机制" (ufo.work/2026/525), §2.1.2), and each kept
// candidate gets the importance weight p^beta / sum p^beta times its parent's
// path weight; candidates are drawn one at a time with probability proportional
// to that weight, so branches are kept and deepened by sampling on the weights
// (page "端侧多模态大模型推测解码草稿模型动态剪枝：详解基于重要性采样的树形验证并行加速策略"
// (ufo.work/2026/500), §3.1).  Node i is the i-th draw (parents precede
// children, the order tree_build_index takes); row i + 1 of the input is the
// context after node i.
//
// One wavefront per sequence.  The truncation and weights of every row are
// computed before the draws (all rows are inputs); the weights, the uniforms and
// the candidates (in creation order) live in LDS, so a draw waits on no global
// memory.  A draw
// sums the weights in 64 contiguous chunks (one per lane), scans the chunk sums
// across the wavefront (DPP), and the lane whose chunk holds u * total walks it.  The
// truncation and the normaliser of the weights are summed by one lane in slot
// order; powers are one per lane.  Everything that decides a draw is fp64 with
// no contraction.
#include "tv_common.h"

#pragma clang fp contract(off)

namespace tv {

namespace {

constexpr int kMaxDraftNodes = 256;
constexpr int kMaxDraftK = 16;
constexpr int kMaxCand = kMaxDraftK * (kMaxDraftNodes + 1);

struct DraftArgs {
  const float* probs;  // [batch, rows, k]
  const float* u;      // [batch, n_max]
  int32_t* parent;     // [batch, n_max]
  int32_t* slot;
  float* q_draft;
  int32_t* count;      // [batch]
  int32_t* err;
  int rows, k, n_max, max_depth;
  float beta, prune;
};

// x of lane (lane - shift) combined by DPP (ctrl / row mask), 0 where there is no
// source lane or the row is masked off; fp64 moves as two 32-bit halves
__device__ __forceinline__ double dpp_shift(double x, int ctrl, int row_mask) {
  const int lo = __double2loint(x), hi = __double2hiint(x);
  int lo2, hi2;
  switch (ctrl) {  // the DPP control must be a constant
#define TV_DPP(c)                                                          \
  case c:                                                                  \
    lo2 = __builtin_amdgcn_update_dpp(0, lo, c, 0xf, 0xf, true);           \
    hi2 = __builtin_amdgcn_update_dpp(0, hi, c, 0xf, 0xf, true);           \
    break;
    TV_DPP(0x111) TV_DPP(0x112) TV_DPP(0x114) TV_DPP(0x118) TV_DPP(0x138)
#undef TV_DPP
    case 0x142:  // row_bcast:15 into rows 1 and 3
      lo2 = __builtin_amdgcn_update_dpp(0, lo, 0x142, 0xa, 0xf, false);
      hi2 = __builtin_amdgcn_update_dpp(0, hi, 0x142, 0xa, 0xf, false);
      break;
    default:  // 0x143, row_bcast:31 into rows 2 and 3
      lo2 = __builtin_amdgcn_update_dpp(0, lo, 0x143, 0xc, 0xf, false);
      hi2 = __builtin_amdgcn_update_dpp(0, hi, 0x143, 0xc, 0xf, false);
      break;
  }
  (void)row_mask;
  return __hiloint2double(hi2, lo2);
}

// inclusive prefix sum over the 64 lanes: shifts 1, 2, 4, 8 inside each 16-lane
// row, then the row totals broadcast into the rows after them
__device__ __forceinline__ double wave_incl_scan(double x) {
  x += dpp_shift(x, 0x111, 0xf);
  x += dpp_shift(x, 0x112, 0xf);
  x += dpp_shift(x, 0x114, 0xf);
  x += dpp_shift(x, 0x118, 0xf);
  x += dpp_shift(x, 0x142, 0xa);
  x += dpp_shift(x, 0x143, 0xc);
  return x;
}

// candidate info: context node + 1 (9 bits), slot (4 bits); depth comes from the node
__device__ __forceinline__ uint16_t pack_info(int ctx, int slot) {
  return static_cast<uint16_t>((ctx + 1) | (slot << 9));
}

// LDS layout (bytes): candidates' path weights and info, then per (row, slot)
// importance weights and renormalised probabilities, then per row / node scalars
constexpr int kRowSlots = (kMaxDraftNodes + 1) * kMaxDraftK;
constexpr int kOffW = 0;
constexpr int kOffWRow = kOffW + kMaxCand * 8;  // reads up to 3 entries past s_w land here
constexpr int kOffQ = kOffWRow + kRowSlots * 8;
constexpr int kOffInfo = kOffQ + kRowSlots * 4;
constexpr int kOffU = kOffInfo + kMaxCand * 2;
constexpr int kOffDepth = kOffU + kMaxDraftNodes * 4;
constexpr int kOffM = kOffDepth + kMaxDraftNodes * 2;
constexpr int kDraftLds = kOffM + kMaxDraftNodes + 8;

__global__ void __launch_bounds__(64) k_draft_build(DraftArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  double* s_w = reinterpret_cast<double*>(smem + kOffW);        // path weight; 0 once taken
  double* s_wrow = reinterpret_cast<double*>(smem + kOffWRow);  // importance weight (row, slot)
  float* s_q = reinterpret_cast<float*>(smem + kOffQ);          // p / kept mass (row, slot)
  uint16_t* s_info = reinterpret_cast<uint16_t*>(smem + kOffInfo);
  float* s_u = reinterpret_cast<float*>(smem + kOffU);
  int16_t* s_depth = reinterpret_cast<int16_t*>(smem + kOffDepth);
  uint8_t* s_m = reinterpret_cast<uint8_t*>(smem + kOffM);      // kept slots of each row
  const int b = blockIdx.x, lane = threadIdx.x;
  const float* P = a.probs + static_cast<long>(b) * a.rows * a.k;
  const float* U = a.u + static_cast<long>(b) * a.n_max;
  int32_t* parent = a.parent + static_cast<long>(b) * a.n_max;
  int32_t* slot = a.slot + static_cast<long>(b) * a.n_max;
  float* qd = a.q_draft + static_cast<long>(b) * a.n_max;

  for (int i = lane; i < a.n_max; i += 64) {  // padding past the count
    parent[i] = -2;
    slot[i] = -2;
    qd[i] = 0.0f;
  }
  bool bad_p = false, bad_u = false;
  for (int i = lane; i < a.rows * a.k; i += 64) {
    const float p = P[i];
    bad_p |= !(p >= 0.0f && p <= 1.0f);
  }
  for (int i = lane; i < a.n_max; i += 64) {
    const float x = U[i];
    bad_u |= !(x >= 0.0f && x < 1.0f);
    s_u[i] = x;
  }
  const int bad = (__ballot(bad_p) ? TV_ERR_DRAFT : 0) | (__ballot(bad_u) ? TV_ERR_UNIFORM : 0);
  if (bad) {
    if (lane == 0) {
      atomicOr(a.err, bad);
      a.count[b] = 0;
    }
    return;
  }

  // Every row a build can expand (rows 0 .. n_max) is known up front, so the
  // truncation, the powers and the normalised weights of all of them are
  // computed before the draws, rows and (row, slot) pairs spread over the lanes.
  // The sums keep slot order within a row.
  const int used_rows = min(a.rows, a.n_max + 1);
  const double target = 1.0 - static_cast<double>(a.prune);
  const double beta = static_cast<double>(a.beta);
  for (int r = lane; r < used_rows; r += 64) {  // kept count and mass of row r
    const float* pr = P + static_cast<long>(r) * a.k;
    int m = a.k;
    double mass = 0.0;
    for (int j = 0; j < a.k; ++j) {
      mass += static_cast<double>(pr[j]);
      if (mass >= target) {
        m = j + 1;
        break;
      }
    }
    s_m[r] = static_cast<uint8_t>(m);
    for (int j = 0; j < a.k; ++j)
      s_q[r * a.k + j] =
          mass > 0.0 ? static_cast<float>(static_cast<double>(pr[j]) / mass) : 0.0f;
  }
  __syncthreads();
  for (int i = lane; i < used_rows * a.k; i += 64) {  // p^beta of the kept slots
    const int r = i / a.k, j = i % a.k;
    const double p = static_cast<double>(P[i]);
    s_wrow[i] = j < s_m[r] && p > 0.0 ? pow(p, beta) : 0.0;
  }
  __syncthreads();
  for (int r = lane; r < used_rows; r += 64) {  // normalise over the kept slots
    const int m = s_m[r];
    double sum = 0.0;
    for (int j = 0; j < m; ++j) sum += s_wrow[r * a.k + j];
    for (int j = 0; j < m; ++j) s_wrow[r * a.k + j] = sum > 0.0 ? s_wrow[r * a.k + j] / sum : 0.0;
  }
  __syncthreads();

  int n_cand = 0;
  // candidates of context row `row` (node ctx, -1 = prefix) appended in slot order
  auto expand = [&](int row, int ctx, double ctx_pw) __attribute__((always_inline)) {
    const int m = s_m[row];
    if (lane < m) {
      s_w[n_cand + lane] = ctx_pw * s_wrow[row * a.k + lane];
      s_info[n_cand + lane] = pack_info(ctx, lane);
    }
    n_cand += m;
    __syncthreads();
  };

  expand(0, -1, 1.0);
  int n = 0;
  for (; n < a.n_max; ++n) {
    // chunk sums, then a scan of them across the wavefront
    const int chunk = (n_cand + 63) / 64;
    const int c0 = min(n_cand, lane * chunk), c1 = min(n_cand, c0 + chunk);
    // weights read 4 at a time (the LDS latency once per 4), added in candidate order;
    // entries past the chunk are read (inside the LDS block: s_wrow follows s_w) but
    // count as +0.0, which leaves a sum of non-negative weights unchanged
    double ls = 0.0;
    for (int j = c0; j < c1; j += 4) {
      double v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = s_w[j + e];
#pragma unroll
      for (int e = 0; e < 4; ++e) ls += j + e < c1 ? v[e] : 0.0;
    }
    const double incl = wave_incl_scan(ls);
    const double excl = dpp_shift(incl, 0x138, 0xf);  // wave_shr:1; lane 0 gets 0
    const double total = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(incl), 63),
                                          __builtin_amdgcn_readlane(__double2loint(incl), 63));
    if (!(total > 0.0)) break;
    const double t = static_cast<double>(s_u[n]) * total;
    const unsigned long long over = __ballot(incl > t);
    const int owner = over ? __ffsll(static_cast<long long>(over)) - 1 : 63;
    int pick = -1;
    if (lane == owner) {
      double run = excl;
      int last = -1;
      for (int j = c0; j < c1 && pick < 0; j += 4) {  // 4 weights per LDS round trip
        double v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = s_w[j + e];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (pick >= 0 || j + e >= c1) continue;
          if (v[e] > 0.0) last = j + e;
          run += v[e];
          if (run > t) pick = j + e;
        }
      }
      if (pick < 0) pick = last;  // rounding left the chunk's walk short: its last live entry
    }
    pick = __shfl(pick, owner, 64);
    if (pick < 0) break;  // unreachable while total > 0 and u < 1; keeps the LDS index valid
    const int info = s_info[pick];
    const double pw = s_w[pick];
    const int ctx = (info & 511) - 1, sl = (info >> 9) & 15;
    const int dep = ctx < 0 ? 1 : s_depth[ctx] + 1;
    __syncthreads();
    if (lane == 0) {
      parent[n] = ctx;
      slot[n] = sl;
      qd[n] = s_q[(ctx + 1) * a.k + sl];  // renormalised by the kept mass of its context row
      s_w[pick] = 0.0;
      s_depth[n] = static_cast<int16_t>(dep);
    }
    __syncthreads();
    if (dep < a.max_depth && n + 1 < a.rows) expand(n + 1, n, pw);
  }
  if (lane == 0) a.count[b] = n;
}

}  // namespace

}  // namespace tv

extern "C" int tree_draft_build(const float* probs, const float* u, int32_t batch, int32_t rows,
                                int32_t k, int32_t n_max, int32_t max_depth, float beta,
                                float prune_ratio, int32_t* parent, int32_t* slot,
                                float* q_draft, int32_t* count, int32_t* err, void* stream) {
  tv::clear_error();
  if (batch < 0) return tv::fail(TV_EINVAL, "tree_draft_build: negative batch");
  if (rows < 1 || k < 1 || n_max < 1 || max_depth < 1)
    return tv::fail(TV_EINVAL, "tree_draft_build: rows, k, n_max and max_depth must be >= 1");
  if (k > tv::kMaxDraftK || n_max > tv::kMaxDraftNodes || max_depth > tv::kMaxDraftNodes)
    return tv::fail(TV_EUNSUPPORTED, "tree_draft_build: k <= 16, n_max <= 256, max_depth <= 256");
  if (!(beta >= 0.0f) || beta == INFINITY)
    return tv::fail(TV_EINVAL, "tree_draft_build: beta must be finite and >= 0");
  if (!(prune_ratio >= 0.0f && prune_ratio <= 1.0f))
    return tv::fail(TV_EINVAL, "tree_draft_build: prune_ratio must be in [0, 1]");
  if (err == nullptr) return tv::fail(TV_EINVAL, "tree_draft_build: null err");
  if (batch == 0) return TV_OK;
  if (probs == nullptr || u == nullptr || parent == nullptr || slot == nullptr ||
      q_draft == nullptr || count == nullptr)
    return tv::fail(TV_EINVAL, "tree_draft_build: null input or output");
  tv::DraftArgs a{};
  a.probs = probs;
  a.u = u;
  a.parent = parent;
  a.slot = slot;
  a.q_draft = q_draft;
  a.count = count;
  a.err = err;
  a.rows = rows;
  a.k = k;
  a.n_max = n_max;
  a.max_depth = max_depth;
  a.beta = beta;
  a.prune = prune_ratio;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&tv::k_draft_build),
                              hipFuncAttributeMaxDynamicSharedMemorySize, tv::kDraftLds);
    attr_set = true;
  }
  hipLaunchKernelGGL(tv::k_draft_build, dim3(batch), dim3(64), tv::kDraftLds,
                     static_cast<hipStream_t>(stream), a);
  return tv::check_launch("tree_draft_build");
}
