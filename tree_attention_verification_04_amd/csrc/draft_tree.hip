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
// memory.  Lane c keeps the sum of the weights of candidates 128c .. 128c + 127 in
// a register (new candidates join it as they are created; the chunk a draw takes
// from is summed afresh).  A draw scans the chunk sums across the wavefront (DPP),
// the first chunk whose running sum passes u * total is read by the whole
// wavefront, two candidates a lane, in one LDS round trip, and a second scan finds
// the candidate.  The truncation and the normaliser of the weights are summed by
// one lane in slot order; powers are one per lane.  Everything that decides a
// draw is fp64 with no contraction.
#include "tv_common.h"

#pragma clang fp contract(off)

namespace tv {

namespace {

constexpr int kMaxDraftNodes = 256;
constexpr int kMaxDraftK = 16;
constexpr int kMaxCand = kMaxDraftK * (kMaxDraftNodes + 1);
constexpr int kChunk = 128;                                // candidates per lane's chunk
constexpr int kChunks = (kMaxCand + kChunk - 1) / kChunk;  // 33
constexpr int kCandCap = kChunks * kChunk;                 // whole chunks are read
static_assert(kChunks <= 64, "one chunk per lane");

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

// inclusive prefix sum inside each 16-lane row (shifts 1, 2, 4, 8)
__device__ __forceinline__ double row_incl_scan(double x) {
  x += dpp_shift(x, 0x111, 0xf);
  x += dpp_shift(x, 0x112, 0xf);
  x += dpp_shift(x, 0x114, 0xf);
  x += dpp_shift(x, 0x118, 0xf);
  return x;
}

// inclusive prefix sum over the 64 lanes: the row scans, then the row totals
// broadcast into the rows after them (lanes 0-15 end as the row scan left them)
__device__ __forceinline__ double wave_incl_scan(double x) {
  x = row_incl_scan(x);
  x += dpp_shift(x, 0x142, 0xa);
  x += dpp_shift(x, 0x143, 0xc);
  return x;
}

// a double of lane `src` (uniform) in every lane
__device__ __forceinline__ double readlane_f64(double x, int src) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), src),
                          __builtin_amdgcn_readlane(__double2loint(x), src));
}

// candidate info: context node + 1 (9 bits), slot (4 bits), depth of the node it
// would become (9 bits)
__device__ __forceinline__ uint32_t pack_info(int ctx, int slot, int depth) {
  return static_cast<uint32_t>((ctx + 1) | (slot << 9) | (depth << 13));
}

// LDS layout (bytes): candidates' path weights and info, then per (row, slot)
// importance weights and renormalised probabilities, then per row / node scalars
constexpr int kRowSlots = (kMaxDraftNodes + 1) * kMaxDraftK;
constexpr int kOffW = 0;
constexpr int kOffWRow = kOffW + kCandCap * 8;
constexpr int kOffQ = kOffWRow + kRowSlots * 8;
constexpr int kOffInfo = kOffQ + kRowSlots * 4;  // whole chunks are read
constexpr int kOffU = kOffInfo + kCandCap * 4;
constexpr int kOffM = kOffU + kMaxDraftNodes * 4;
// the built nodes' outputs, written out once after the draws (so a draw never
// waits for a global store to complete)
constexpr int kOffPOut = (kOffM + kMaxDraftNodes + 8 + 1) & ~1;
constexpr int kOffSOut = kOffPOut + kMaxDraftNodes * 2;
constexpr int kDraftLds = kOffSOut + kMaxDraftNodes;

__global__ void __launch_bounds__(64) k_draft_build(DraftArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  double* s_w = reinterpret_cast<double*>(smem + kOffW);        // path weight; 0 once taken
  double* s_wrow = reinterpret_cast<double*>(smem + kOffWRow);  // importance weight (row, slot)
  float* s_q = reinterpret_cast<float*>(smem + kOffQ);          // p / kept mass (row, slot)
  uint32_t* s_info = reinterpret_cast<uint32_t*>(smem + kOffInfo);
  float* s_u = reinterpret_cast<float*>(smem + kOffU);
  uint8_t* s_m = reinterpret_cast<uint8_t*>(smem + kOffM);      // kept slots of each row
  int16_t* s_po = reinterpret_cast<int16_t*>(smem + kOffPOut);
  uint8_t* s_so = reinterpret_cast<uint8_t*>(smem + kOffSOut);
  const int b = blockIdx.x, lane = threadIdx.x;
  const float* P = a.probs + static_cast<long>(b) * a.rows * a.k;
  const float* U = a.u + static_cast<long>(b) * a.n_max;
  int32_t* parent = a.parent + static_cast<long>(b) * a.n_max;
  int32_t* slot = a.slot + static_cast<long>(b) * a.n_max;
  float* qd = a.q_draft + static_cast<long>(b) * a.n_max;

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
    for (int i = lane; i < a.n_max; i += 64) {  // no nodes: all padding
      parent[i] = -2;
      slot[i] = -2;
      qd[i] = 0.0f;
    }
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

  for (int j = lane; j < kCandCap; j += 64) s_w[j] = 0.0;  // whole chunks are read
  __syncthreads();

  int n_cand = 0;
  double cs = 0.0;  // lane c: sum of the weights of candidates kChunk c .. kChunk (c + 1) - 1
  // candidates of a context row appended in slot order: m kept slots, this lane's
  // weight w (0 past m), info for slot `lane`; each new weight joins its chunk's sum
  // in that order
  auto expand = [&](int m, double w, uint32_t info) __attribute__((always_inline)) {
    if (lane < m) {
      s_w[n_cand + lane] = w;
      s_info[n_cand + lane] = info;
    }
    // the new weights' sum per chunk (they span at most two: m <= 16 < kChunk), one
    // running sum per chunk over its lanes rather than one lane read per candidate;
    // each is a sum of that chunk's new weights alone, so it is 0 exactly when they
    // all are.  The new weights sit in lanes 0 .. m - 1 (m <= 16), one DPP row, so a
    // row scan is the whole scan there.
    const int c_lo = n_cand / kChunk, split = min(m, (c_lo + 1) * kChunk - n_cand);
    if (split > 0) {
      const double lo = readlane_f64(row_incl_scan(lane < split ? w : 0.0), split - 1);
      if (lane == c_lo) cs += lo;
    }
    if (split < m) {
      const double hi = readlane_f64(row_incl_scan(lane >= split ? w : 0.0), m - 1);
      if (lane == c_lo + 1) cs += hi;
    }
    n_cand += m;
    // one wavefront: its LDS accesses complete in issue order, so a later read sees
    // these writes; only the compiler must keep the order
    __builtin_amdgcn_wave_barrier();
  };

  {
    const int m0 = s_m[0];
    expand(m0, lane < m0 ? s_wrow[lane] : 0.0, pack_info(-1, lane, 1));
  }
  int n = 0;
  int m_next = 1 < a.rows ? s_m[1] : 0;  // kept count of row n + 1
  for (; n < a.n_max; ++n) {
    // the row a node drawn now would expand (row n + 1), read ahead of the draw (all
    // of its first k slots, masked by the kept count when the candidates are made)
    const bool has_row = n + 1 < a.rows;
    const double w_row = s_wrow[(has_row ? n + 1 : 0) * a.k + min(lane, a.k - 1)];
    const float u_n = s_u[n];
    const double incl = wave_incl_scan(cs);
    const double excl = dpp_shift(incl, 0x138, 0xf);  // wave_shr:1; lane 0 gets 0
    const double total = readlane_f64(incl, 63);
    const double t = static_cast<double>(u_n) * total;
    // the chunk: the first whose running sum passes t (lane 63's always does, as
    // u < 1); it holds weight, since adding a zero chunk leaves every partial sum
    const unsigned long long over = __ballot(incl > t);
    if (!(total > 0.0)) break;  // (tested after the ballot: one block with the reads above)
    const int owner = min(over ? __ffsll(static_cast<long long>(over)) - 1 : kChunks - 1, kChunks - 1);
    const double base = readlane_f64(excl, owner);
    // the chunk's candidates, two a lane (weights and info), and their running sums
    const double2 v = *reinterpret_cast<const double2*>(s_w + owner * kChunk + 2 * lane);
    const uint2 vi = *reinterpret_cast<const uint2*>(s_info + owner * kChunk + 2 * lane);
    // the next draw's kept count, read beside the chunk (no LDS wait of its own)
    const int m_after = n + 2 < a.rows ? s_m[n + 2] : 0;
    const double ps = v.x + v.y;
    const double pincl = wave_incl_scan(ps);
    const double pexcl = dpp_shift(pincl, 0x138, 0xf);
    const unsigned long long hit = __ballot(base + pincl > t);
    int jl, sel;
    if (hit) {
      jl = __ffsll(static_cast<long long>(hit)) - 1;
    } else {
      // rounding left the chunk's running sum short of t: its last candidate with weight
      const unsigned long long live = __ballot(v.x > 0.0 || v.y > 0.0);
      if (!live) break;  // unreachable: the chunk's sum is positive
      jl = 63 - __clzll(static_cast<long long>(live));
    }
    const double vx = readlane_f64(v.x, jl), vy = readlane_f64(v.y, jl);
    if (hit) {
      // its first candidate if it passes t on its own; a candidate without weight
      // is never taken (the scan's rounding cannot make an empty pair pass)
      const double pe = readlane_f64(pexcl, jl);
      sel = (vx > 0.0 && (vy == 0.0 || base + pe + vx > t)) ? 0 : 1;
    } else {
      sel = vy > 0.0 ? 1 : 0;
    }
    const int pick = owner * kChunk + 2 * jl + sel;
    // the chunk's sum without the taken candidate: its fresh sum minus the taken
    // weight.  Never negative (a sum of non-negative weights is at least each of
    // them) and 0 exactly when the taken one was its last (adding zeros is exact);
    // only remaining weights below the sum's rounding can be left out, until the
    // chunk gains a candidate.  (Read out in every lane: a read of lane 63 inside the
    // owner's branch would let the compiler finish the scan there, where lane 63 is
    // inactive.)
    const double rest = readlane_f64(pincl, 63) - (sel ? vy : vx);
    if (lane == owner) cs = rest;
    const uint32_t info = __builtin_amdgcn_readlane(sel ? vi.y : vi.x, jl);
    const double pw = sel ? vy : vx;
    const int ctx = static_cast<int>(info & 511) - 1, sl = (info >> 9) & 15;
    const int dep = static_cast<int>(info >> 13);
    if (lane == 0) {
      s_po[n] = static_cast<int16_t>(ctx);
      s_so[n] = static_cast<uint8_t>(sl);
      s_w[pick] = 0.0;
    }
    __builtin_amdgcn_wave_barrier();  // (one wavefront: see expand)
    if (dep < a.max_depth && has_row)
      expand(m_next, lane < m_next ? pw * w_row : 0.0, pack_info(n, lane, dep + 1));
    m_next = m_after;
  }
  __syncthreads();
  for (int i = lane; i < a.n_max; i += 64) {  // the nodes, then padding past the count
    const int c = i < n ? s_po[i] : -2, sl = i < n ? s_so[i] : -2;
    parent[i] = c;
    slot[i] = sl;
    // q_draft: renormalised by the kept mass of the node's context row
    qd[i] = i < n ? s_q[(c + 1) * a.k + sl] : 0.0f;
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
