// tree_softmax_rows: probability rows from target logits, before acceptance.
//
// One forward pass of the target model over the tree gives one logits row per
// context (page "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力机制与显存碎片
// 整理联合加速" (ufo.work/2026/537), §2.2.3); a drafted token is judged by the
// distribution at its parent's context, so siblings share a row: output row i is
// softmax(t * logits[row_of[i]]).  The row maximum is subtracted before exp (page
// "端侧大模型推测解码草稿模型动态剪枝策略：详解基于重要性采样的树形验证并行加速机制"
// (ufo.work/2026/525), §7.1, log-sum-exp trick).
//
// Two kernels, both HBM-bound: k_row_stats takes the (max, sum of exp) of each
// 8192-element chunk of each context row; k_row_write merges the chunk statistics
// of a row and writes one chunk of probabilities for 8 consecutive output rows,
// loading a context chunk once for a run of siblings.  Logits are read twice
// (once per pass), probabilities written once.
//
// tree_softmax_rows_kept: the same rows restricted to a kept set of tokens per
// context row, zero elsewhere -- the distribution a pruned draft actually samples
// from, q~ = q * 1[x in R] / Z (page "端侧大模型推测解码草稿模型动态剪枝策略…" (ufo.work/
// 2026/525), §2.2.1; §2.2.2's edit of the logits, log(1/Z) on the kept tokens and
// minus infinity elsewhere, gives the same softmax because the constant cancels).
// One workgroup per output row (k_row_keep).
#include <algorithm>

#include "tv_common.h"

namespace tv {

namespace {

constexpr int kRowThreads = 256;
constexpr int kRowChunk = 8192;                      // elements per workgroup
constexpr int kPerThread = kRowChunk / kRowThreads;  // 32
constexpr int kRowGroup = 8;                         // most output rows per write workgroup
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct RowArgs {
  const float* logits;
  const int32_t* row_of;
  float* probs;
  float2* stats;  // [ctx_rows, chunks]: (max, sum of exp(x - max)) of t * logits
  int32_t* err;
  int ctx_rows, rows, vocab, chunks, group;  // group: output rows per write workgroup
  float t;
};

__device__ __forceinline__ void merge_stat(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * expf(m - mn) + s2 * expf(m2 - mn);
  m = mn;
}

// workgroup reduction of (max, sum) pairs; result valid in every thread
__device__ __forceinline__ void block_stat(float& m, float& s, float2* s_red) {
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64), s2 = __shfl_xor(s, off, 64);
    merge_stat(m, s, m2, s2);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) s_red[wave] = make_float2(m, s);
  __syncthreads();
  m = -INFINITY;
  s = 0.0f;
  for (int w = 0; w < kRowThreads / 64; ++w) merge_stat(m, s, s_red[w].x, s_red[w].y);
}

template <bool kVec>
__global__ void __launch_bounds__(kRowThreads) k_row_stats(RowArgs a) {
  __shared__ float2 s_red[kRowThreads / 64];
  const int c = blockIdx.x, r = blockIdx.y;
  const long row = static_cast<long>(r) * a.vocab;
  const int k0 = c * kRowChunk, k1 = min(a.vocab, k0 + kRowChunk);
  float x[kPerThread];
  if (kVec) {
#pragma unroll
    for (int j = 0; j < kPerThread / 4; ++j) {
      const int k = k0 + 4 * (threadIdx.x + kRowThreads * j);
      float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (k < k1) v = *reinterpret_cast<const float4*>(a.logits + row + k);  // k1 - k >= 4
      x[4 * j] = v.x;
      x[4 * j + 1] = v.y;
      x[4 * j + 2] = v.z;
      x[4 * j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int k = k0 + threadIdx.x + kRowThreads * j;
      x[j] = k < k1 ? a.logits[row + k] : -INFINITY;
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    x[j] = x[j] == -INFINITY ? -INFINITY : a.t * x[j];
    m = fmaxf(m, x[j]);
  }
  float s = 0.0f;
  if (m != -INFINITY) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) s += expf(x[j] - m);
  }
  block_stat(m, s, s_red);
  if (threadIdx.x == 0) a.stats[static_cast<long>(r) * a.chunks + c] = make_float2(m, s);
}

// One workgroup writes one chunk of `group` consecutive output rows; consecutive
// rows with the same context row (siblings, in level order) reuse the exponentials
// already computed, so a shared logits chunk is read once per group.  Groups are
// used only when there are enough workgroups to fill the GPU anyway.
template <bool kVec>
__global__ void __launch_bounds__(kRowThreads) k_row_write(RowArgs a) {
  const int c = blockIdx.x;
  const int i0 = blockIdx.y * a.group, i1 = min(a.rows, i0 + a.group);
  const int k0 = c * kRowChunk, k1 = min(a.vocab, k0 + kRowChunk);
  float p[kPerThread];
  int r_prev = -1;
  for (int i = i0; i < i1; ++i) {
    const int r = a.row_of != nullptr ? a.row_of[i] : i;
    const long out = static_cast<long>(i) * a.vocab;
    if (r < 0 || r >= a.ctx_rows) {  // bad context row: zeros and the error bit
      if (c == 0 && threadIdx.x == 0) atomicOr(a.err, TV_ERR_ROW);
      for (int k = k0 + threadIdx.x; k < k1; k += kRowThreads) a.probs[out + k] = 0.0f;
      continue;
    }
    if (r != r_prev) {
      float m = -INFINITY, s = 0.0f;
      for (int cc = 0; cc < a.chunks; ++cc) {
        const float2 st = a.stats[static_cast<long>(r) * a.chunks + cc];
        merge_stat(m, s, st.x, st.y);
      }
      const float inv = 1.0f / s;
      const long row = static_cast<long>(r) * a.vocab;
      if (kVec) {
#pragma unroll
        for (int j = 0; j < kPerThread / 4; ++j) {
          const int k = k0 + 4 * (threadIdx.x + kRowThreads * j);
          float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          if (k < k1) v = *reinterpret_cast<const float4*>(a.logits + row + k);
          p[4 * j] = expf(a.t * v.x - m) * inv;
          p[4 * j + 1] = expf(a.t * v.y - m) * inv;
          p[4 * j + 2] = expf(a.t * v.z - m) * inv;
          p[4 * j + 3] = expf(a.t * v.w - m) * inv;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
          const int k = k0 + threadIdx.x + kRowThreads * j;
          p[j] = k < k1 ? expf(a.t * a.logits[row + k] - m) * inv : 0.0f;
        }
      }
      r_prev = r;
    }
    if (kVec) {
#pragma unroll
      for (int j = 0; j < kPerThread / 4; ++j) {
        const int k = k0 + 4 * (threadIdx.x + kRowThreads * j);
        if (k < k1) {  // streaming store: the rows are written once and not read here
          const f32x4_t v = {p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]};
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(a.probs + out + k));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const int k = k0 + threadIdx.x + kRowThreads * j;
        if (k < k1) a.probs[out + k] = p[j];
      }
    }
  }
}

constexpr int kKeepMax = kRowThreads;  // kept ids per context row: one per thread

struct KeptArgs {
  const float* logits;
  const int32_t* keep;    // [ctx_rows, keep_max], -1 = padding
  const int32_t* row_of;
  float* probs;
  int32_t* err;
  int ctx_rows, rows, vocab, keep_max;
  float t;
};

// Output row i: the kept ids of its context row r go to LDS; an id that repeats an
// earlier entry, or is padding, drops out; the kept logits are gathered and reduced
// to (max, sum of exp); the row is zero-filled by streaming stores and, once those
// have completed (so no zero lands after a probability), the kept probabilities are
// written.  A bad context row index, an id outside [-1, vocab) or an empty set
// leaves the row zero and sets its error bit.
template <bool kVec>
__global__ void __launch_bounds__(kRowThreads) k_row_keep(KeptArgs a) {
  __shared__ int s_ids[kKeepMax];
  __shared__ float2 s_red[kRowThreads / 64];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const long i = blockIdx.x;
  const int r = a.row_of != nullptr ? a.row_of[i] : static_cast<int>(i);
  const bool row_ok = r >= 0 && r < a.ctx_rows;
  if (tid == 0) s_bad = row_ok ? 0 : TV_ERR_ROW;
  __syncthreads();
  int id = -1;
  if (row_ok && tid < a.keep_max) {
    id = a.keep[static_cast<long>(r) * a.keep_max + tid];
    if (id < -1 || id >= a.vocab) atomicOr(&s_bad, TV_ERR_TOKEN);
    s_ids[tid] = id;
  }
  __syncthreads();
  const int bad_in = s_bad;
  if (bad_in != 0) id = -1;
  if (id >= 0)
    for (int j = 0; j < tid; ++j)
      if (s_ids[j] == id) {
        id = -1;
        break;
      }
  const float x = id >= 0 ? a.t * a.logits[static_cast<long>(r) * a.vocab + id] : -INFINITY;
  float m = x, sum = id >= 0 ? 1.0f : 0.0f;
  block_stat(m, sum, s_red);
  float* out = a.probs + i * a.vocab;
  if (kVec) {
    for (int k = 4 * tid; k < a.vocab; k += 4 * kRowThreads)
      __builtin_nontemporal_store(f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, reinterpret_cast<f32x4_t*>(out + k));
  } else {
    for (int k = tid; k < a.vocab; k += kRowThreads) __builtin_nontemporal_store(0.0f, out + k);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's zeros have landed
  __syncthreads();
  const int bad = bad_in | (bad_in == 0 && m == -INFINITY ? TV_ERR_ZERO_MASS : 0);
  if (bad == 0 && id >= 0) out[id] = expf(x - m) / sum;
  if (tid == 0 && bad != 0) atomicOr(a.err, bad);
}

}  // namespace

}  // namespace tv

extern "C" size_t tree_softmax_rows_workspace_size(int32_t ctx_rows, int32_t vocab) {
  if (ctx_rows <= 0 || vocab <= 0) return 0;
  return static_cast<size_t>(ctx_rows) * tv::ceil_div(vocab, tv::kRowChunk) * sizeof(float2);
}

extern "C" int tree_softmax_rows(const float* logits, int32_t ctx_rows, int32_t vocab,
                                 const int32_t* row_of, int32_t rows, float inv_temperature,
                                 float* probs, void* workspace, size_t workspace_bytes,
                                 int32_t* err, void* stream) {
  tv::clear_error();
  if (ctx_rows < 0 || rows < 0 || vocab < 0)
    return tv::fail(TV_EINVAL, "tree_softmax_rows: negative size");
  if (!(inv_temperature > 0.0f) || inv_temperature == INFINITY)
    return tv::fail(TV_EINVAL, "tree_softmax_rows: inverse temperature must be positive and finite");
  if (row_of == nullptr && rows != ctx_rows)
    return tv::fail(TV_EINVAL, "tree_softmax_rows: without row_of, rows must equal ctx_rows");
  if (err == nullptr) return tv::fail(TV_EINVAL, "tree_softmax_rows: null err");
  if (rows == 0 || vocab == 0) return TV_OK;
  if (ctx_rows == 0) return tv::fail(TV_EINVAL, "tree_softmax_rows: rows without context rows");
  if (logits == nullptr || probs == nullptr)
    return tv::fail(TV_EINVAL, "tree_softmax_rows: null logits or probs");
  if (static_cast<long>(ctx_rows) * vocab > (1L << 40))
    return tv::fail(TV_EUNSUPPORTED, "tree_softmax_rows: logits too large");
  const size_t need = tree_softmax_rows_workspace_size(ctx_rows, vocab);
  if (workspace == nullptr || workspace_bytes < need)
    return tv::fail(TV_EWORKSPACE, "tree_softmax_rows: workspace missing or too small");
  const int chunks = tv::ceil_div(vocab, tv::kRowChunk);
  if (chunks > 65535 || ctx_rows > 65535 || rows > 65535)
    return tv::fail(TV_EUNSUPPORTED, "tree_softmax_rows: more than 65535 rows or chunks");
  tv::RowArgs a{};
  a.logits = logits;
  a.row_of = row_of;
  a.probs = probs;
  a.stats = static_cast<float2*>(workspace);
  a.err = err;
  a.ctx_rows = ctx_rows;
  a.rows = rows;
  a.vocab = vocab;
  a.chunks = chunks;
  a.t = inv_temperature;
  auto s = static_cast<hipStream_t>(stream);
  // float4 rows need every row to start 16-byte aligned
  const bool vec = vocab % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(probs) % 16) == 0;
  if (vec)
    hipLaunchKernelGGL(tv::k_row_stats<true>, dim3(chunks, ctx_rows), dim3(tv::kRowThreads), 0, s, a);
  else
    hipLaunchKernelGGL(tv::k_row_stats<false>, dim3(chunks, ctx_rows), dim3(tv::kRowThreads), 0, s, a);
  int st = tv::check_launch("tree_softmax_rows/stats");
  if (st != TV_OK) return st;
  // rows per write workgroup: 1 while there are few workgroups, up to 8 with many
  a.group = std::max(1, std::min(tv::kRowGroup, static_cast<int>(static_cast<long>(rows) * chunks / 2048)));
  const int groups = tv::ceil_div(rows, a.group);
  if (vec)
    hipLaunchKernelGGL(tv::k_row_write<true>, dim3(chunks, groups), dim3(tv::kRowThreads), 0, s, a);
  else
    hipLaunchKernelGGL(tv::k_row_write<false>, dim3(chunks, groups), dim3(tv::kRowThreads), 0, s, a);
  return tv::check_launch("tree_softmax_rows/write");
}

extern "C" int tree_softmax_rows_kept(const float* logits, int32_t ctx_rows, int32_t vocab,
                                      const int32_t* keep, int32_t keep_max, const int32_t* row_of,
                                      int32_t rows, float inv_temperature, float* probs,
                                      int32_t* err, void* stream) {
  tv::clear_error();
  if (ctx_rows < 0 || rows < 0 || vocab < 0)
    return tv::fail(TV_EINVAL, "tree_softmax_rows_kept: negative size");
  if (keep_max < 1 || keep_max > tv::kKeepMax)
    return tv::fail(TV_EUNSUPPORTED, "tree_softmax_rows_kept: keep_max must be in [1, 256]");
  if (!(inv_temperature > 0.0f) || inv_temperature == INFINITY)
    return tv::fail(TV_EINVAL,
                    "tree_softmax_rows_kept: inverse temperature must be positive and finite");
  if (row_of == nullptr && rows != ctx_rows)
    return tv::fail(TV_EINVAL, "tree_softmax_rows_kept: without row_of, rows must equal ctx_rows");
  if (err == nullptr) return tv::fail(TV_EINVAL, "tree_softmax_rows_kept: null err");
  if (rows == 0 || vocab == 0) return TV_OK;
  if (ctx_rows == 0) return tv::fail(TV_EINVAL, "tree_softmax_rows_kept: rows without context rows");
  if (logits == nullptr || probs == nullptr || keep == nullptr)
    return tv::fail(TV_EINVAL, "tree_softmax_rows_kept: null logits, keep or probs");
  if (static_cast<long>(ctx_rows) * vocab > (1L << 40) || static_cast<long>(rows) * vocab > (1L << 40))
    return tv::fail(TV_EUNSUPPORTED, "tree_softmax_rows_kept: rows too large");
  tv::KeptArgs a{};
  a.logits = logits;
  a.keep = keep;
  a.row_of = row_of;
  a.probs = probs;
  a.err = err;
  a.ctx_rows = ctx_rows;
  a.rows = rows;
  a.vocab = vocab;
  a.keep_max = keep_max;
  a.t = inv_temperature;
  auto s = static_cast<hipStream_t>(stream);
  const bool vec = vocab % 4 == 0 && (reinterpret_cast<uintptr_t>(probs) % 16) == 0;
  if (vec)
    hipLaunchKernelGGL(tv::k_row_keep<true>, dim3(rows), dim3(tv::kRowThreads), 0, s, a);
  else
    hipLaunchKernelGGL(tv::k_row_keep<false>, dim3(rows), dim3(tv::kRowThreads), 0, s, a);
  return tv::check_launch("tree_softmax_rows_kept");
}
