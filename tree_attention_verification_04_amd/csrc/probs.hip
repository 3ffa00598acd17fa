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
// With many output rows (enough workgroups to fill the GPU) and a row that fits on
// one compute unit, one kernel (k_row_fused): a workgroup of 1024 threads reads a
// context row once into registers and LDS, reduces it to (max, sum of exp), keeps
// the exponentials, and writes the probability rows of the consecutive output rows
// of its group that share that context (siblings in level order).  Otherwise two
// kernels, both HBM-bound: k_row_stats takes the (max, sum of exp) of each
// 8192-element chunk of each context row; k_row_write merges the chunk statistics
// of a row and writes one chunk of probabilities for 8 consecutive output rows,
// loading a context chunk once for a run of siblings.  There, logits are read twice
// (once per pass); probabilities are written once either way.
//
// tree_softmax_rows_kept: the same rows restricted to a kept set of tokens per
// context row, zero elsewhere -- the distribution a pruned draft actually samples
// from, q~ = q * 1[x in R] / Z (page "端侧大模型推测解码草稿模型动态剪枝策略…" (ufo.work/
// 2026/525), §2.2.1; §2.2.2's edit of the logits, log(1/Z) on the kept tokens and
// minus infinity elsewhere, gives the same softmax because the constant cancels).
// One workgroup per output row (k_row_keep).
#include <algorithm>
#include <mutex>

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

// ---- one pass, the context row on chip
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr int kFusedLdsFloats = 40448;  // the part of a row past the registers (158 KB)
constexpr int kFusedMinRows = 256;      // output rows for at least one workgroup per CU
constexpr float kLog2E = 1.44269504088896340736f;

template <int kR>
constexpr int fused_min_vocab() { return kFusedThreads * kR; }
template <int kR>
constexpr int fused_max_vocab() { return kFusedThreads * kR + kFusedLdsFloats; }

// the workgroup's maximum / sum of one value per thread (every thread gets it);
// s_red holds one value per wavefront
__device__ __forceinline__ float fused_max(float v, float* s_red) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  __syncthreads();  // s_red free (its previous use has been read by every thread)
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = s_red[0];
#pragma unroll
  for (int w = 1; w < kFusedWaves; ++w) m = fmaxf(m, s_red[w]);
  return m;
}
__device__ __forceinline__ float fused_sum(float v, float* s_red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = s_red[0];
#pragma unroll
  for (int w = 1; w < kFusedWaves; ++w) s += s_red[w];
  return s;
}

// Workgroup g writes output rows g * group .. + group - 1.  Thread t holds the
// float4s at 4 (t + 1024 j), j < kR / 4, of the current context row in registers,
// and the row past 1024 kR in LDS (its own float4s at the same stride), first as
// c * logits with c = t log2(e), then as exp2(c * logits - max), which is
// exp(t * logits - max / log2(e)).  A bad context row index writes a zero
// row and sets its error bit.  The vocabulary is a multiple of 4 in
// [fused_min_vocab<kR>(), fused_max_vocab<kR>()] (the register part is always
// whole, so its accesses need no bounds); rows are 16-byte aligned.
template <int kR>
__global__ void __launch_bounds__(kFusedThreads) k_row_fused(RowArgs a) {
  extern __shared__ __attribute__((aligned(16))) float s_tail[];
  __shared__ float s_red[kFusedWaves];
  static_assert(kR % 4 == 0, "whole float4s in registers");
  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * a.group, i1 = min(a.rows, i0 + a.group);
  constexpr int reg_end = kFusedThreads * kR;
  float e[kR];
  float inv = 0.0f;
  int r_prev = -1;
  for (int i = i0; i < i1; ++i) {
    const int r = a.row_of != nullptr ? a.row_of[i] : i;
    float* out = a.probs + static_cast<long>(i) * a.vocab;
    if (r < 0 || r >= a.ctx_rows) {  // bad context row: zeros and the error bit
      if (tid == 0) atomicOr(a.err, TV_ERR_ROW);
      for (int k = 4 * tid; k < a.vocab; k += 4 * kFusedThreads)
        __builtin_nontemporal_store(f32x4_t{0.0f, 0.0f, 0.0f, 0.0f},
                                    reinterpret_cast<f32x4_t*>(out + k));
      continue;
    }
    if (r != r_prev) {
      const float* x = a.logits + static_cast<long>(r) * a.vocab;
      // (a thread reads and writes only its own float4s of the LDS part, so a new
      // row needs no barrier; s_red is guarded inside the reductions)
      // the register part, then the LDS part by direct loads (lane l of a wavefront
      // writes 16 bytes at the wavefront's base + 16 l, which is this thread's own
      // float4): every load of the row in flight at once
      const float4* xt = reinterpret_cast<const float4*>(x) + tid;
#pragma unroll
      for (int j = 0; j < kR / 4; ++j) {
        const float4 v = xt[kFusedThreads * j];
        e[4 * j] = v.x;
        e[4 * j + 1] = v.y;
        e[4 * j + 2] = v.z;
        e[4 * j + 3] = v.w;
      }
      const int wave_base = 4 * (tid & ~63);
      for (int k = reg_end + 4 * tid, j = 0; k < a.vocab; k += 4 * kFusedThreads, ++j)
        __builtin_amdgcn_global_load_lds(
            x + k,
            (__attribute__((address_space(3))) void*)(s_tail + wave_base + 4 * kFusedThreads * j),
            16, 0, 0);
      // in log2 units: c x with c = t log2(e) (t > 0, so -inf stays -inf), then
      // exp2 on the vector ALU; the argument's rounding is that of t x in expf(t x - m)
      const float c = a.t * kLog2E;
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < kR; ++q) {
        e[q] = c * e[q];
        m = fmaxf(m, e[q]);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the LDS part has landed
      for (int k = reg_end + 4 * tid; k < a.vocab; k += 4 * kFusedThreads) {
        float4 w = *reinterpret_cast<const float4*>(s_tail + (k - reg_end));
        w.x = c * w.x;
        w.y = c * w.y;
        w.z = c * w.z;
        w.w = c * w.w;
        m = fmaxf(fmaxf(m, fmaxf(w.x, w.y)), fmaxf(w.z, w.w));
        *reinterpret_cast<float4*>(s_tail + (k - reg_end)) = w;
      }
      m = fused_max(m, s_red);
      // four running sums per thread (one per float4 lane), then the workgroup's
      float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
      for (int j = 0; j < kR / 4; ++j) {
        e[4 * j] = __builtin_amdgcn_exp2f(e[4 * j] - m);
        e[4 * j + 1] = __builtin_amdgcn_exp2f(e[4 * j + 1] - m);
        e[4 * j + 2] = __builtin_amdgcn_exp2f(e[4 * j + 2] - m);
        e[4 * j + 3] = __builtin_amdgcn_exp2f(e[4 * j + 3] - m);
        s0 += e[4 * j];
        s1 += e[4 * j + 1];
        s2 += e[4 * j + 2];
        s3 += e[4 * j + 3];
      }
      for (int k = reg_end + 4 * tid; k < a.vocab; k += 4 * kFusedThreads) {
        float4 w = *reinterpret_cast<const float4*>(s_tail + (k - reg_end));
        w.x = __builtin_amdgcn_exp2f(w.x - m);
        w.y = __builtin_amdgcn_exp2f(w.y - m);
        w.z = __builtin_amdgcn_exp2f(w.z - m);
        w.w = __builtin_amdgcn_exp2f(w.w - m);
        s0 += w.x;
        s1 += w.y;
        s2 += w.z;
        s3 += w.w;
        *reinterpret_cast<float4*>(s_tail + (k - reg_end)) = w;
      }
      const float sum = fused_sum((s0 + s1) + (s2 + s3), s_red);
      inv = 1.0f / sum;
      r_prev = r;
    }
    // streaming stores: the rows are written once and not read here
    f32x4_t* ot = reinterpret_cast<f32x4_t*>(out) + tid;
#pragma unroll
    for (int j = 0; j < kR / 4; ++j) {
      const f32x4_t v = {e[4 * j] * inv, e[4 * j + 1] * inv, e[4 * j + 2] * inv,
                         e[4 * j + 3] * inv};
      __builtin_nontemporal_store(v, ot + kFusedThreads * j);
    }
    for (int k = reg_end + 4 * tid; k < a.vocab; k += 4 * kFusedThreads) {
      const float4 w = *reinterpret_cast<const float4*>(s_tail + (k - reg_end));
      const f32x4_t v = {w.x * inv, w.y * inv, w.z * inv, w.w * inv};
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(out + k));
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

// register floats per thread of the one-pass instances: 88 (vocabularies 90112 ..
// 130560) and 112 (114688 .. 155136); four wavefronts per SIMD
constexpr int kFusedR1 = 88;
constexpr int kFusedR2 = 112;

void set_fused_attributes() {
  static std::mutex mu;
  static uint32_t done = 0;  // one bit per device
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 32) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (done & (1u << dev)) return;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_row_fused<kFusedR1>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kFusedLdsFloats * 4);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_row_fused<kFusedR2>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kFusedLdsFloats * 4);
  done |= 1u << dev;
}

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
  const bool fit1 = vocab >= tv::fused_min_vocab<tv::kFusedR1>() &&
                    vocab <= tv::fused_max_vocab<tv::kFusedR1>();
  const bool fit2 = vocab >= tv::fused_min_vocab<tv::kFusedR2>() &&
                    vocab <= tv::fused_max_vocab<tv::kFusedR2>();
  if (vec && rows >= tv::kFusedMinRows && (fit1 || fit2)) {
    // one pass: groups of consecutive output rows, at least one workgroup per CU
    tv::set_fused_attributes();
    a.group = std::max(1, std::min(tv::kRowGroup, rows / tv::kFusedMinRows));
    const int groups = tv::ceil_div(rows, a.group);
    const bool small = fit1;
    const int reg = (small ? tv::kFusedR1 : tv::kFusedR2) * tv::kFusedThreads;
    const size_t lds = static_cast<size_t>(vocab - reg) * sizeof(float);
    if (small)
      hipLaunchKernelGGL(tv::k_row_fused<tv::kFusedR1>, dim3(groups), dim3(tv::kFusedThreads), lds,
                         s, a);
    else
      hipLaunchKernelGGL(tv::k_row_fused<tv::kFusedR2>, dim3(groups), dim3(tv::kFusedThreads), lds,
                         s, a);
    return tv::check_launch("tree_softmax_rows/fused");
  }
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
