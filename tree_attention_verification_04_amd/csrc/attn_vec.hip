// Vector-ALU tree attention: fp32 (or bf16) inputs, head_dim 64 or 128.
//
// This is the precise path (fp32 end to end, natural exp) used for fp32 inputs
// and for head sizes the matrix-core kernel does not take; it also serves as an
// independent cross-check of that kernel.  One wavefront per (node, query head)
// row.  Keys are taken 64 at a time, one key per lane for the scores and one key
// row per step, read by the whole wavefront, for P.V: first the prefix, one
// paged block per step, then each 64-node word of the row's ancestor bitset
// (page "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力机制与显存碎片整理联合加速"
// (ufo.work/2026/537), §2.2.2 mask M_tree, appendix B ancestor bitmap and online
// softmax with running max and sum).  Words with no visible node are skipped.
#include "attn.h"

namespace tv {

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, int i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int i) {
  return bf16_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void store_elem(T* p, long i, float v);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, long i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* p, long i, float v) {
  p[i] = f32_to_bf16(v);
}

// <q, row> with q in LDS; the lane reads its own key row.
template <typename T, int D>
__device__ __forceinline__ float dot_row(const T* __restrict__ row, const float* q) {
  float s = 0.0f;
  if constexpr (sizeof(T) == 4) {
    const float4* r4 = reinterpret_cast<const float4*>(row);
#pragma unroll 8
    for (int i = 0; i < D / 4; ++i) {
      const float4 v = r4[i];
      s = fmaf(q[4 * i + 0], v.x, s);
      s = fmaf(q[4 * i + 1], v.y, s);
      s = fmaf(q[4 * i + 2], v.z, s);
      s = fmaf(q[4 * i + 3], v.w, s);
    }
  } else {
    const uint4* r4 = reinterpret_cast<const uint4*>(row);
#pragma unroll 4
    for (int i = 0; i < D / 8; ++i) {
      const uint4 v = r4[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s = fmaf(q[8 * i + 2 * j], __uint_as_float(w[j] << 16), s);
        s = fmaf(q[8 * i + 2 * j + 1], __uint_as_float(w[j] & 0xffff0000u), s);
      }
    }
  }
  return s;
}

template <typename T, int D>
__global__ void __launch_bounds__(256) k_attn_vec(AttnArgs a) {
  constexpr int PER = D / 64;  // output elements per lane
  __shared__ float s_q[4][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  const bool live = row < a.total_rows;
  const int node = live ? row / a.hq : 0;
  const int head = live ? row % a.hq : 0;
  const T* q = static_cast<const T*>(a.q);
  if (live) {
#pragma unroll
    for (int j = 0; j < PER; ++j) s_q[wave][lane + 64 * j] = load_elem(q, static_cast<long>(row) * D + lane + 64 * j);
  }
  __syncthreads();
  if (!live) return;

  const int b = seq_of_node(a.cu_nodes, a.batch, node);
  const int n0 = a.cu_nodes[b];
  const int count = a.cu_nodes[b + 1] - n0;
  const int local = node - n0;
  const int g = head / a.group;
  int plen = a.prefix_len[b];
  if (plen > a.max_prefix || plen > a.max_blocks * 64 || plen < 0 || count > a.max_nodes) {
    if (lane == 0 && local == 0 && head == 0)
      atomicOr(a.err, count > a.max_nodes ? TV_ERR_TOO_MANY_NODES : TV_ERR_BLOCK);
    plen = max(0, min(plen, min(a.max_prefix, a.max_blocks * 64)));
  }
  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  const T* kt = static_cast<const T*>(a.k_tree);
  const T* vt = static_cast<const T*>(a.v_tree);
  const float* qs = s_q[wave];

  float m = -INFINITY, l = 0.0f;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.0f;

  const int nblk = (plen + 63) / 64;
  const int ntw = min((count + 63) / 64, a.words);
  const uint64_t* anc_row = a.anc + static_cast<long>(node) * a.words;
  for (int c = 0; c < nblk + ntw; ++c) {
    bool valid;
    const T* kbase = nullptr;  // key 0 of the tile; key k at kbase + k * stride
    const T* vbase = nullptr;
    long stride;
    int nrows;                 // rows of the tile that exist in memory
    if (c < nblk) {
      const int t = c * 64 + lane;
      int blk = a.block_table[static_cast<long>(b) * a.max_blocks + c];
      if (blk < 0 || blk >= a.num_blocks) {
        if (lane == 0) atomicOr(a.err, TV_ERR_BLOCK);
        continue;
      }
      valid = t < plen;
      const long base = (static_cast<long>(blk) * a.hkv + g) * 64 * D;
      kbase = kc + base;
      vbase = vc + base;
      stride = D;
      nrows = 64;  // a paged block always holds 64 rows
    } else {
      const int w = c - nblk;
      const uint64_t word = anc_row[w];
      if (word == 0) continue;
      valid = ((word >> lane) & 1ull) && w * 64 + lane < count;
      const long base = (static_cast<long>(n0 + w * 64) * a.hkv + g) * D;
      kbase = kt + base;
      vbase = vt + base;
      stride = static_cast<long>(a.hkv) * D;
      nrows = min(64, count - w * 64);
    }
    const float s =
        valid ? dot_row<T, D>(kbase + static_cast<long>(lane) * stride, qs) * a.scale : -INFINITY;
    const float m_new = fmaxf(m, wave_max(s));
    if (m_new == -INFINITY) continue;
    const float p = valid ? expf(s - m_new) : 0.0f;
    const float alpha = expf(m - m_new);
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] *= alpha;
    // P.V: lane owns output dims lane + 64 j; key k's row is read by the whole wave
    // (coalesced); every row's loads are issued before the first is used, rows past
    // the tile's end repeat its last row with probability 0
    float vv[64][PER];
#pragma unroll
    for (int k = 0; k < 64; ++k) {
      const T* vk = vbase + static_cast<long>(min(k, nrows - 1)) * stride;
#pragma unroll
      for (int j = 0; j < PER; ++j) vv[k][j] = load_elem(vk, lane + 64 * j);
    }
#pragma unroll
    for (int k = 0; k < 64; ++k) {
      const float pk = __shfl(p, k, 64);
#pragma unroll
      for (int j = 0; j < PER; ++j) acc[j] = fmaf(pk, vv[k][j], acc[j]);
    }
    m = m_new;
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  T* out = static_cast<T*>(a.out);
#pragma unroll
  for (int j = 0; j < PER; ++j) store_elem(out, static_cast<long>(row) * D + lane + 64 * j, acc[j] * inv);
  if (a.lse != nullptr && lane == 0) a.lse[row] = l > 0.0f ? m + logf(l) : -INFINITY;
}

int launch_attn_vec(const AttnArgs& a, int head_dim, int dtype, hipStream_t s) {
  const int grid = ceil_div(a.total_rows, 4);
  if (dtype == TV_DTYPE_F32 && head_dim == 64)
    hipLaunchKernelGGL((k_attn_vec<float, 64>), dim3(grid), dim3(256), 0, s, a);
  else if (dtype == TV_DTYPE_F32 && head_dim == 128)
    hipLaunchKernelGGL((k_attn_vec<float, 128>), dim3(grid), dim3(256), 0, s, a);
  else if (dtype == TV_DTYPE_BF16 && head_dim == 64)
    hipLaunchKernelGGL((k_attn_vec<uint16_t, 64>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn_vec<uint16_t, 128>), dim3(grid), dim3(256), 0, s, a);
  return check_launch("tree_verify_attention/vec");
}

}  // namespace tv
