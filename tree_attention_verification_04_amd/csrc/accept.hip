// tree_accept: fused acceptance of a verified draft tree, no host round-trip.
//
// What is computed follows page "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力
// 机制与显存碎片整理联合加速" (ufo.work/2026/537), §2.2.3: each node's acceptance
// probability min(1, p_target / p_draft) at its drafted token, one uniform per node,
// a depth-first walk from the root that stops below the first rejected node, and the
// longest accepted path, all inside GPU kernels.  At the rejection point a token is
// resampled (page "端侧大模型推测解码草稿模型动态剪枝策略：详解基于重要性采样的树形验证并行加速
// 机制" (ufo.work/2026/525), §1.2) from norm(max(0, p_target - p_draft)), falling back
// to p_target itself when that has no mass (same page, §7.2).
//
// Up to 65536 vocabulary entries one kernel does everything (the walk's workgroup
// scans the rejection row); for larger vocabularies three kernels on the stream:
//   k_accept_walk    one workgroup per sequence: ratio tests, ancestor walks, the
//                    deepest accepted node (ties: smallest index), the path, and the
//                    rejection node c (smallest-index child of the winner).
//   k_resid_partial  (vocab chunk, sequence) workgroups: integer residual weights
//                    of row c summed per chunk.
//   k_resid_select   one workgroup per sequence: total mass, exact threshold, the
//                    chunk and then the element where the running sum passes it.
// The weights are integers (floor of the fp64 difference times 2^40), so every sum
// is exact and the token does not depend on how the vocabulary is split.
#include <limits.h>

#include "tv_common.h"

namespace tv {

constexpr int kAcceptThreads = 256;
constexpr int kResidChunk = 4096;                       // vocabulary entries per chunk
constexpr int kResidPerThread = kResidChunk / kAcceptThreads;
constexpr int kFusedVocab = 65536;  // up to this vocabulary the walk's workgroup resamples
constexpr int kMaxVocab = 1 << 18;
constexpr int kMaxResidChunks = kMaxVocab / kResidChunk;
static_assert(kResidPerThread % 4 == 0, "whole float4 per thread");

#pragma clang fp contract(off)

// Fixed-point residual weight of one vocabulary entry.
__device__ __forceinline__ uint64_t resid_weight(float pt, float pd) {
  const double r = static_cast<double>(pt) - static_cast<double>(pd);
  return r > 0.0 ? static_cast<uint64_t>(r * 1099511627776.0) : 0ull;  // 2^40
}

__device__ __forceinline__ uint64_t target_weight(float pt) {
  const double r = static_cast<double>(pt);
  return r > 0.0 ? static_cast<uint64_t>(r * 1099511627776.0) : 0ull;
}

// floor(u * z) for u in [0, 1), taken exactly: u = M * 2^E with an integer M.
__device__ __forceinline__ uint64_t exact_threshold(float u, uint64_t z) {
  const uint32_t bits = __float_as_uint(u);
  const uint32_t e = (bits >> 23) & 0xffu;
  const uint64_t m = e ? ((bits & 0x7fffffu) | 0x800000u) : (bits & 0x7fffffu);
  const int shift = e ? static_cast<int>(150 - e) : 149;  // u = m * 2^-shift
  const uint64_t lo = m * z;
  const uint64_t hi = __umul64hi(m, z);
  if (shift >= 128) return 0;
  if (shift >= 64) return hi >> (shift - 64);
  return (lo >> shift) | (hi << (64 - shift));
}

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int d) {
  const uint32_t lo = __shfl_up(static_cast<uint32_t>(v), d, 64);
  const uint32_t hi = __shfl_up(static_cast<uint32_t>(v >> 32), d, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int d) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), d, 64);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), d, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Exclusive prefix sum over the 256 threads of a workgroup; returns the
// thread's exclusive sum, and the block total in *total.
__device__ uint64_t block_exclusive_scan(uint64_t v, uint64_t* total) {
  __shared__ uint64_t wave_tot[kAcceptThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t o = shfl_up_u64(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  uint64_t before = 0, all = 0;
  for (int w = 0; w < kAcceptThreads / 64; ++w) {
    if (w < wave) before += wave_tot[w];
    all += wave_tot[w];
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

__device__ uint64_t block_sum_u64(uint64_t v) {
  __shared__ uint64_t wave_tot[kAcceptThreads / 64];
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v += shfl_xor_u64(v, d);
  if ((threadIdx.x & 63) == 0) wave_tot[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t all = 0;
  for (int w = 0; w < kAcceptThreads / 64; ++w) all += wave_tot[w];
  __syncthreads();
  return all;
}

// Residual resample of row c inside one workgroup (small vocabularies): thread t
// sums the integer weights of its contiguous slice, a block scan over the slices
// finds the one where the running sum passes the threshold, and that thread walks
// its slice again.  Same integers as the multi-workgroup path, so the same token.
__device__ void resample_in_block(const float* __restrict__ pt_row, const float* __restrict__ pd_row,
                                  int vocab, float u, int32_t* __restrict__ out_token,
                                  int32_t* __restrict__ err) {
  const int tid = threadIdx.x;
  const int len = ((vocab + kAcceptThreads - 1) / kAcceptThreads + 3) & ~3;
  const int k0 = min(vocab, tid * len), k1 = min(vocab, k0 + len);
  uint64_t sr = 0, st = 0;
  for (int k = k0; k < k1; ++k) {
    const float t = pt_row[k];
    sr += resid_weight(t, pd_row[k]);
    st += target_weight(t);
  }
  const uint64_t zr = block_sum_u64(sr);
  const uint64_t zt = block_sum_u64(st);
  const int mode = zr > 0 ? 0 : (zt > 0 ? 1 : -1);
  if (mode < 0) {
    if (tid == 0) {
      *out_token = -1;
      atomicOr(err, TV_ERR_ZERO_MASS);
    }
    return;
  }
  const uint64_t t_thr = exact_threshold(u, mode == 0 ? zr : zt);
  const uint64_t local = mode == 0 ? sr : st;
  uint64_t total;
  const uint64_t excl = block_exclusive_scan(local, &total);
  if (local > 0 && excl <= t_thr && t_thr < excl + local) {
    uint64_t run = excl;
    for (int k = k0; k < k1; ++k) {
      run += mode == 0 ? resid_weight(pt_row[k], pd_row[k]) : target_weight(pt_row[k]);
      if (run > t_thr) {
        *out_token = k;
        break;
      }
    }
  }
}

template <bool kFused>
__global__ void __launch_bounds__(kAcceptThreads) k_accept_walk(
    const float* __restrict__ pt, const float* __restrict__ pd, const int32_t* __restrict__ token,
    const float* __restrict__ u_acc, const float* __restrict__ u_res,
    const int32_t* __restrict__ parent, const int32_t* __restrict__ cu_nodes, int max_nodes,
    int vocab, int max_path, int32_t* __restrict__ accept_len, int32_t* __restrict__ path,
    int32_t* __restrict__ resample_node, int32_t* __restrict__ resample_token,
    uint8_t* __restrict__ node_ok, int32_t* __restrict__ ws_c, int32_t* __restrict__ err) {
  __shared__ int16_t s_par[TV_MAX_NODES];
  __shared__ uint8_t s_acc[TV_MAX_NODES];
  __shared__ int s_bad, s_key, s_child, s_err, s_pending;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int n0 = cu_nodes[b];
  const int n = cu_nodes[b + 1] - n0;
  if (tid == 0) {
    s_bad = 0;
    s_key = -1;
    s_child = INT_MAX;
    s_err = 0;
  }
  for (int j = tid; j < max_path; j += kAcceptThreads) path[static_cast<long>(b) * max_path + j] = -1;
  __syncthreads();
  if (n > max_nodes) {
    if (node_ok != nullptr)
      for (int i = tid; i < n; i += kAcceptThreads) node_ok[n0 + i] = 0;
    if (tid == 0) {
      atomicOr(err, TV_ERR_TOO_MANY_NODES);
      accept_len[b] = 0;
      resample_node[b] = -1;
      resample_token[b] = -1;
      ws_c[b] = -1;
    }
    return;
  }
  for (int i = tid; i < n; i += kAcceptThreads) {
    const int p = parent[n0 + i];
    s_par[i] = static_cast<int16_t>(p);
    if (p >= i || p < -1) s_bad = 1;
  }
  __syncthreads();
  if (s_bad) {
    if (node_ok != nullptr)
      for (int i = tid; i < n; i += kAcceptThreads) node_ok[n0 + i] = 0;
    if (tid == 0) {
      atomicOr(err, TV_ERR_BAD_PARENT);
      accept_len[b] = 0;
      resample_node[b] = -1;
      resample_token[b] = -1;
      ws_c[b] = -1;
    }
    return;
  }
  // 1-2. ratio test per node: u < min(1, pt/pd)  <=>  (double)u * pd < pt for u in [0, 1)
  int my_err = 0;
  for (int i = tid; i < n; i += kAcceptThreads) {
    const long g = n0 + i;
    const int tok = token[g];
    bool a = false;
    if (tok < 0 || tok >= vocab) {
      my_err |= TV_ERR_TOKEN;
    } else {
      const float u = u_acc[g];
      if (!(u >= 0.0f && u < 1.0f)) {
        my_err |= TV_ERR_UNIFORM;
      } else {
        const long off = g * vocab + tok;
        a = static_cast<double>(u) * static_cast<double>(pd[off]) < static_cast<double>(pt[off]);
      }
    }
    s_acc[i] = a ? 1 : 0;
  }
  if (my_err) atomicOr(&s_err, my_err);
  __syncthreads();
  // 3. a node is reached by the walk iff it and all its ancestors passed;
  //    the winner is the reached node of largest depth, smallest index on ties
  for (int i = tid; i < n; i += kAcceptThreads) {
    int v = i, depth = 0;
    bool ok = true;
    while (v >= 0) {
      if (!s_acc[v]) {
        ok = false;
        break;
      }
      ++depth;
      v = s_par[v];
    }
    if (node_ok != nullptr) node_ok[n0 + i] = ok ? 1 : 0;
    if (ok) atomicMax(&s_key, (depth << 12) | (4095 - i));
  }
  __syncthreads();
  const int key = s_key;
  const int w = key < 0 ? -1 : 4095 - (key & 4095);
  const int depth_w = key < 0 ? 0 : (key >> 12);
  // rejection point: smallest-index child of the winner (w = -1: of the prefix)
  for (int i = tid; i < n; i += kAcceptThreads)
    if (s_par[i] == w) atomicMin(&s_child, i);
  __syncthreads();
  if (tid == 0) {
    int e = s_err;
    accept_len[b] = depth_w;
    int v = w;
    for (int k = depth_w - 1; k >= 0; --k) {
      if (k < max_path) path[static_cast<long>(b) * max_path + k] = v;
      v = s_par[v];
    }
    if (depth_w > max_path) e |= TV_ERR_PATH;
    const int c = s_child == INT_MAX ? -1 : s_child;
    resample_node[b] = c;
    int pending = -1;
    if (c >= 0) {
      const float u = u_res[n0 + c];
      if (u >= 0.0f && u < 1.0f) pending = c;
      else e |= TV_ERR_UNIFORM;
    }
    ws_c[b] = pending;
    s_pending = pending;
    if (pending < 0) resample_token[b] = -1;
    if (e) atomicOr(err, e);
  }
  if constexpr (kFused) {
    __syncthreads();
    const int c = s_pending;
    if (c < 0) return;
    const long row = static_cast<long>(n0 + c) * vocab;
    resample_in_block(pt + row, pd + row, vocab, u_res[n0 + c], resample_token + b, err);
  }
}

__global__ void __launch_bounds__(kAcceptThreads) k_resid_partial(
    const float* __restrict__ pt, const float* __restrict__ pd, const int32_t* __restrict__ cu_nodes,
    int vocab, int chunks, const int32_t* __restrict__ ws_c, uint64_t* __restrict__ part) {
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int c = ws_c[b];
  if (c < 0) return;
  const long row = static_cast<long>(cu_nodes[b] + c) * vocab;
  const int k0 = chunk * kResidChunk;
  const int k1 = min(vocab, k0 + kResidChunk);
  uint64_t sr = 0, st = 0;
  const bool aligned =
      ((vocab & 3) | ((reinterpret_cast<uintptr_t>(pt) | reinterpret_cast<uintptr_t>(pd)) & 15)) == 0;
  if (aligned && k1 - k0 == kResidChunk) {
    // whole chunk, rows 16-byte aligned: each thread takes 4 float4 of each row,
    // all 8 loads in flight at once
    const float4* t4 = reinterpret_cast<const float4*>(pt + row + k0);
    const float4* d4 = reinterpret_cast<const float4*>(pd + row + k0);
    float4 tv[kResidPerThread / 4], dv[kResidPerThread / 4];
#pragma unroll
    for (int j = 0; j < kResidPerThread / 4; ++j) {
      tv[j] = t4[threadIdx.x + j * kAcceptThreads];
      dv[j] = d4[threadIdx.x + j * kAcceptThreads];
    }
#pragma unroll
    for (int j = 0; j < kResidPerThread / 4; ++j) {
      sr += resid_weight(tv[j].x, dv[j].x) + resid_weight(tv[j].y, dv[j].y) +
            resid_weight(tv[j].z, dv[j].z) + resid_weight(tv[j].w, dv[j].w);
      st += target_weight(tv[j].x) + target_weight(tv[j].y) + target_weight(tv[j].z) +
            target_weight(tv[j].w);
    }
  } else {
    for (int k = k0 + threadIdx.x; k < k1; k += kAcceptThreads) {
      const float t = pt[row + k];
      sr += resid_weight(t, pd[row + k]);
      st += target_weight(t);
    }
  }
  sr = block_sum_u64(sr);
  st = block_sum_u64(st);
  if (threadIdx.x == 0) {
    part[(static_cast<long>(b) * chunks + chunk) * 2 + 0] = sr;
    part[(static_cast<long>(b) * chunks + chunk) * 2 + 1] = st;
  }
}

__global__ void __launch_bounds__(kAcceptThreads) k_resid_select(
    const float* __restrict__ pt, const float* __restrict__ pd, const float* __restrict__ u_res,
    const int32_t* __restrict__ cu_nodes, int vocab, int chunks, const int32_t* __restrict__ ws_c,
    const uint64_t* __restrict__ part, int32_t* __restrict__ resample_token,
    int32_t* __restrict__ err) {
  __shared__ int s_mode, s_chunk;
  __shared__ uint64_t s_rem;
  __shared__ uint64_t s_part[2 * kMaxResidChunks];
  const int b = blockIdx.x, tid = threadIdx.x;
  // the rejection node, the sequence's first node and the per-chunk sums (which do
  // not depend on the node) are requested together; then the node's uniform
  const uint64_t* mine = part + static_cast<long>(b) * chunks * 2;
  const int c = ws_c[b];
  const int n0 = cu_nodes[b];
  uint64_t pv[2 * kMaxResidChunks / kAcceptThreads + 1];
  int np = 0;
  for (int k = tid; k < 2 * chunks; k += kAcceptThreads) pv[np++] = mine[k];
  if (c < 0) return;
  const float u = u_res[n0 + c];
  np = 0;
  for (int k = tid; k < 2 * chunks; k += kAcceptThreads) s_part[k] = pv[np++];
  __syncthreads();
  if (tid == 0) {
    uint64_t zr = 0, zt = 0;
    for (int k = 0; k < chunks; ++k) {
      zr += s_part[2 * k];
      zt += s_part[2 * k + 1];
    }
    const int mode = zr > 0 ? 0 : (zt > 0 ? 1 : -1);
    s_mode = mode;
    if (mode >= 0) {
      const uint64_t t = exact_threshold(u, mode == 0 ? zr : zt);
      uint64_t cum = 0;
      int kc = chunks - 1;
      for (int k = 0; k < chunks; ++k) {
        const uint64_t s = s_part[2 * k + mode];
        if (t < cum + s) {
          kc = k;
          break;
        }
        cum += s;
      }
      s_chunk = kc;
      s_rem = t - cum;
    } else {
      resample_token[b] = -1;
      atomicOr(err, TV_ERR_ZERO_MASS);
    }
  }
  __syncthreads();
  const int mode = s_mode;
  if (mode < 0) return;
  const long row = static_cast<long>(n0 + c) * vocab;
  const int k0 = s_chunk * kResidChunk + tid * kResidPerThread;
  const int k1 = min(vocab, min(k0 + kResidPerThread, (s_chunk + 1) * kResidChunk));
  // this thread's weights, loaded once (all loads in flight together) and kept for
  // the walk
  uint64_t wgt[kResidPerThread];
#pragma unroll
  for (int e = 0; e < kResidPerThread; ++e) {
    const int k = k0 + e;
    wgt[e] = 0;
    if (k < k1) wgt[e] = mode == 0 ? resid_weight(pt[row + k], pd[row + k]) : target_weight(pt[row + k]);
  }
  uint64_t local = 0;
#pragma unroll
  for (int e = 0; e < kResidPerThread; ++e) local += wgt[e];
  uint64_t total;
  const uint64_t excl = block_exclusive_scan(local, &total);
  const uint64_t rem = s_rem;
  if (local > 0 && excl <= rem && rem < excl + local) {
    uint64_t run = excl;
    int tok = -1;
#pragma unroll
    for (int e = 0; e < kResidPerThread; ++e) {
      run += wgt[e];
      if (tok < 0 && run > rem) tok = k0 + e;
    }
    resample_token[b] = tok;
  }
}

}  // namespace tv

extern "C" size_t tree_accept_workspace_size(int32_t batch, int32_t vocab) {
  if (batch <= 0 || vocab <= 0) return 0;
  const size_t chunks = static_cast<size_t>(tv::ceil_div(vocab, tv::kResidChunk));
  const size_t head = (static_cast<size_t>(batch) * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
  return head + static_cast<size_t>(batch) * chunks * 2 * sizeof(uint64_t);
}

extern "C" int tree_accept(const float* p_target, const float* p_draft, const int32_t* token,
                           const float* u_accept, const float* u_resample, const int32_t* parent,
                           const int32_t* cu_nodes, int32_t batch, int32_t total_nodes,
                           int32_t max_nodes, int32_t vocab, int32_t max_path,
                           int32_t* accept_len, int32_t* path, int32_t* resample_node,
                           int32_t* resample_token, uint8_t* node_ok, void* workspace,
                           size_t workspace_bytes, int32_t* err, void* stream) {
  tv::clear_error();
  if (batch < 0 || total_nodes < 0 || max_path < 0)
    return tv::fail(TV_EINVAL, "tree_accept: negative size");
  if (vocab <= 0 || vocab > tv::kMaxVocab)
    return tv::fail(TV_EUNSUPPORTED, "tree_accept: vocab must be in [1, 262144]");
  if (max_nodes < 1 || max_nodes > TV_MAX_NODES)
    return tv::fail(TV_EUNSUPPORTED, "tree_accept: max_nodes must be in [1, 2048]");
  if (batch == 0) return TV_OK;
  if (cu_nodes == nullptr || err == nullptr || accept_len == nullptr ||
      resample_node == nullptr || resample_token == nullptr || (max_path > 0 && path == nullptr))
    return tv::fail(TV_EINVAL, "tree_accept: null output or cu_nodes/err");
  if (total_nodes > 0 && (p_target == nullptr || p_draft == nullptr || token == nullptr ||
                          u_accept == nullptr || u_resample == nullptr || parent == nullptr))
    return tv::fail(TV_EINVAL, "tree_accept: null input array");
  const size_t need = tree_accept_workspace_size(batch, vocab);
  if (workspace == nullptr || workspace_bytes < need)
    return tv::fail(TV_EWORKSPACE, "tree_accept: workspace missing or too small");
  auto s = static_cast<hipStream_t>(stream);
  const int chunks = tv::ceil_div(vocab, tv::kResidChunk);
  int32_t* ws_c = static_cast<int32_t*>(workspace);
  const size_t head = (static_cast<size_t>(batch) * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
  uint64_t* part = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + head);
  if (vocab <= tv::kFusedVocab) {  // one kernel: the walk's workgroup also resamples
    hipLaunchKernelGGL(tv::k_accept_walk<true>, dim3(batch), dim3(tv::kAcceptThreads), 0, s,
                       p_target, p_draft, token, u_accept, u_resample, parent, cu_nodes, max_nodes,
                       vocab, max_path, accept_len, path, resample_node, resample_token, node_ok,
                       ws_c, err);
    return tv::check_launch("tree_accept/walk");
  }
  hipLaunchKernelGGL(tv::k_accept_walk<false>, dim3(batch), dim3(tv::kAcceptThreads), 0, s,
                     p_target, p_draft, token, u_accept, u_resample, parent, cu_nodes, max_nodes,
                     vocab, max_path, accept_len, path, resample_node, resample_token, node_ok,
                     ws_c, err);
  int st = tv::check_launch("tree_accept/walk");
  if (st != TV_OK) return st;
  hipLaunchKernelGGL(tv::k_resid_partial, dim3(chunks, batch), dim3(tv::kAcceptThreads), 0, s,
                     p_target, p_draft, cu_nodes, vocab, chunks, ws_c, part);
  st = tv::check_launch("tree_accept/partial");
  if (st != TV_OK) return st;
  hipLaunchKernelGGL(tv::k_resid_select, dim3(batch), dim3(tv::kAcceptThreads), 0, s, p_target,
                     p_draft, u_resample, cu_nodes, vocab, chunks, ws_c, part, resample_token, err);
  return tv::check_launch("tree_accept/select");
}
