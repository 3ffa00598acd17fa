// tree_accept: fused acceptance of a verified draft tree, no host round-trip.
//
// What is computed follows page "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力
// 机制与显存碎片整理联合加速" (ufo.work/2026/537), §2.2.3: each node's acceptance
// probability min(1, p_target / p_draft) at its drafted token, one uniform per node,
// a depth-first walk from the root that stops below the first rejected node, and the
// longest accepted path, all inside one GPU kernel.  At the rejection point a token is
// resampled (page "端侧大模型推测解码草稿模型动态剪枝策略：详解基于重要性采样的树形验证并行加速
// 机制" (ufo.work/2026/525), §1.2) from norm(max(0, p_target - p_draft)), falling back
// to p_target itself when that has no mass (same page, §7.2).  When the path ends at
// a leaf and the caller passes the target distribution at that leaf's own context
// (the one forward pass over the tree gives one at every node, page 537 §2.2.3), the
// extra token is drawn from it instead: the bonus token.
//
// One launch per call.  Up to 65536 vocabulary entries, one workgroup per sequence
// walks the tree and scans the row it samples.  Above that, there is a workgroup per
// (sequence, vocabulary chunk), all chunks of a sequence on one die: every workgroup
// of a sequence repeats the walk (a few hundred gathered floats, cached in the die's
// L2 after the first), sums the integer weights of its chunk of
// the sampled row, publishes them and takes a ticket; the workgroup that takes the
// sequence's last ticket finds the chunk and then the element where the running sum
// passes the threshold.  No workgroup waits for another.  The weights are integers
// (floor of the fp64 difference times 2^40), so every sum is exact and the token does
// not depend on how the vocabulary is split.
#include <limits.h>

#include <cstdio>

#include "accept.h"

namespace tv {

namespace {

constexpr int kAcceptThreads = 256;
constexpr int kResidChunk = 4096;                       // vocabulary entries per chunk
constexpr int kResidPerThread = kResidChunk / kAcceptThreads;
constexpr int kFusedVocab = kAcceptFusedVocab;  // up to this vocabulary one workgroup per sequence
constexpr int kMaxVocab = 1 << 18;
constexpr int kMaxResidChunks = kMaxVocab / kResidChunk;
// A sequence's ticket word sits alone in a 128-byte line: the 32 chunk workgroups of
// 16 sequences took their tickets on one line before (serving-64: 30.6 -> 28.6 us)
constexpr int kTicketStride = 32;
static_assert(kResidPerThread % 4 == 0, "whole float4 per thread");

#pragma clang fp contract(off)

struct AcceptArgs {
  const float* pt;          // [total_nodes, vocab]
  const float* pd;
  const int32_t* token;
  const float* u_acc;
  const float* u_res;
  const int32_t* parent;
  const int32_t* cu_nodes;
  const float* p_own;       // [own_rows, vocab] or null
  const int32_t* own_row;   // [total_nodes] or null
  int own_rows, max_nodes, vocab, max_path;
  int32_t* accept_len;
  int32_t* path;
  int32_t* resample_node;
  int32_t* resample_token;
  uint8_t* node_ok;
  int* tickets;             // finish tickets (chunked launch), one per kTicketStride ints,
                            // zero between calls
  uint64_t* part;           // [batch, chunks, 2] chunk sums (chunked launch)
  int32_t* err;
};

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

// weight of entry k in mode 0 (residual pt - pd) or 1 (pt alone); pd_row is null for
// a bonus row, whose residual weights are all zero
__device__ __forceinline__ uint64_t weight_at(const float* __restrict__ pt_row,
                                              const float* __restrict__ pd_row, int k, int mode) {
  if (mode == 1) return target_weight(pt_row[k]);
  return pd_row != nullptr ? resid_weight(pt_row[k], pd_row[k]) : 0ull;
}

// Token of row (pt_row, pd_row) inside one workgroup (small vocabularies): thread t
// sums the integer weights of its contiguous slice, a block scan over the slices
// finds the one where the running sum passes the threshold, and that thread walks
// its slice again.  Same integers as the chunked path, so the same token.
__device__ void sample_in_block(const float* __restrict__ pt_row, const float* __restrict__ pd_row,
                                int vocab, float u, int32_t* __restrict__ out_token,
                                int32_t* __restrict__ err) {
  const int tid = threadIdx.x;
  const int len = ((vocab + kAcceptThreads - 1) / kAcceptThreads + 3) & ~3;
  const int k0 = min(vocab, tid * len), k1 = min(vocab, k0 + len);
  uint64_t sr = 0, st = 0;
  for (int k = k0; k < k1; ++k) {
    const float t = pt_row[k];
    if (pd_row != nullptr) sr += resid_weight(t, pd_row[k]);
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
      run += weight_at(pt_row, pd_row, k, mode);
      if (run > t_thr) {
        *out_token = k;
        break;
      }
    }
  }
}

// Chunk `chunk` of the sampled row: sums of the residual and target weights.
__device__ __forceinline__ void chunk_sums(const float* __restrict__ pt_row,
                                           const float* __restrict__ pd_row, int vocab, int chunk,
                                           uint64_t& sr, uint64_t& st) {
  const int k0 = chunk * kResidChunk;
  const int k1 = min(vocab, k0 + kResidChunk);
  sr = 0;
  st = 0;
  const uintptr_t align = reinterpret_cast<uintptr_t>(pt_row) |
                          (pd_row != nullptr ? reinterpret_cast<uintptr_t>(pd_row) : 0);
  if ((align & 15) == 0 && k1 - k0 == kResidChunk) {
    // whole chunk, rows 16-byte aligned: each thread takes 4 float4 of each row,
    // all loads in flight at once
    const float4* t4 = reinterpret_cast<const float4*>(pt_row + k0);
    float4 tv[kResidPerThread / 4];
#pragma unroll
    for (int j = 0; j < kResidPerThread / 4; ++j) tv[j] = t4[threadIdx.x + j * kAcceptThreads];
    if (pd_row != nullptr) {
      const float4* d4 = reinterpret_cast<const float4*>(pd_row + k0);
      float4 dv[kResidPerThread / 4];
#pragma unroll
      for (int j = 0; j < kResidPerThread / 4; ++j) dv[j] = d4[threadIdx.x + j * kAcceptThreads];
#pragma unroll
      for (int j = 0; j < kResidPerThread / 4; ++j)
        sr += resid_weight(tv[j].x, dv[j].x) + resid_weight(tv[j].y, dv[j].y) +
              resid_weight(tv[j].z, dv[j].z) + resid_weight(tv[j].w, dv[j].w);
    }
#pragma unroll
    for (int j = 0; j < kResidPerThread / 4; ++j)
      st += target_weight(tv[j].x) + target_weight(tv[j].y) + target_weight(tv[j].z) +
            target_weight(tv[j].w);
  } else {
    for (int k = k0 + threadIdx.x; k < k1; k += kAcceptThreads) {
      const float t = pt_row[k];
      if (pd_row != nullptr) sr += resid_weight(t, pd_row[k]);
      st += target_weight(t);
    }
  }
}

// The workgroup that takes a sequence's last ticket: total mass, exact threshold,
// the chunk where the running sum passes it, then the element inside that chunk.
__device__ void select_token(const AcceptArgs& a, int b, int chunks, const float* __restrict__ pt_row,
                             const float* __restrict__ pd_row, float u) {
  __shared__ int s_mode, s_chunk;
  __shared__ uint64_t s_rem;
  __shared__ uint64_t s_part[2 * kMaxResidChunks];
  const int tid = threadIdx.x;
  uint64_t* mine = a.part + static_cast<long>(b) * chunks * 2;
  for (int k = tid; k < 2 * chunks; k += kAcceptThreads)
    s_part[k] = __hip_atomic_load(mine + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
      a.resample_token[b] = -1;
      atomicOr(a.err, TV_ERR_ZERO_MASS);
    }
  }
  __syncthreads();
  const int mode = s_mode;
  if (mode < 0) return;
  const int k0 = s_chunk * kResidChunk + tid * kResidPerThread;
  const int k1 = min(a.vocab, min(k0 + kResidPerThread, (s_chunk + 1) * kResidChunk));
  // this thread's weights, loaded once (all loads in flight together) and kept for
  // the walk
  uint64_t wgt[kResidPerThread];
  const uintptr_t align = reinterpret_cast<uintptr_t>(pt_row + k0) |
                          (pd_row != nullptr ? reinterpret_cast<uintptr_t>(pd_row + k0) : 0);
  if (k1 - k0 == kResidPerThread && (align & 15) == 0) {
    // a whole slice, 16-byte aligned: 16-byte loads (four per row), all in flight
    float t[kResidPerThread], d[kResidPerThread];
#pragma unroll
    for (int j = 0; j < kResidPerThread / 4; ++j) {
      const float4 x = reinterpret_cast<const float4*>(pt_row + k0)[j];
      t[4 * j] = x.x, t[4 * j + 1] = x.y, t[4 * j + 2] = x.z, t[4 * j + 3] = x.w;
    }
    if (mode == 0 && pd_row != nullptr) {
#pragma unroll
      for (int j = 0; j < kResidPerThread / 4; ++j) {
        const float4 x = reinterpret_cast<const float4*>(pd_row + k0)[j];
        d[4 * j] = x.x, d[4 * j + 1] = x.y, d[4 * j + 2] = x.z, d[4 * j + 3] = x.w;
      }
    }
#pragma unroll
    for (int e = 0; e < kResidPerThread; ++e)
      wgt[e] = mode == 1 ? target_weight(t[e])
                         : (pd_row != nullptr ? resid_weight(t[e], d[e]) : 0ull);
  } else {
#pragma unroll
    for (int e = 0; e < kResidPerThread; ++e) {
      const int k = k0 + e;
      wgt[e] = k < k1 ? weight_at(pt_row, pd_row, k, mode) : 0ull;
    }
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
    a.resample_token[b] = tok;
  }
}

// Grid (chunks, batch).  kChunked false: one chunk, the workgroup samples its row
// alone.  Workgroup (0, b) writes the walk's outputs; with chunks, every workgroup of
// the sequence repeats the walk (same inputs, same decisions).
template <bool kChunked>
__global__ void __launch_bounds__(kAcceptThreads) k_accept(AcceptArgs a, int batch, int chunks) {
  __shared__ int16_t s_par[TV_MAX_NODES];
  __shared__ uint8_t s_acc[TV_MAX_NODES];
  __shared__ float s_ures[TV_MAX_NODES];
  __shared__ int s_bad, s_key, s_child, s_err, s_last;
  const int tid = threadIdx.x;
  // workgroup i runs on die i % 8: the chunks of sequence b all go to die b % 8, so
  // the walk's gathers and the chunk the last one re-reads are shared in its L2
  const int lin = blockIdx.x, die = lin % 8, q = lin / 8;
  const int chunk = q % chunks, b = (q / chunks) * 8 + die;
  if (b >= batch) return;
  const bool writer = chunk == 0;
  const int n0 = a.cu_nodes[b];
  const int n = a.cu_nodes[b + 1] - n0;
  if (tid == 0) {
    s_bad = 0;
    s_key = -1;
    s_child = INT_MAX;
    s_err = 0;
  }
  if (writer)
    for (int j = tid; j < a.max_path; j += kAcceptThreads)
      a.path[static_cast<long>(b) * a.max_path + j] = -1;
  __syncthreads();
  if (n > a.max_nodes) {
    if (!writer) return;
    if (a.node_ok != nullptr)
      for (int i = tid; i < n; i += kAcceptThreads) a.node_ok[n0 + i] = 0;
    if (tid == 0) {
      atomicOr(a.err, TV_ERR_TOO_MANY_NODES);
      a.accept_len[b] = 0;
      a.resample_node[b] = -1;
      a.resample_token[b] = -1;
    }
    return;
  }
  // parent links, and 1-2. the ratio test per node: u < min(1, pt/pd)  <=>
  // (double)u * pd < pt for u in [0, 1); every node's resample uniform is kept too,
  // so that all of a node's loads go out together
  int my_err = 0;
  for (int i = tid; i < n; i += kAcceptThreads) {
    const long g = n0 + i;
    const int p = a.parent[g];
    const int tok = a.token[g];
    const float u = a.u_acc[g];
    s_ures[i] = a.u_res[g];
    s_par[i] = static_cast<int16_t>(p);
    if (p >= i || p < -1) s_bad = 1;
    bool acc = false;
    if (tok < 0 || tok >= a.vocab) {
      my_err |= TV_ERR_TOKEN;
    } else if (!(u >= 0.0f && u < 1.0f)) {
      my_err |= TV_ERR_UNIFORM;
    } else {
      const long off = g * a.vocab + tok;
      acc = static_cast<double>(u) * static_cast<double>(a.pd[off]) < static_cast<double>(a.pt[off]);
    }
    s_acc[i] = acc ? 1 : 0;
  }
  if (my_err) atomicOr(&s_err, my_err);
  __syncthreads();
  if (s_bad) {
    if (!writer) return;
    if (a.node_ok != nullptr)
      for (int i = tid; i < n; i += kAcceptThreads) a.node_ok[n0 + i] = 0;
    if (tid == 0) {
      atomicOr(a.err, TV_ERR_BAD_PARENT);
      a.accept_len[b] = 0;
      a.resample_node[b] = -1;
      a.resample_token[b] = -1;
    }
    return;
  }
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
    if (writer && a.node_ok != nullptr) a.node_ok[n0 + i] = ok ? 1 : 0;
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
  // the row to sample: the rejection node's (residual), or the bonus row at the
  // winner's own context when the winner is a leaf
  const int c = s_child == INT_MAX ? -1 : s_child;
  int e = 0, snode = -1;
  const float* row_t = nullptr;
  const float* row_d = nullptr;
  float u = 0.0f;
  if (c >= 0) {
    snode = c;
    u = s_ures[c];
    if (u >= 0.0f && u < 1.0f) {
      row_t = a.pt + static_cast<long>(n0 + c) * a.vocab;
      row_d = a.pd + static_cast<long>(n0 + c) * a.vocab;
    } else {
      e |= TV_ERR_UNIFORM;
    }
  } else if (w >= 0 && a.own_row != nullptr) {
    const int r = a.own_row[n0 + w];
    if (r < -1 || r >= a.own_rows) {
      e |= TV_ERR_ROW;
    } else if (r >= 0) {
      snode = w;
      u = s_ures[w];
      if (u >= 0.0f && u < 1.0f) row_t = a.p_own + static_cast<long>(r) * a.vocab;
      else e |= TV_ERR_UNIFORM;
    }
  }
  if (writer && tid == 0) {
    e |= s_err;
    a.accept_len[b] = depth_w;
    int v = w;
    for (int k = depth_w - 1; k >= 0; --k) {
      if (k < a.max_path) a.path[static_cast<long>(b) * a.max_path + k] = v;
      v = s_par[v];
    }
    if (depth_w > a.max_path) e |= TV_ERR_PATH;
    a.resample_node[b] = snode;
    if (row_t == nullptr) a.resample_token[b] = -1;
    if (e) atomicOr(a.err, e);
  }
  if (row_t == nullptr) return;
  if constexpr (!kChunked) {
    sample_in_block(row_t, row_d, a.vocab, u, a.resample_token + b, a.err);
  } else {
    uint64_t sr, st;
    chunk_sums(row_t, row_d, a.vocab, chunk, sr, st);
    sr = block_sum_u64(sr);
    st = block_sum_u64(st);
    // publish the chunk's sums and take a ticket; the last of the sequence's
    // workgroups selects.  The sums are written by device-scope atomic exchanges,
    // which complete at the device's coherence point before they return (the wait
    // below), and only then is the ticket taken; the selecting workgroup reads them
    // with device-scope atomic loads.  So it sees every chunk's sums whichever die
    // wrote them, without a cache-wide release or acquire (an L2 write-back per
    // workgroup made 64 sequences x 32 chunks take 63 us instead of 28).
    if (tid == 0) {
      uint64_t* slot = a.part + (static_cast<long>(b) * chunks + chunk) * 2;
      const uint64_t o0 = __hip_atomic_exchange(slot, sr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t o1 =
          __hip_atomic_exchange(slot + 1, st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("s_waitcnt vmcnt(0)" : : "v"(o0), "v"(o1) : "memory");  // both returned
      const bool last = __hip_atomic_fetch_add(a.tickets + kTicketStride * b, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) == chunks - 1;
      // every workgroup of the sequence has taken its ticket: zero it for the next call
      if (last) __hip_atomic_store(a.tickets + kTicketStride * b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    select_token(a, b, chunks, row_t, row_d, u);
  }
}

}  // namespace

}  // namespace tv

// Workspace: [batch] finish tickets, one per 128-byte line (256-byte aligned), then
// [batch, chunks, 2] sums.
namespace tv {
size_t accept_ticket_bytes(int batch) {
  return (static_cast<size_t>(batch) * kTicketStride * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
}
}  // namespace tv

extern "C" size_t tree_accept_workspace_size(int32_t batch, int32_t vocab) {
  if (batch <= 0 || vocab <= 0) return 0;
  const size_t chunks = static_cast<size_t>(tv::ceil_div(vocab, tv::kResidChunk));
  return tv::accept_ticket_bytes(batch) + static_cast<size_t>(batch) * chunks * 2 * sizeof(uint64_t);
}

namespace tv {

// Shared body of tree_accept and its variants: checks, then one launch.
int accept_launch(const char* fn, const float* p_target, const float* p_draft,
                  const int32_t* token, const float* u_accept, const float* u_resample,
                  const int32_t* parent, const int32_t* cu_nodes, const float* p_own,
                  const int32_t* own_row, int32_t own_rows, int32_t batch, int32_t total_nodes,
                  int32_t max_nodes, int32_t vocab, int32_t max_path, int32_t* accept_len,
                  int32_t* path, int32_t* resample_node, int32_t* resample_token,
                  uint8_t* node_ok, void* workspace, size_t workspace_bytes, int32_t* err,
                  void* stream) {
  char msg[160];
  auto bad = [&](int status, const char* what) {
    snprintf(msg, sizeof(msg), "%s: %s", fn, what);
    return fail(status, msg);
  };
  if (batch < 0 || total_nodes < 0 || max_path < 0 || own_rows < 0)
    return bad(TV_EINVAL, "negative size");
  if (vocab <= 0 || vocab > kMaxVocab)
    return bad(TV_EUNSUPPORTED, "vocab must be in [1, 262144]");
  if (max_nodes < 1 || max_nodes > TV_MAX_NODES)
    return bad(TV_EUNSUPPORTED, "max_nodes must be in [1, 2048]");
  if (batch == 0) return TV_OK;
  if (cu_nodes == nullptr || err == nullptr || accept_len == nullptr ||
      resample_node == nullptr || resample_token == nullptr || (max_path > 0 && path == nullptr))
    return bad(TV_EINVAL, "null output or cu_nodes/err");
  if (total_nodes > 0 && (p_target == nullptr || p_draft == nullptr || token == nullptr ||
                          u_accept == nullptr || u_resample == nullptr || parent == nullptr))
    return bad(TV_EINVAL, "null input array");
  if (own_row != nullptr && own_rows > 0 && p_own == nullptr)
    return bad(TV_EINVAL, "own_row given without p_own");
  const int chunks = ceil_div(vocab, kResidChunk);
  const bool chunked = vocab > kFusedVocab;
  if (chunked && (workspace == nullptr || workspace_bytes < tree_accept_workspace_size(batch, vocab)))
    return bad(TV_EWORKSPACE, "workspace missing or too small");
  AcceptArgs a{};
  a.pt = p_target;
  a.pd = p_draft;
  a.token = token;
  a.u_acc = u_accept;
  a.u_res = u_resample;
  a.parent = parent;
  a.cu_nodes = cu_nodes;
  a.p_own = p_own;
  a.own_row = own_row;
  a.own_rows = own_row != nullptr ? own_rows : 0;
  a.max_nodes = max_nodes;
  a.vocab = vocab;
  a.max_path = max_path;
  a.accept_len = accept_len;
  a.path = path;
  a.resample_node = resample_node;
  a.resample_token = resample_token;
  a.node_ok = node_ok;
  a.err = err;
  auto s = static_cast<hipStream_t>(stream);
  const int padded = ceil_div(batch, 8) * 8;
  if (!chunked) {
    hipLaunchKernelGGL(k_accept<false>, dim3(padded), dim3(kAcceptThreads), 0, s, a, batch, 1);
  } else {
    const size_t head = accept_ticket_bytes(batch);
    a.tickets = static_cast<int*>(workspace);
    a.part = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + head);
    hipLaunchKernelGGL(k_accept<true>, dim3(padded * chunks), dim3(kAcceptThreads), 0, s, a,
                       batch, chunks);
  }
  return check_launch(fn);
}

}  // namespace tv

extern "C" int tree_accept(const float* p_target, const float* p_draft, const int32_t* token,
                           const float* u_accept, const float* u_resample, const int32_t* parent,
                           const int32_t* cu_nodes, const float* p_own, const int32_t* own_row,
                           int32_t own_rows, int32_t batch, int32_t total_nodes,
                           int32_t max_nodes, int32_t vocab, int32_t max_path,
                           int32_t* accept_len, int32_t* path, int32_t* resample_node,
                           int32_t* resample_token, uint8_t* node_ok, void* workspace,
                           size_t workspace_bytes, int32_t* err, void* stream) {
  tv::clear_error();
  return tv::accept_launch("tree_accept", p_target, p_draft, token, u_accept, u_resample, parent,
                           cu_nodes, p_own, own_row, own_rows, batch, total_nodes, max_nodes,
                           vocab, max_path, accept_len, path, resample_node, resample_token,
                           node_ok, workspace, workspace_bytes, err, stream);
}
