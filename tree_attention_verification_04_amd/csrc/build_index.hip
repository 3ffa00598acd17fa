// tree_build_index: parent array -> depth and ancestor-or-self bitsets.
//
// The visibility rule is the tree mask of page "端云协同推测解码中草稿模型动态生成与验证并行化：
// 探究树形注意力机制与显存碎片整理联合加速" (ufo.work/2026/537), §2.2.2, equation M_tree:
// node i sees node j iff j is i or one of its ancestors.  Appendix B of the same
// page keeps a per-node ancestor bitmap instead of a dense mask; here each node
// gets `words` 64-bit words, so memory grows linearly with the node count.
//
// A workgroup per (sequence, block of 256 nodes): the parent links of the block's
// nodes and of every node before them (ancestors have smaller indices) go to LDS
// (16-bit; a link that does not point to a smaller index is stored as -2), then one
// thread per node walks from its node towards the prefix through LDS.  The walk
// visits the node's words in descending order, so the thread keeps the current word
// in a register and writes each word once as the walk leaves it (words above the
// node's own and below its last ancestor are zero).  (Staging the rows in LDS for a
// coalesced copy-out measured no faster.)  A -2 link ends the walk and raises
// TV_ERR_BAD_PARENT, so every walk terminates whatever the input.  Nodes outside
// [0, total_nodes) (a cu_nodes array that breaks the contract) are neither read nor
// written.
#include <stdio.h>

#include "tv_common.h"

namespace tv {

constexpr int kIndexThreads = 256;  // nodes per workgroup, one per thread
constexpr int16_t kBadLink = -2;

__global__ void __launch_bounds__(kIndexThreads) k_build_index(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ cu_nodes, int /*batch*/,
    int total_nodes, int max_nodes, const int32_t* __restrict__ prefix_len,
    uint64_t* __restrict__ anc, int words, int32_t* __restrict__ depth_out,
    int32_t* __restrict__ pos_out, int32_t* __restrict__ err) {
  __shared__ int16_t s_par[TV_MAX_NODES];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int c0 = blockIdx.y * kIndexThreads;  // first local node of this workgroup
  const bool last_block = blockIdx.y == gridDim.y - 1;
  const int n0 = cu_nodes[b];
  const int count = cu_nodes[b + 1] - n0;
  // local nodes that exist in the arrays: all of [0, count) for a valid cu_nodes
  const int i_lo = max(0, -n0);
  const int i_hi = static_cast<int>(min(static_cast<long>(count), static_cast<long>(total_nodes) - n0));
  if (count > max_nodes) {  // the last block also takes the nodes past the grid
    const int j_lo = max(i_lo, c0), j_hi = last_block ? i_hi : min(i_hi, c0 + kIndexThreads);
    for (long t = tid; t < static_cast<long>(j_hi - j_lo) * words; t += kIndexThreads)
      anc[(static_cast<long>(n0) + j_lo) * words + t] = 0;
    for (int i = j_lo + tid; i < j_hi; i += kIndexThreads) depth_out[n0 + i] = 0;
    if (tid == 0 && blockIdx.y == 0) atomicOr(err, TV_ERR_TOO_MANY_NODES);
    return;
  }
  const int j_lo = max(i_lo, c0), j_hi = min(i_hi, c0 + kIndexThreads);
  const int need = min(count, c0 + kIndexThreads);  // links of nodes [0, need)
  for (int i = tid; i < need; i += kIndexThreads) {
    int p = -1;
    if (i >= i_lo && i < i_hi) p = parent[n0 + i];
    s_par[i] = (p >= i || p < -1) ? kBadLink : static_cast<int16_t>(p);
  }
  __syncthreads();
  const int i = c0 + tid;
  if (i >= j_lo && i < j_hi) {
    uint64_t* row = anc + static_cast<long>(n0 + i) * words;
    int cw = i >> 6;  // the word being filled
    for (int w = words - 1; w > cw; --w) row[w] = 0;
    uint64_t cur = 0;
    int v = i, steps = 0;
    bool bad = false;
    while (v >= 0) {
      const int vw = v >> 6;
      while (cw > vw) {
        row[cw] = cur;
        cur = 0;
        --cw;
      }
      cur |= 1ull << (v & 63);
      ++steps;
      const int p = s_par[v];
      if (p == kBadLink) {
        bad = true;
        break;
      }
      v = p;
    }
    row[cw] = cur;
    for (int w = cw - 1; w >= 0; --w) row[w] = 0;
    depth_out[n0 + i] = steps;
    if (pos_out != nullptr) pos_out[n0 + i] = prefix_len[b] + steps - 1;
    if (bad) atomicOr(err, TV_ERR_BAD_PARENT);
  }
}

}  // namespace tv

extern "C" int tree_build_index(const int32_t* parent, const int32_t* cu_nodes, int32_t batch,
                                int32_t total_nodes, int32_t max_nodes,
                                const int32_t* prefix_len, uint64_t* anc_bits, int32_t words,
                                int32_t* depth, int32_t* pos, int32_t* err, void* stream) {
  tv::clear_error();
  if (batch < 0 || total_nodes < 0) return tv::fail(TV_EINVAL, "tree_build_index: negative size");
  if (max_nodes < 1 || max_nodes > TV_MAX_NODES)
    return tv::fail(TV_EUNSUPPORTED, "tree_build_index: max_nodes must be in [1, 2048]");
  if (words < tv::ceil_div(max_nodes, 64))
    return tv::fail(TV_EINVAL, "tree_build_index: words < ceil(max_nodes / 64)");
  if (cu_nodes == nullptr || err == nullptr)
    return tv::fail(TV_EINVAL, "tree_build_index: null cu_nodes or err");
  if (pos != nullptr && prefix_len == nullptr)
    return tv::fail(TV_EINVAL, "tree_build_index: pos requested without prefix_len");
  if (total_nodes == 0 || batch == 0) return TV_OK;
  if (parent == nullptr || anc_bits == nullptr || depth == nullptr)
    return tv::fail(TV_EINVAL, "tree_build_index: null parent, anc_bits or depth");
  const dim3 grid(static_cast<unsigned>(batch), tv::ceil_div(max_nodes, tv::kIndexThreads));
  hipLaunchKernelGGL(tv::k_build_index, grid, dim3(tv::kIndexThreads), 0,
                     static_cast<hipStream_t>(stream), parent, cu_nodes, batch, total_nodes,
                     max_nodes, prefix_len, anc_bits, words, depth, pos, err);
  return tv::check_launch("tree_build_index");
}
