// tree_build_index: parent array -> depth and ancestor-or-self bitsets.
//
// The visibility rule is the tree mask of page "端云协同推测解码中草稿模型动态生成与验证并行化：
// 探究树形注意力机制与显存碎片整理联合加速" (ufo.work/2026/537), §2.2.2, equation M_tree:
// node i sees node j iff j is i or one of its ancestors.  Appendix B of the same
// page keeps a per-node ancestor bitmap instead of a dense mask; here each node
// gets `words` 64-bit words, so memory grows linearly with the node count.
//
// One thread per (node, word).  The thread walks from its node towards the
// prefix; ancestors have strictly smaller indices, so the thread for word w
// stops as soon as the walk drops below 64 * w.  The word-0 thread walks the
// whole path and also writes the depth.  A parent link that does not point to
// a smaller index ends the walk and raises TV_ERR_BAD_PARENT, so every walk
// terminates whatever the input.
#include <stdio.h>

#include "tv_common.h"

namespace tv {

__global__ void __launch_bounds__(256) k_build_index(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ cu_nodes, int batch,
    int total_nodes, int max_nodes, const int32_t* __restrict__ prefix_len,
    uint64_t* __restrict__ anc, int words, int32_t* __restrict__ depth_out,
    int32_t* __restrict__ pos_out, int32_t* __restrict__ err) {
  const long tid = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tid >= static_cast<long>(total_nodes) * words) return;
  const int node = static_cast<int>(tid / words);
  const int w = static_cast<int>(tid % words);
  const int b = seq_of_node(cu_nodes, batch, node);
  const int n0 = cu_nodes[b];
  const int count = cu_nodes[b + 1] - n0;
  if (count > max_nodes) {
    if (node == n0 && w == 0) atomicOr(err, TV_ERR_TOO_MANY_NODES);
    anc[tid] = 0;
    if (w == 0) depth_out[node] = 0;
    return;
  }
  const int word_lo = w * 64;
  uint64_t bits = 0;
  int v = node - n0;
  int steps = 0;
  bool bad = false;
  while (v >= 0) {
    if (v < word_lo) {
      if (w != 0) break;  // word 0 has word_lo == 0 and never gets here
    } else if (v < word_lo + 64) {
      bits |= 1ull << (v - word_lo);
    }
    ++steps;
    const int p = parent[n0 + v];
    if (p >= v || p < -1) {
      bad = true;
      break;
    }
    v = p;
  }
  anc[tid] = bits;
  if (w == 0) {
    depth_out[node] = steps;
    if (pos_out != nullptr) pos_out[node] = prefix_len[b] + steps - 1;
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
  const long threads = static_cast<long>(total_nodes) * words;
  const int grid = static_cast<int>((threads + 255) / 256);
  hipLaunchKernelGGL(tv::k_build_index, dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), parent, cu_nodes, batch, total_nodes,
                     max_nodes, prefix_len, anc_bits, words, depth, pos, err);
  return tv::check_launch("tree_build_index");
}
