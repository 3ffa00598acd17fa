// tree_commit_kv: append each sequence's accepted path to its paged prefix.
//
// Node path[b][j] holds the keys and values of position prefix_len[b] + j; its rows
// of every KV head are copied there, and the prefix grows by the accepted length, so
// the next verify round reads them as shared prefix (page
// "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力机制与显存碎片整理联合加速"
// (ufo.work/2026/537), §5.2, prefix caching; page "端侧大模型推测解码草稿模型动态剪枝策略：
// 详解基于重要性采样的树形验证并行加速机制" (ufo.work/2026/525), §2.3.2, the tree's KV
// slots return to the pool after verification).
//
// One workgroup per sequence: thread 0 validates the path and the blocks the new
// positions fall in, every thread then scans a stripe of the other sequences' table
// rows for those blocks (a prefix block shared by several sequences may be read by
// all of them, but the block a commit writes must be the sequence's own: a shared
// prefix whose length is not a multiple of 64 ends inside such a block, and copying
// on write is the caller's job), every thread copies 16-byte chunks of (path row, KV
// head), and thread 0 writes the new prefix length after the copy (all threads read
// the old one first).  Pure data movement: HBM-bound, 2 x rows x hkv x head_dim x
// elt bytes read and written.
#include "tv_common.h"

namespace tv {

namespace {

constexpr int kCommitThreads = 256;
constexpr int kMaxPath = 4096;      // positions one commit may append
constexpr int kMaxDestBlocks = kMaxPath / TV_BLOCK + 1;  // blocks they may fall in

struct CommitArgs {
  const char* k_tree;
  const char* v_tree;
  const int32_t* cu_nodes;
  const int32_t* accept_len;
  const int32_t* path;
  char* k_cache;
  char* v_cache;
  const int32_t* block_table;
  int32_t* prefix_len;
  int32_t* err;
  int max_path, hkv, row_bytes, num_blocks, max_blocks, batch;
};

__global__ void __launch_bounds__(kCommitThreads) k_commit_kv(CommitArgs a) {
  __shared__ int s_ok, s_ndest;
  __shared__ int s_dest[kMaxDestBlocks];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int n0 = a.cu_nodes[b];
  const int count = a.cu_nodes[b + 1] - n0;
  const int len = a.accept_len[b];
  const int p0 = a.prefix_len[b];
  const int32_t* path = a.path + static_cast<long>(b) * a.max_path;
  const int32_t* bt = a.block_table + static_cast<long>(b) * a.max_blocks;
  if (tid == 0) {
    int bits = 0;
    if (len < 0 || len > a.max_path) {
      bits = TV_ERR_PATH;
    } else {
      for (int j = 0; j < len; ++j)
        if (path[j] < 0 || path[j] >= count) bits = TV_ERR_PATH;
      if (bits == 0 && len > 0) {
        if (p0 < 0 || static_cast<long>(p0) + len > static_cast<long>(a.max_blocks) * TV_BLOCK) {
          bits = TV_ERR_BLOCK;
        } else if ((p0 + len - 1) / TV_BLOCK - p0 / TV_BLOCK >= kMaxDestBlocks) {
          bits = TV_ERR_PATH;
        } else {
          for (int lb = p0 / TV_BLOCK; lb <= (p0 + len - 1) / TV_BLOCK; ++lb) {
            if (bt[lb] < 0 || bt[lb] >= a.num_blocks) bits = TV_ERR_BLOCK;
            s_dest[lb - p0 / TV_BLOCK] = bt[lb];
          }
        }
      }
    }
    s_ndest = bits == 0 && len > 0 ? (p0 + len - 1) / TV_BLOCK - p0 / TV_BLOCK + 1 : 0;
    s_ok = bits;
  }
  __syncthreads();
  // a destination block that another sequence's table also maps is not written
  const int ndest = s_ndest;
  if (ndest > 0) {
    bool shared = false;
    const long entries = static_cast<long>(a.batch) * a.max_blocks;
    for (long e = tid; e < entries; e += kCommitThreads) {
      if (e / a.max_blocks == b) continue;
      const int blk = a.block_table[e];
      for (int d = 0; d < ndest; ++d) shared |= blk == s_dest[d];
    }
    if (shared) atomicOr(&s_ok, TV_ERR_BLOCK);
    __syncthreads();
  }
  if (tid == 0 && s_ok) atomicOr(a.err, s_ok);
  if (s_ok) return;
  const int chunks = a.row_bytes / 16;  // 16-byte chunks of one (row, KV head)
  const int items = len * a.hkv * chunks;
  for (int it = tid; it < items; it += kCommitThreads) {
    const int j = it / (a.hkv * chunks);
    const int rem = it % (a.hkv * chunks);
    const int g = rem / chunks, c = rem % chunks;
    const int t = p0 + j;
    const long src = (static_cast<long>(n0 + path[j]) * a.hkv + g) * a.row_bytes + c * 16;
    const long dst = ((static_cast<long>(bt[t / TV_BLOCK]) * a.hkv + g) * TV_BLOCK + t % TV_BLOCK) *
                         a.row_bytes + c * 16;
    const uint4 kv = *reinterpret_cast<const uint4*>(a.k_tree + src);
    const uint4 vv = *reinterpret_cast<const uint4*>(a.v_tree + src);
    *reinterpret_cast<uint4*>(a.k_cache + dst) = kv;
    *reinterpret_cast<uint4*>(a.v_cache + dst) = vv;
  }
  __syncthreads();
  if (tid == 0) a.prefix_len[b] = p0 + len;
}

}  // namespace

}  // namespace tv

extern "C" int tree_commit_kv(const void* k_tree, const void* v_tree, const int32_t* cu_nodes,
                              const int32_t* accept_len, const int32_t* path, int32_t batch,
                              int32_t total_nodes, int32_t max_path, int32_t hkv,
                              int32_t head_dim, int32_t dtype, void* k_cache, void* v_cache,
                              int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                              int32_t* prefix_len, int32_t* err, void* stream) {
  tv::clear_error();
  if (batch < 0 || total_nodes < 0 || max_path < 0 || num_blocks < 0 || max_blocks < 0)
    return tv::fail(TV_EINVAL, "tree_commit_kv: negative size");
  if (hkv <= 0) return tv::fail(TV_EINVAL, "tree_commit_kv: hkv must be positive");
  if (head_dim != 64 && head_dim != 128)
    return tv::fail(TV_EUNSUPPORTED, "tree_commit_kv: head_dim must be 64 or 128");
  if (dtype != TV_DTYPE_F32 && dtype != TV_DTYPE_BF16)
    return tv::fail(TV_EUNSUPPORTED, "tree_commit_kv: dtype must be F32 or BF16");
  if (err == nullptr) return tv::fail(TV_EINVAL, "tree_commit_kv: null err");
  if (max_path > tv::kMaxPath)
    return tv::fail(TV_EUNSUPPORTED, "tree_commit_kv: max_path must be at most 4096");
  if (batch == 0) return TV_OK;
  if (cu_nodes == nullptr || accept_len == nullptr || prefix_len == nullptr ||
      block_table == nullptr || k_cache == nullptr || v_cache == nullptr)
    return tv::fail(TV_EINVAL, "tree_commit_kv: null cu_nodes, accept_len, prefix_len, block "
                               "table or cache");
  if (max_path > 0 && path == nullptr) return tv::fail(TV_EINVAL, "tree_commit_kv: null path");
  if (total_nodes > 0 && (k_tree == nullptr || v_tree == nullptr))
    return tv::fail(TV_EINVAL, "tree_commit_kv: null tree K/V");
  tv::CommitArgs a{};
  a.k_tree = static_cast<const char*>(k_tree);
  a.v_tree = static_cast<const char*>(v_tree);
  a.cu_nodes = cu_nodes;
  a.accept_len = accept_len;
  a.path = path;
  a.k_cache = static_cast<char*>(k_cache);
  a.v_cache = static_cast<char*>(v_cache);
  a.block_table = block_table;
  a.prefix_len = prefix_len;
  a.err = err;
  a.max_path = max_path;
  a.hkv = hkv;
  a.row_bytes = head_dim * (dtype == TV_DTYPE_F32 ? 4 : 2);
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  a.batch = batch;
  auto s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(tv::k_commit_kv, dim3(batch), dim3(tv::kCommitThreads), 0, s, a);
  return tv::check_launch("tree_commit_kv");
}
