// tree_verify_attention: argument checks and launch plan.
//
// The plan picks the kernel (matrix-core for bf16 head_dim 128, vector ALU
// otherwise) and, for the matrix-core kernel, how many workgroups share one
// (sequence, KV head) prefix.  When one row tile per KV head cannot fill the
// 256 compute units (a single short verify), the prefix blocks are split over
// several workgroups and a second kernel merges the partial results by
// log-sum-exp, the same rescaling the online softmax applies between tiles (page
// "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力机制与显存碎片整理联合加速"
// (ufo.work/2026/537), appendix B).
#include <algorithm>
#include <cstdio>

#include "attn.h"

namespace tv {

AttnPlan plan_attention(int batch, int total_nodes, int max_nodes, int max_prefix, int hq, int hkv,
                        int head_dim, int dtype, int kv_format) {
  AttnPlan p{};
  p.mfma = dtype == TV_DTYPE_BF16 && head_dim == 128;
  p.splits = 1;
  p.blocks_per_split = 0;
  p.row_tiles = 0;
  p.total_work = 0;
  p.tail_pieces = 1;
  p.persistent = false;
  p.merge_in_kernel = false;
  p.die_slots = 0;
  p.workspace = 0;
  if (!p.mfma || batch <= 0 || hkv <= 0) return p;
  const int group = hq / hkv;
  const int nblk = ceil_div(std::max(0, max_prefix), 64);
  p.row_tiles = std::max(1, ceil_div(group * max_nodes, kMfmaRowsPerWG));
  const long base = static_cast<long>(batch) * hkv * p.row_tiles;
  // one 512-thread workgroup fits a compute unit (LDS): split the prefix so that a
  // short verify still spreads over the CUs, without a second round of workgroups,
  // but keep enough blocks per split for the tile pipeline to hide memory latency
  if (nblk > kMinSplitBlocks && 2 * base <= kCUs) {
    const int want = std::min<long>(std::min(nblk, kMaxSplits), kCUs / base);
    p.blocks_per_split = std::max(kMinSplitBlocks, ceil_div(nblk, want));
    p.splits = ceil_div(nblk, p.blocks_per_split);
  } else {
    p.blocks_per_split = std::max(1, nblk);
    p.splits = 1;
  }
  p.total_work = base * p.splits;
  // (an FP8 prefix cache goes through the pipelined kernel's register path for long
  // items, through the register-staged kernel for short ones)
  // (the FP8 matrix-core format exists in the pipelined kernel only)
  p.long_items = p.blocks_per_split + ceil_div(max_nodes, 64) >= kLongMinTiles ||
                 kv_format == kKvMma8;
  // more long work items than compute units, from sequences of different lengths:
  // rank the (sequence, KV head) pairs by cost and start the longest first
  const long pairs = static_cast<long>(batch) * hkv;
  p.ordered = p.long_items && batch > 1 && p.total_work > kCUs && pairs <= kMaxOrderedPairs;
  // Long items over more than one round run persistently: one workgroup per compute
  // unit pulls its die's items from a queue head (then other dies' items), so that a
  // die whose units are all busy does not hold up the dispatch of the others (the
  // hardware hands workgroups to dies in launch order).  Each die's queue holds its
  // pairs' items, pair-major; per die, die_slots queue slots.
  p.tail_pieces = 1;
  p.tail_whole = 0;
  p.tail_items = 0;
  // (the pipelined kernel deals pairs to dies, pair r to die r % 8; the staged
  // kernel deals each die a contiguous range of work indices)
  const long per_die =
      p.long_items ? ceil_div(static_cast<int>(pairs), kXCDs) * static_cast<long>(p.row_tiles) *
                         p.splits
                   : (p.total_work + kXCDs - 1) / kXCDs;
  p.die_slots = per_die <= INT32_MAX / kMaxTailPieces ? static_cast<int>(per_die) : 0;
  p.persistent = p.die_slots > kCUsPerXCD;
  // tail balancing: when a die's items do not fill its last round evenly, the items
  // of that round are cut into prefix pieces, so the last round ends sooner
  if (p.persistent && p.long_items && p.splits == 1) {
    const int tail = p.die_slots % kCUsPerXCD;
    const int k = tail_pieces_for(tail, kCUsPerXCD);
    if (k > 1) {
      p.tail_pieces = k;
      p.tail_items = tail;
      p.tail_whole = p.die_slots - tail;
      p.die_slots = p.tail_whole + tail * k;
    }
  }
  if (p.persistent && p.long_items && pairs <= kMaxOrderedPairs) p.ordered = true;
  // Workspace: [counter words, kCounterBytes] [partial outputs] [partial lse] [pair
  // order].  The counter words are zero between calls: every call that uses them
  // (tickets of the in-kernel split merge, queue heads of a persistent launch)
  // leaves them zero again, so the caller zero-fills a new workspace once.
  size_t prow = 0;  // partial rows
  if (p.splits > 1) prow = static_cast<size_t>(p.splits) * total_nodes * hq;
  if (p.tail_pieces > 1)
    prow = static_cast<size_t>(kXCDs) * p.tail_items * p.tail_pieces * kMfmaRowsPerWG;
  p.merge_in_kernel = p.tail_pieces > 1;  // at most 8 * 31 tickets (< kMaxTickets)
  // every plan with a workspace keeps the counter words first, whether it uses them
  size_t ws = prow > 0 || p.persistent || p.ordered ? kCounterBytes : 0;
  p.part_off = ws;
  if (prow > 0) {
    p.lse_off = (p.part_off + prow * head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
    ws = p.lse_off + prow * sizeof(float);
  }
  if (p.ordered) {
    p.order_off = (ws + 255) & ~static_cast<size_t>(255);
    ws = p.order_off + static_cast<size_t>(pairs) * sizeof(int);
  }
  p.workspace = ws;
  return p;
}

// The last round holds `tail` items on `cus` units.  Cut into k pieces each, it
// takes ceil(tail * k / cus) rounds of 1/k of an item; every cut piece also
// writes and re-reads a partial result, charged as 2% of an item.
int tail_pieces_for(int tail, int cus) {
  if (tail <= 0 || cus <= 0) return 1;
  int best_k = 1;
  float best = 1.0f;
  for (int k = 2; k <= kMaxTailPieces; ++k) {
    const float t = static_cast<float>(ceil_div(tail * k, cus)) / k + 0.02f * (k - 1);
    if (t < best - 1e-6f) {
      best = t;
      best_k = k;
    }
  }
  return best_k;
}

}  // namespace tv

extern "C" size_t tree_verify_attention_workspace_size(int32_t batch, int32_t total_nodes,
                                                       int32_t max_nodes, int32_t max_prefix,
                                                       int32_t hq, int32_t hkv, int32_t head_dim,
                                                       int32_t dtype) {
  if (hkv <= 0 || hq <= 0 || hq % hkv != 0) return 0;
  return tv::plan_attention(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, dtype,
                            tv::kKvBf16)
      .workspace;
}

extern "C" size_t tree_verify_attention_fp8kv_workspace_size(int32_t batch, int32_t total_nodes,
                                                             int32_t max_nodes, int32_t max_prefix,
                                                             int32_t hq, int32_t hkv) {
  if (hkv <= 0 || hq <= 0 || hq % hkv != 0) return 0;
  return tv::plan_attention(batch, total_nodes, max_nodes, max_prefix, hq, hkv, 128,
                            TV_DTYPE_BF16, tv::kKvFp8)
      .workspace;
}

extern "C" size_t tree_verify_attention_fp8_workspace_size(int32_t batch, int32_t total_nodes,
                                                           int32_t max_nodes, int32_t max_prefix,
                                                           int32_t hq, int32_t hkv) {
  if (hkv <= 0 || hq <= 0 || hq % hkv != 0) return 0;
  return tv::plan_attention(batch, total_nodes, max_nodes, max_prefix, hq, hkv, 128,
                            TV_DTYPE_BF16, tv::kKvMma8)
      .workspace;
}

namespace {

// Shared body of the bf16/fp32 and the two FP8-cache entry points (kv_format: the
// cache has the dtype of q; E4M3 with fp32 row scales; E4M3 with E8M0 row exponents).
int verify_attention(const char* fn, int kv_format, const void* q, const void* k_cache,
                     const void* v_cache, const float* k_scale, const float* v_scale,
                     const uint8_t* k_exp, const uint8_t* v_exp, const uint8_t* kt_exp,
                     const uint8_t* vt_exp, int32_t num_blocks,
                     const int32_t* block_table, int32_t max_blocks, const int32_t* prefix_len,
                     const void* k_tree, const void* v_tree, const int32_t* cu_nodes,
                     const uint64_t* anc_bits, int32_t words, int32_t batch, int32_t total_nodes,
                     int32_t max_nodes, int32_t max_prefix, int32_t hq, int32_t hkv,
                     int32_t head_dim, int32_t dtype, float softmax_scale, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, int32_t* err, void* stream) {
  char msg[160];
  auto bad = [&](int status, const char* what) {
    snprintf(msg, sizeof(msg), "%s: %s", fn, what);
    return tv::fail(status, msg);
  };
  if (batch < 0 || total_nodes < 0 || max_prefix < 0 || num_blocks < 0 || max_blocks < 0)
    return bad(TV_EINVAL, "negative size");
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
    return bad(TV_EINVAL, "hq must be a positive multiple of hkv");
  if (head_dim != 64 && head_dim != 128) return bad(TV_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (dtype != TV_DTYPE_F32 && dtype != TV_DTYPE_BF16)
    return bad(TV_EUNSUPPORTED, "dtype must be F32 or BF16");
  if (max_nodes < 1 || max_nodes > TV_MAX_NODES)
    return bad(TV_EUNSUPPORTED, "max_nodes must be in [1, 2048]");
  if (words < tv::ceil_div(max_nodes, 64)) return bad(TV_EINVAL, "words < ceil(max_nodes / 64)");
  if (!(softmax_scale > 0.0f) || softmax_scale == INFINITY)
    return bad(TV_EINVAL, "softmax_scale must be positive and finite");
  if (err == nullptr || cu_nodes == nullptr) return bad(TV_EINVAL, "null err or cu_nodes");
  if (batch == 0 || total_nodes == 0) return TV_OK;
  if (q == nullptr || k_tree == nullptr || v_tree == nullptr || anc_bits == nullptr ||
      out == nullptr || prefix_len == nullptr)
    return bad(TV_EINVAL, "null q, tree K/V, anc_bits, out or prefix_len");
  if (max_prefix > 0 && (k_cache == nullptr || v_cache == nullptr || block_table == nullptr))
    return bad(TV_EINVAL, "null paged cache or block table");
  if (max_prefix > 0 && kv_format == tv::kKvFp8 && (k_scale == nullptr || v_scale == nullptr))
    return bad(TV_EINVAL, "null cache scales");
  if (max_prefix > 0 && kv_format == tv::kKvMma8 && (k_exp == nullptr || v_exp == nullptr))
    return bad(TV_EINVAL, "null cache exponents");
  if (kv_format == tv::kKvMma8 && (kt_exp == nullptr || vt_exp == nullptr))
    return bad(TV_EINVAL, "null tree exponents");
  if (kv_format == tv::kKvMma8) {  // rows are loaded in 16-byte chunks
    auto misaligned = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 != 0; };
    if (misaligned(k_tree) || misaligned(v_tree) ||
        (max_prefix > 0 && (misaligned(k_cache) || misaligned(v_cache))))
      return bad(TV_EINVAL, "E4M3 arrays must be 16-byte aligned");
  }
  if (max_prefix > 0 && num_blocks < 1)
    return bad(TV_EINVAL, "max_prefix > 0 needs num_blocks >= 1");
  if (static_cast<long>(max_blocks) * 64 < max_prefix)
    return bad(TV_EINVAL, "max_prefix exceeds max_blocks * 64");
  if (static_cast<long>(total_nodes) * hq > INT32_MAX)
    return bad(TV_EUNSUPPORTED, "too many (node, head) rows");

  const tv::AttnPlan plan =
      tv::plan_attention(batch, total_nodes, max_nodes, max_prefix, hq, hkv, head_dim, dtype,
                         kv_format);
  if (plan.workspace > 0 && (workspace == nullptr || workspace_bytes < plan.workspace))
    return bad(TV_EWORKSPACE, "workspace missing or too small");

  tv::AttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.prefix_len = prefix_len;
  a.k_tree = k_tree;
  a.v_tree = v_tree;
  a.cu_nodes = cu_nodes;
  a.anc = anc_bits;
  if (kv_format == tv::kKvFp8) {  // the kernel choice keys on a non-null scale pointer
    a.k_scale = k_scale;
    a.v_scale = v_scale;
  }
  a.out = out;
  a.lse = lse;
  a.err = err;
  a.words = words;
  a.batch = batch;
  a.total_nodes = total_nodes;
  a.total_rows = total_nodes * hq;
  a.max_nodes = max_nodes;
  a.max_prefix = max_prefix;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  a.hq = hq;
  a.hkv = hkv;
  a.group = hq / hkv;
  a.scale = softmax_scale;
  a.splits = plan.splits;
  a.blocks_per_split = plan.blocks_per_split;
  a.row_tiles = plan.row_tiles;
  a.total_work = static_cast<int>(plan.total_work);
  a.tail_pieces = plan.tail_pieces;
  a.tail_whole = plan.tail_whole;
  a.tail_items = plan.tail_items;
  a.die_slots = plan.die_slots;
  char* wsb = static_cast<char*>(workspace);
  if (plan.splits > 1 || plan.tail_pieces > 1) {
    a.part_o = reinterpret_cast<float*>(wsb + plan.part_off);
    a.part_lse = reinterpret_cast<float*>(wsb + plan.lse_off);
  }
  if (plan.persistent) a.queue = reinterpret_cast<int*>(wsb) + tv::kQueueWord;
  if (plan.merge_in_kernel) a.tickets = reinterpret_cast<int*>(wsb) + tv::kTicketWord;
  auto s = static_cast<hipStream_t>(stream);
  if (kv_format == tv::kKvMma8) {  // the kernel keys on kt8
    a.k_exp = k_exp;
    a.v_exp = v_exp;
    a.kt8 = static_cast<const uint8_t*>(k_tree);
    a.vt8 = static_cast<const uint8_t*>(v_tree);
    a.kt_e = kt_exp;
    a.vt_e = vt_exp;
  }
  if (!plan.mfma) return tv::launch_attn_vec(a, head_dim, dtype, s);
  if (plan.ordered) {
    int* order = reinterpret_cast<int*>(static_cast<char*>(workspace) + plan.order_off);
    const int st = tv::launch_attn_order(a, order, s);
    if (st != TV_OK) return st;
    a.pair_order = order;
  }
  return plan.long_items ? tv::launch_attn_long(a, s) : tv::launch_attn_mfma(a, s);
}

}  // namespace

extern "C" int tree_verify_attention(const void* q, const void* k_cache, const void* v_cache,
                                     int32_t num_blocks, const int32_t* block_table,
                                     int32_t max_blocks, const int32_t* prefix_len,
                                     const void* k_tree, const void* v_tree,
                                     const int32_t* cu_nodes, const uint64_t* anc_bits,
                                     int32_t words, int32_t batch, int32_t total_nodes,
                                     int32_t max_nodes, int32_t max_prefix, int32_t hq,
                                     int32_t hkv, int32_t head_dim, int32_t dtype,
                                     float softmax_scale, void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, int32_t* err, void* stream) {
  tv::clear_error();
  return verify_attention("tree_verify_attention", tv::kKvBf16, q, k_cache, v_cache, nullptr,
                          nullptr, nullptr, nullptr, nullptr, nullptr, num_blocks, block_table, max_blocks, prefix_len, k_tree, v_tree,
                          cu_nodes, anc_bits, words, batch, total_nodes, max_nodes, max_prefix, hq,
                          hkv, head_dim, dtype, softmax_scale, out, lse, workspace,
                          workspace_bytes, err, stream);
}

extern "C" int tree_verify_attention_fp8kv(
    const void* q, const uint8_t* k_cache, const uint8_t* v_cache, const float* k_scale,
    const float* v_scale, int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
    const int32_t* prefix_len, const void* k_tree, const void* v_tree, const int32_t* cu_nodes,
    const uint64_t* anc_bits, int32_t words, int32_t batch, int32_t total_nodes,
    int32_t max_nodes, int32_t max_prefix, int32_t hq, int32_t hkv, float softmax_scale,
    void* out, float* lse, void* workspace, size_t workspace_bytes, int32_t* err, void* stream) {
  tv::clear_error();
  return verify_attention("tree_verify_attention_fp8kv", tv::kKvFp8, q, k_cache, v_cache, k_scale,
                          v_scale, nullptr, nullptr, nullptr, nullptr, num_blocks, block_table,
                          max_blocks, prefix_len, k_tree, v_tree, cu_nodes, anc_bits, words, batch,
                          total_nodes, max_nodes, max_prefix, hq, hkv, 128, TV_DTYPE_BF16,
                          softmax_scale, out, lse, workspace, workspace_bytes, err, stream);
}

extern "C" int tree_verify_attention_fp8(
    const void* q, const uint8_t* k_cache, const uint8_t* v_cache, const uint8_t* k_exp,
    const uint8_t* v_exp, int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
    const int32_t* prefix_len, const uint8_t* k_tree, const uint8_t* v_tree, const uint8_t* kt_exp,
    const uint8_t* vt_exp, const int32_t* cu_nodes, const uint64_t* anc_bits, int32_t words,
    int32_t batch, int32_t total_nodes, int32_t max_nodes, int32_t max_prefix, int32_t hq,
    int32_t hkv, float softmax_scale, void* out, float* lse, void* workspace,
    size_t workspace_bytes, int32_t* err, void* stream) {
  tv::clear_error();
  return verify_attention("tree_verify_attention_fp8", tv::kKvMma8, q, k_cache, v_cache, nullptr,
                          nullptr, k_exp, v_exp, kt_exp, vt_exp, num_blocks, block_table,
                          max_blocks, prefix_len, k_tree, v_tree, cu_nodes, anc_bits, words, batch,
                          total_nodes, max_nodes, max_prefix, hq, hkv, 128, TV_DTYPE_BF16,
                          softmax_scale, out, lse, workspace, workspace_bytes, err, stream);
}
