/*
 * treeverify.h — C ABI of the tree-verification step of speculative decoding
 * (one target-model pass over a whole draft tree), for AMD MI355X (gfx950).
 *
 * Sources, cited below by tag and section:
 *   [P500]   "端侧多模态大模型推测解码草稿模型动态剪枝：详解基于重要性采样的树形验证并行加速策略"
 *            https://www.ufo.work/2026/500.html
 *   [P525]   "端侧大模型推测解码草稿模型动态剪枝策略：详解基于重要性采样的树形验证并行加速机制"
 *            https://www.ufo.work/2026/525.html
 *   [P537]   "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力机制与显存碎片整理联合加速"
 *            https://www.ufo.work/2026/537.html
 *
 * The step has three calls, enqueued in order on one HIP stream:
 *   tree_build_index      parent array -> depth, ancestor-or-self bitsets
 *   tree_verify_attention every tree node attends to the shared paged prefix
 *                         and to its own ancestors (mask M_tree)
 *   tree_accept           ratio test, longest accepted path, residual resample
 * two variants of the second for an FP8 cache:
 *   tree_verify_attention_fp8kv   (E4M3 prefix with fp32 row scales, exact q)
 *   tree_verify_attention_fp8     (E4M3 Q, K, V with power-of-two row scales, FP8 matrix cores)
 * one that builds the tree before them:
 *   tree_draft_build      draft top-K rows -> parent array of the candidate tree
 * and a fourth that follows them:
 *   tree_commit_kv        the accepted path's K/V become prefix positions
 * and the probability rows before acceptance (the draft's restricted to its kept
 * set by the second):
 *   tree_softmax_rows, tree_softmax_rows_kept
 * and a counter-based generator of the acceptance uniforms:
 *   tree_uniforms         per-node uniforms from (seed, request, tree level, node, step)
 * The three calls of the step also come as one call and as a HIP graph:
 *   tree_verify_step, tree_verify_graph_create / _launch / _destroy
 *
 * Conventions shared by every call
 *   - Every array pointer is DEVICE memory owned by the caller; the library
 *     keeps no pointer after a call returns (a graph made by
 *     tree_verify_graph_create keeps those of its capture).  The library
 *     allocates no device memory: scratch comes from a caller-provided
 *     workspace whose size is returned by the matching *_workspace_size query
 *     (tree_accept_noalloc instead uses a fixed scratch array of the library,
 *     one per GPU; a graph handle is host memory plus the runtime's graph).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued on it; no call synchronises the device or the host.
 *     Buffers must stay alive until the stream has passed the call.
 *   - Return value: TV_OK, or a TV_E* status when a host-side check fails (no
 *     work is enqueued then); tree_last_error() gives the reason.
 *   - Data-dependent faults (a bad parent index, a token outside the
 *     vocabulary, ...) cannot be seen on the host without a sync.  Kernels OR
 *     TV_ERR_* bits into the caller's device word `*err`, which the caller
 *     zeroes before the first call and may read after the stream passes.
 *     Outputs are unspecified for the sequences concerned when a bit is set.
 *   - Trees are flattened: sequence b owns nodes cu_nodes[b] .. cu_nodes[b+1]-1
 *     (a [batch+1] prefix-sum array).  Node indices inside a tree ("local")
 *     run from 0; parent[i] is local, -1 meaning the node hangs directly off
 *     the prefix ([P537] appendix B: parent index per node, -1 for the root).
 *     Parents precede children (parent[i] < i); several nodes may hang off
 *     the prefix.  At most TV_MAX_NODES nodes per sequence.
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* host-side status codes */
#define TV_OK 0
#define TV_EINVAL 1          /* bad argument: null pointer, negative size, ... */
#define TV_EUNSUPPORTED 2    /* shape or dtype the kernels do not handle */
#define TV_EHIP 3            /* a HIP launch failed */
#define TV_EWORKSPACE 4      /* workspace missing or smaller than required */

/* device error bits OR-ed into *err */
#define TV_ERR_BAD_PARENT 1      /* parent[i] >= i or < -1 */
#define TV_ERR_TOO_MANY_NODES 2  /* a sequence holds more than max_nodes nodes */
#define TV_ERR_TOKEN 4           /* drafted token outside [0, vocab) */
#define TV_ERR_BLOCK 8           /* block id outside [0, num_blocks), or prefix longer than the
                                    block table / max_prefix */
#define TV_ERR_ZERO_MASS 16      /* residual and target mass both zero at the rejection node */
#define TV_ERR_PATH 32           /* accepted path longer than max_path */
#define TV_ERR_UNIFORM 64        /* a uniform outside [0, 1) or NaN */
#define TV_ERR_ROW 128           /* a context-row index outside [0, ctx_rows) */
#define TV_ERR_DRAFT 256         /* a draft probability outside [0, 1] or NaN */

/* element types */
#define TV_DTYPE_F32 0
#define TV_DTYPE_BF16 1

#define TV_MAX_NODES 2048    /* nodes per sequence (page [P525] appendix: 2048-slot KV pool) */
#define TV_BLOCK 64          /* tokens per paged KV block ([P525] §2.3.1: 64/128-token blocks) */

/*
 * tree_build_index — per-node depth and ancestor-or-self bitset.
 *
 * Defines the mask of [P537] §2.2.2 (equation M_tree): node i may see node j
 * iff j is i or an ancestor of i.  Instead of a dense N x N mask, node i gets
 * `words` 64-bit words; bit (j % 64) of word (j / 64) is set iff j is visible
 * to i.  depth[i] is 1 for a node under the prefix and grows by one per edge;
 * the optional pos[i] = prefix_len[b] + depth[i] - 1 is the node's position
 * id ([P500] §9.1, static tree position tensor).
 *
 *   parent      [total_nodes] int32, local parent index (-1 = under the prefix)
 *   cu_nodes    [batch + 1] int32
 *   max_nodes   upper bound on any sequence's node count, 1..TV_MAX_NODES
 *   prefix_len  [batch] int32 or NULL (then pos is not written)
 *   anc_bits    out [total_nodes, words] uint64; words >= ceil(max_nodes / 64)
 *   depth       out [total_nodes] int32
 *   pos         out [total_nodes] int32 or NULL
 *   err         in/out device word, see above (TV_ERR_BAD_PARENT, TV_ERR_TOO_MANY_NODES)
 */
int tree_build_index(const int32_t* parent, const int32_t* cu_nodes, int32_t batch,
                     int32_t total_nodes, int32_t max_nodes, const int32_t* prefix_len,
                     uint64_t* anc_bits, int32_t words, int32_t* depth, int32_t* pos,
                     int32_t* err, void* stream);

/*
 * tree_verify_attention — one attention layer over every draft-tree node.
 *
 * For sequence b, local node n and query head h (KV head g = h / (hq / hkv)):
 *   visible keys = prefix positions t < prefix_len[b]  (the prefix is stored
 *                  once and shared by every branch, [P500] §3.2; read through
 *                  the paged block table, [P525] §2.3.1)
 *                + tree nodes j with bit j set in anc_bits[n] ([P537] §2.2.2)
 *   out[n, h]    = softmax_j(softmax_scale * <q[n,h], k_j[g]>) . v_j[g]
 *   lse[n, h]    = log sum_j exp(softmax_scale * <q[n,h], k_j[g]>)   (natural log)
 * Accumulation is fp32; bf16 probabilities feed the P.V product
 * ([P537] appendix B; §5.1 mixed-precision accumulation).
 *
 *   q            [total_nodes, hq, head_dim], dtype
 *   k_cache/v_cache [num_blocks, hkv, TV_BLOCK, head_dim], dtype: paged prefix
 *   block_table  [batch, max_blocks] int32: physical block of logical block j
 *                (only entries j < ceil(prefix_len[b] / 64) are read; tables
 *                may alias the same physical blocks)
 *   prefix_len   [batch] int32, each <= max_prefix and <= max_blocks * 64
 *   k_tree/v_tree [total_nodes, hkv, head_dim], dtype: keys/values of the nodes
 *   cu_nodes     [batch + 1] int32; anc_bits [total_nodes, words] from tree_build_index
 *   max_nodes, max_prefix  host-side upper bounds that size the launch
 *   hq % hkv == 0; head_dim 64 or 128; dtype TV_DTYPE_F32 or TV_DTYPE_BF16
 *   out          [total_nodes, hq, head_dim], dtype
 *   lse          [total_nodes, hq] float or NULL
 *   workspace    device scratch of >= tree_verify_attention_workspace_size(...) bytes
 *                (may be NULL when that size is 0).  Zero-fill it once before its
 *                first use: its first 2048 bytes hold counters (finish tickets of
 *                work items whose partial results are merged inside the kernel,
 *                queue heads of a launch that schedules its own work items), and
 *                every call leaves them zero again.  Calls that share one
 *                workspace must not overlap.
 *   err          TV_ERR_BLOCK, TV_ERR_TOO_MANY_NODES
 */
size_t tree_verify_attention_workspace_size(int32_t batch, int32_t total_nodes, int32_t max_nodes,
                                            int32_t max_prefix, int32_t hq, int32_t hkv,
                                            int32_t head_dim, int32_t dtype);

int tree_verify_attention(const void* q, const void* k_cache, const void* v_cache,
                          int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                          const int32_t* prefix_len, const void* k_tree, const void* v_tree,
                          const int32_t* cu_nodes, const uint64_t* anc_bits, int32_t words,
                          int32_t batch, int32_t total_nodes, int32_t max_nodes,
                          int32_t max_prefix, int32_t hq, int32_t hkv, int32_t head_dim,
                          int32_t dtype, float softmax_scale, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, int32_t* err, void* stream);

/*
 * tree_verify_attention_fp8kv — tree_verify_attention over an FP8 prefix cache.
 *
 * The paged cache holds OCP E4M3 bytes (4 exponent bits with bias 7, 3 mantissa
 * bits, no infinities, 0x7F/0xFF NaN) with one fp32 scale per block of 128
 * elements, i.e. per (cache block, KV head, position) row of head_dim 128; the
 * value of element d of a row is e4m3(byte) * scale ([P537] §9.2: Q, K, V in FP8
 * E4M3 with block scaling, one scale per 128 elements, fp32 accumulators;
 * appendix B: block scales beside K and V, applied when a block is loaded).  Only
 * the streamed prefix is FP8: q, the tree K/V and out are bf16, head_dim is 128,
 * and the result is tree_verify_attention's on the dequantized cache.  Each
 * dequantized element is rounded once to bf16 before the matrix cores use it.
 *
 *   k_cache/v_cache [num_blocks, hkv, 64, 128] uint8 (E4M3)
 *   k_scale/v_scale [num_blocks, hkv, 64] float (may be NULL when max_prefix == 0)
 *   everything else as for tree_verify_attention with head_dim 128 and dtype
 *   TV_DTYPE_BF16; workspace >= tree_verify_attention_fp8kv_workspace_size(...)
 */
size_t tree_verify_attention_fp8kv_workspace_size(int32_t batch, int32_t total_nodes,
                                                  int32_t max_nodes, int32_t max_prefix,
                                                  int32_t hq, int32_t hkv);

int tree_verify_attention_fp8kv(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                const float* k_scale, const float* v_scale, int32_t num_blocks,
                                const int32_t* block_table, int32_t max_blocks,
                                const int32_t* prefix_len, const void* k_tree, const void* v_tree,
                                const int32_t* cu_nodes, const uint64_t* anc_bits, int32_t words,
                                int32_t batch, int32_t total_nodes, int32_t max_nodes,
                                int32_t max_prefix, int32_t hq, int32_t hkv, float softmax_scale,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                int32_t* err, void* stream);

/*
 * tree_quantize_rows_e4m3 — rows of 128 elements to OCP E4M3 codes with one
 * power-of-two scale per row ([P537] §9.2: Q, K, V in FP8 E4M3 with one scale per
 * 128 elements), the format tree_verify_attention_fp8 reads.
 *
 * Row i with amax = max |x[i][:]| gets the smallest power of two 2^s with
 * amax <= 448 * 2^s (s in [-127, 127]; s = 0 for an all-zero row), stored as the
 * E8M0 byte exps[i] = s + 127; codes[i][d] = round-to-nearest-even E4M3 of
 * x[i][d] * 2^-s (exact product; the sign of zero is kept).  Dequantized value:
 * e4m3(code) * 2^(exps - 127).
 *
 *   x      [rows, 128] dtype (TV_DTYPE_BF16 or TV_DTYPE_F32), 16-byte aligned
 *   codes  out [rows, 128] uint8; exps out [rows] uint8
 */
int tree_quantize_rows_e4m3(const void* x, int32_t dtype, int64_t rows, uint8_t* codes,
                            uint8_t* exps, void* stream);

/*
 * tree_verify_attention_fp8 — tree attention on the FP8 matrix cores: Q, K and V in
 * OCP E4M3 with one power-of-two scale per 128-element row ([P537] §9.2: Q, K, V
 * in FP8 E4M3 with block scaling, one scale per 128 elements, fp32 accumulation).
 *
 * K and V, of the paged prefix and of the tree alike, arrive as E4M3 codes with one
 * E8M0 exponent byte per row (value = e4m3(code) * 2^(e - 127), as
 * tree_quantize_rows_e4m3 writes it: the forward pass that writes the FP8 cache
 * writes the tree's rows the same way).  q arrives in bf16 and is quantized by the
 * same rule inside the call.  The scores Q.K run on the scaled FP8 matrix
 * instructions (the row exponents applied by the hardware); V is converted exactly
 * to bf16 and P.V runs in bf16 as in tree_verify_attention.  The result is
 * tree_verify_attention's on the dequantized Q, K and V (within its bf16 tolerance).
 *
 *   k_cache/v_cache [num_blocks, hkv, 64, 128] uint8 (E4M3)
 *   k_exp/v_exp     [num_blocks, hkv, 64] uint8 (E8M0; may be NULL when max_prefix == 0)
 *   k_tree/v_tree   [total_nodes, hkv, 128] uint8 (E4M3)
 *   kt_exp/vt_exp   [total_nodes, hkv] uint8 (E8M0)
 *   everything else as for tree_verify_attention with head_dim 128, bf16 q and out;
 *   workspace >= tree_verify_attention_fp8_workspace_size(...), zero-filled before its
 *   first use as there
 */
size_t tree_verify_attention_fp8_workspace_size(int32_t batch, int32_t total_nodes,
                                                int32_t max_nodes, int32_t max_prefix, int32_t hq,
                                                int32_t hkv);

int tree_verify_attention_fp8(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                              const uint8_t* k_exp, const uint8_t* v_exp, int32_t num_blocks,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* prefix_len, const uint8_t* k_tree,
                              const uint8_t* v_tree, const uint8_t* kt_exp, const uint8_t* vt_exp,
                              const int32_t* cu_nodes, const uint64_t* anc_bits, int32_t words,
                              int32_t batch, int32_t total_nodes, int32_t max_nodes,
                              int32_t max_prefix, int32_t hq, int32_t hkv, float softmax_scale,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              int32_t* err, void* stream);

/*
 * tree_draft_build — the candidate tree of each sequence from the draft model's
 * top-K rows, before the step: importance-sampled expansion ([P500] §3.1: weights
 * w = p^beta / sum p^beta over a context's top-K, branches kept and deepened by
 * sampling on w) after a cumulative-mass soft truncation ([P525] §2.1.2: in
 * descending order, keep candidates until their mass reaches 1 - prune_ratio,
 * renormalise the kept ones by that mass).
 *
 * Per sequence: row 0 of probs is the context at the end of the prefix, row i+1
 * the context after node i.  A context's kept candidates (the shortest leading
 * run of slots whose fp64 mass reaches 1 - prune_ratio) get path weight = parent's
 * path weight * p^beta / (sum over the kept slots of p^beta).  Node i is drawn
 * from all candidates not yet taken with probability proportional to path weight:
 * the first candidate, in creation order, whose running sum exceeds
 * u[i] * (sum of all); if its depth < max_depth and row i+1 exists, its kept
 * children become candidates.  Building stops at n_max nodes or when no
 * candidate has weight.  The decision arithmetic is fp64; a draw whose
 * threshold falls within rounding of a running-sum boundary may resolve either
 * way (the sums are chunked across a wavefront).
 *
 *   probs     [batch, rows, k] float, each row non-increasing, values in [0, 1]
 *   u         [batch, n_max] float in [0, 1)
 *   k <= 16, n_max <= 256, max_depth in [1, 256], beta >= 0, prune_ratio in [0, 1]
 *   parent    out [batch, n_max] int32: local parent (-1 = the prefix), -2 past count
 *   slot      out [batch, n_max] int32: the top-K slot of the node's token, -2 past count
 *   q_draft   out [batch, n_max] float: p / kept mass of its context (the draft
 *             probability the acceptance test must use for the node), 0 past count
 *   count     out [batch] int32: nodes built (parents precede children, so
 *             parent[b][0 .. count-1] is a valid tree_build_index input)
 *   err       TV_ERR_DRAFT (a probability outside [0, 1]), TV_ERR_UNIFORM; such a
 *             sequence builds nothing
 */
int tree_draft_build(const float* probs, const float* u, int32_t batch, int32_t rows, int32_t k,
                     int32_t n_max, int32_t max_depth, float beta, float prune_ratio,
                     int32_t* parent, int32_t* slot, float* q_draft, int32_t* count, int32_t* err,
                     void* stream);

/*
 * tree_uniforms — the acceptance and resample uniforms of every node from a
 * counter-based generator ([P537] §8.2: every rank draws the same numbers for a
 * node because they come from a stateless generator whose input is built from
 * the request, the tree level, the node index and the step; nothing is broadcast,
 * and a restarted request draws the same numbers).
 *
 * Generator: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11).  For local node j
 * of sequence b: counter = (j, (uint32) depth[j], step, (uint64) request_id[b]),
 * key = (seed, purpose); word 0 of the output block gives u_accept, word 1
 * u_resample, each = (word >> 40) * 2^-24, exact in fp32, in [0, 1 - 2^-24].
 * The values depend only on these inputs, not on the batch layout.
 *
 *   seed, purpose  key words (purpose separates independent draw families of a step)
 *   step           decoding step
 *   request_id     [batch] int64: the request that sequence b serves
 *   depth          [total_nodes] int32, tree_build_index's output
 *   cu_nodes       [batch + 1] int32
 *   u_accept, u_resample  out [total_nodes] float; either may be NULL (not written)
 * One thread per node; no workspace, no error bits.
 */
int tree_uniforms(uint64_t seed, uint64_t purpose, uint64_t step, const int64_t* request_id,
                  const int32_t* depth, const int32_t* cu_nodes, int32_t batch,
                  int32_t total_nodes, float* u_accept, float* u_resample, void* stream);

/*
 * tree_accept — fused acceptance for every sequence, one launch, no host
 * round-trip ([P537] §2.2.3: per-node p_accept = min(1, p_target / p_draft), one
 * uniform per node, depth-first walk from the root cut at the first rejected
 * node, longest accepted path, sampling fused with the traversal; [P525] §1.2:
 * resample at the rejection point).
 *
 * Per sequence:
 *   accept bit   u_accept[i] < min(1, pt_i[tok_i] / pd_i[tok_i]), evaluated
 *                exactly as (double)u * (double)pd < (double)pt
 *   node_ok[i]   1 iff i and all its ancestors pass
 *   winner w     the passing node of largest depth, ties to the smallest index
 *                (none: w = -1)
 *   accept_len   depth(w), 0 if none; path[0 .. accept_len-1] = the root-level
 *                ancestor of w down to w (local ids), the rest -1
 *   rejection    c = smallest-index child of w (w = -1: smallest-index node
 *                under the prefix)
 *   resample     token drawn from norm(max(0, pt_c - pd_c)), or from pt_c when
 *                that has no mass, by an integer inverse CDF: q_k =
 *                floor(((double)pt - (double)pd) * 2^40) for positive
 *                differences, Z = sum q_k, T = floor(u_resample[c] * Z)
 *                (exact), token = smallest k with q_0 + .. + q_k > T.
 *                Integer sums make the token independent of summation order.
 *   bonus        when w has no child (the whole path to a leaf passed) and
 *                own_row[w] >= 0: token drawn from p_own[own_row[w]] (p_target at
 *                w's own context: the one forward pass over the tree gives it,
 *                [P537] §2.2.3) with u_resample[w], same integer inverse CDF on
 *                q_k = floor((double)p_own_k * 2^40); resample_node = w.  Without
 *                own_row (NULL), or own_row[w] = -1, nothing: -1 outputs.
 *
 *   p_target/p_draft [total_nodes, vocab] float: row i = the two distributions
 *                that judged node i's drafted token (those at its parent's context)
 *   token        [total_nodes] int32; u_accept/u_resample [total_nodes] float in [0, 1)
 *   parent, cu_nodes as for tree_build_index; max_nodes <= TV_MAX_NODES
 *   p_own        [own_rows, vocab] float or NULL: target rows at nodes' own contexts
 *   own_row      [total_nodes] int32 or NULL: row of p_own at node i's own context,
 *                -1 = none (only the winner's entry is read)
 *   accept_len   out [batch] int32; path out [batch, max_path] int32
 *   resample_node out [batch] int32: c (residual), w (bonus) or -1
 *   resample_token out [batch] int32 (-1 = none)
 *   node_ok      out [total_nodes] uint8 or NULL
 *   workspace    vocab <= 65536: unused (may be NULL); larger vocabularies: at least
 *                tree_accept_workspace_size(batch, vocab) bytes, zero-filled before its
 *                first use (every call leaves its ticket words zero again); calls that
 *                share one workspace must not overlap on the device
 *   err          TV_ERR_BAD_PARENT, TV_ERR_TOO_MANY_NODES, TV_ERR_TOKEN, TV_ERR_ZERO_MASS,
 *                TV_ERR_PATH, TV_ERR_UNIFORM, TV_ERR_ROW (own_row[w] outside
 *                [-1, own_rows): no bonus)
 */
size_t tree_accept_workspace_size(int32_t batch, int32_t vocab);

int tree_accept(const float* p_target, const float* p_draft, const int32_t* token,
                const float* u_accept, const float* u_resample, const int32_t* parent,
                const int32_t* cu_nodes, const float* p_own, const int32_t* own_row,
                int32_t own_rows, int32_t batch, int32_t total_nodes, int32_t max_nodes,
                int32_t vocab, int32_t max_path, int32_t* accept_len, int32_t* path,
                int32_t* resample_node, int32_t* resample_token, uint8_t* node_ok,
                void* workspace, size_t workspace_bytes, int32_t* err, void* stream);

/*
 * tree_accept_noalloc — tree_accept for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, outputs, launch and errors as tree_accept, minus
 * the workspace: the chunked launch (vocab > 65536) keeps its ticket words and
 * chunk sums in a fixed scratch array of this library, one copy per GPU (1 MiB +
 * 128 KiB, held until the process ends; its device address is looked up once per
 * device and its ticket words cleared then).  Nothing is allocated per call.
 *
 *   limits       vocab > 65536 needs batch <= 1024 (else TV_EUNSUPPORTED, nothing
 *                launched); smaller vocabularies use no scratch and have no limit
 *   concurrency  every call on one GPU shares that GPU's scratch: calls that can
 *                overlap on the device (different streams, or graphs replayed
 *                concurrently) race and must be serialised by the caller
 */
int tree_accept_noalloc(const float* p_target, const float* p_draft, const int32_t* token,
                        const float* u_accept, const float* u_resample, const int32_t* parent,
                        const int32_t* cu_nodes, const float* p_own, const int32_t* own_row,
                        int32_t own_rows, int32_t batch, int32_t total_nodes, int32_t max_nodes,
                        int32_t vocab, int32_t max_path, int32_t* accept_len, int32_t* path,
                        int32_t* resample_node, int32_t* resample_token, uint8_t* node_ok,
                        int32_t* err, void* stream);

/*
 * tree_commit_kv — append each sequence's accepted path to its paged prefix.
 *
 * Node path[b][j] (local id, j < accept_len[b]) holds the keys and values of
 * position prefix_len[b] + j: its rows of every KV head are copied to that
 * position of the paged cache, and prefix_len[b] grows by accept_len[b], so the
 * next verify round reads them as shared prefix ([P537] §5.2, prefix caching of
 * the accepted path; [P525] §2.3.2, the tree's KV slots return to the pool after
 * verification; [P525] §8.1, accepted length and new KV indices as verify outputs).
 * The block table must already map the logical blocks of the new positions (the
 * caller reserves them; nothing is allocated here), and those blocks must belong
 * to this sequence alone: prefix blocks may be shared between sequences for
 * reading ([P537] §2.3.3, shared prefix pool), but a block that another
 * sequence's table row also maps is not written (a shared prefix whose length is
 * not a multiple of 64 ends inside such a block; copying it first is the
 * caller's job).
 *
 *   k_tree/v_tree   [total_nodes, hkv, head_dim], dtype (must not overlap the cache)
 *   cu_nodes        [batch + 1] int32
 *   accept_len      [batch] int32; path [batch, max_path] int32 (tree_accept's outputs)
 *   k_cache/v_cache [num_blocks, hkv, TV_BLOCK, head_dim], dtype: written
 *   block_table     [batch, max_blocks] int32
 *   prefix_len      [batch] int32: read, then increased in place
 *   head_dim 64 or 128; dtype TV_DTYPE_F32 or TV_DTYPE_BF16
 *   max_path        at most 4096 (else TV_EUNSUPPORTED)
 *   err             TV_ERR_PATH (accept_len outside [0, max_path], or a path entry
 *                   outside the sequence's nodes), TV_ERR_BLOCK (a new position beyond
 *                   the table, mapped to a block outside [0, num_blocks), or mapped to a
 *                   block that another sequence's table row also holds); such a
 *                   sequence is left untouched (cache and prefix_len)
 */
int tree_commit_kv(const void* k_tree, const void* v_tree, const int32_t* cu_nodes,
                   const int32_t* accept_len, const int32_t* path, int32_t batch,
                   int32_t total_nodes, int32_t max_path, int32_t hkv, int32_t head_dim,
                   int32_t dtype, void* k_cache, void* v_cache, int32_t num_blocks,
                   const int32_t* block_table, int32_t max_blocks, int32_t* prefix_len,
                   int32_t* err, void* stream);

/*
 * tree_softmax_rows — probability rows from target logits, before tree_accept.
 *
 * One forward pass over the tree gives one logits row per context ([P537] §2.2.3);
 * a drafted token is judged by the distribution at its parent's context, so
 * siblings share a row:
 *   probs[i][k] = exp(t*logits[r][k] - M_r) / sum_k' exp(t*logits[r][k'] - M_r),
 *   r = row_of[i] (or i when row_of is NULL), M_r = max_k t*logits[r][k]
 * (the maximum subtracted first: [P525] §7.1, log-sum-exp trick).  Computed in
 * fp32: relative error of each probability below 5e-6.
 *
 *   logits      [ctx_rows, vocab] float
 *   row_of      [rows] int32 or NULL (then rows == ctx_rows)
 *   inv_temperature  t > 0 (1 = plain softmax)
 *   probs       out [rows, vocab] float; a row whose row_of entry is outside
 *               [0, ctx_rows) is zero-filled and sets TV_ERR_ROW
 *   workspace   >= tree_softmax_rows_workspace_size(ctx_rows, vocab) bytes; no
 *               initial contents needed; calls sharing one must not overlap
 * HBM-bound.  With at least 256 output rows, a vocabulary that is a multiple of 4
 * in [90112, 155136] and 16-byte aligned logits and probs, one kernel holds each
 * context row on one compute unit and reads it once (the workspace is then not
 * touched); otherwise two kernels read it twice.  rows and vocab / 8192 at most
 * 65535.
 */
size_t tree_softmax_rows_workspace_size(int32_t ctx_rows, int32_t vocab);

int tree_softmax_rows(const float* logits, int32_t ctx_rows, int32_t vocab, const int32_t* row_of,
                      int32_t rows, float inv_temperature, float* probs, void* workspace,
                      size_t workspace_bytes, int32_t* err, void* stream);

/*
 * tree_softmax_rows_kept — probability rows restricted to a kept set of tokens.
 *
 * Pruning the draft keeps a set R of candidates per context, so the drafted tokens
 * come from q~(x) = q(x) * 1[x in R] / Z, Z the mass of R under q ([P525] §2.2.1);
 * acceptance must divide by q~, not q.  [P525] §2.2.2 writes it as an edit of the
 * logits before the softmax (log(1/Z) added on R, minus infinity elsewhere); the
 * constant cancels, so a kept row is the softmax over R alone:
 *   probs[i][k] = exp(t*logits[r][k] - M_R) / sum_{k' in R} exp(t*logits[r][k'] - M_R)
 *   for k in R = the ids in keep[r], 0 elsewhere; r = row_of[i] (or i), M_R the
 *   maximum of t*logits[r] over R.
 * Meant for the draft's rows (p_draft of tree_accept); the target's rows stay the
 * plain softmax of tree_softmax_rows.  fp32, relative error below 5e-6.
 *
 *   logits      [ctx_rows, vocab] float
 *   keep        [ctx_rows, keep_max] int32: context row r's kept token ids; -1 is
 *               padding and a repeated id counts once; keep_max in [1, 256]
 *               (else TV_EUNSUPPORTED)
 *   row_of      [rows] int32 or NULL (then rows == ctx_rows)
 *   inv_temperature  t > 0
 *   probs       out [rows, vocab] float.  The row is zero and a bit set when its
 *               row_of entry is outside [0, ctx_rows) (TV_ERR_ROW), an id is
 *               outside [-1, vocab) (TV_ERR_TOKEN) or the set is empty
 *               (TV_ERR_ZERO_MASS)
 * One kernel, one workgroup per output row; writes the whole row (HBM-bound on
 * vocab * 4 bytes a row); no workspace.
 */
int tree_softmax_rows_kept(const float* logits, int32_t ctx_rows, int32_t vocab,
                           const int32_t* keep, int32_t keep_max, const int32_t* row_of,
                           int32_t rows, float inv_temperature, float* probs, int32_t* err,
                           void* stream);

/*
 * tree_verify_step — the step's three calls in one: tree_build_index, then
 * tree_verify_attention, then tree_accept, enqueued in that order on `stream`
 * with the arguments below (each field means what the same-named argument of
 * those calls means; anc_bits/words/depth link the first to the other two).
 * Returns the first non-TV_OK status of the three; the calls before the
 * failing one are then already enqueued.
 *
 * tree_verify_graph_create — captures the same three calls once into a HIP
 * graph (a stream capture; [ViSpec] §3.2: the whole verification flow is
 * captured in a graph so that no host code runs between its kernels) and
 * instantiates it.  The graph holds the pointers and sizes of `args` as they are
 * at capture: every replay reads and writes those same buffers, so the caller
 * refreshes the inputs in place between replays.  `stream` (NULL: a temporary
 * stream of the library) is used for the capture only; nothing executes.  The
 * handle and the runtime's graph objects are the only allocations (host side, and
 * whatever the HIP runtime needs for an executable graph).
 * tree_verify_graph_launch — replays the graph on `stream` (any stream of the
 * same device); replays of one graph, or of graphs sharing a workspace, must not
 * overlap on the device.
 * tree_verify_graph_destroy — releases the handle (NULL is ignored); the caller
 * makes sure no replay is still running.
 */
typedef struct tree_verify_step_args {
  /* tree_build_index */
  const int32_t* parent;
  const int32_t* cu_nodes;
  int32_t batch;
  int32_t total_nodes;
  int32_t max_nodes;
  int32_t words;
  const int32_t* prefix_len;
  uint64_t* anc_bits;
  int32_t* depth;
  int32_t* pos; /* may be NULL */
  /* tree_verify_attention */
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t max_prefix;
  int32_t hq;
  int32_t hkv;
  int32_t head_dim;
  int32_t dtype;
  float softmax_scale;
  const void* k_tree;
  const void* v_tree;
  void* out;
  float* lse; /* may be NULL */
  void* attn_workspace;
  size_t attn_workspace_bytes;
  /* tree_accept */
  const float* p_target;
  const float* p_draft;
  const int32_t* token;
  const float* u_accept;
  const float* u_resample;
  const float* p_own;      /* may be NULL */
  const int32_t* own_row;  /* may be NULL */
  int32_t own_rows;
  int32_t vocab;
  int32_t max_path;
  int32_t reserved; /* 0 */
  int32_t* accept_len;
  int32_t* path;
  int32_t* resample_node;
  int32_t* resample_token;
  uint8_t* node_ok; /* may be NULL */
  void* accept_workspace;
  size_t accept_workspace_bytes;
  /* all three */
  int32_t* err;
} tree_verify_step_args;

typedef struct tree_verify_graph tree_verify_graph; /* opaque */

/* sizeof(tree_verify_step_args) as compiled into the library (a binding checks it) */
size_t tree_verify_step_args_size(void);

int tree_verify_step(const tree_verify_step_args* args, void* stream);

int tree_verify_graph_create(const tree_verify_step_args* args, void* stream,
                             tree_verify_graph** graph);

int tree_verify_graph_launch(tree_verify_graph* graph, void* stream);

int tree_verify_graph_destroy(tree_verify_graph* graph);

/* Reason for the last non-TV_OK status on the calling thread ("" if none). */
const char* tree_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TREEVERIFY_H */
