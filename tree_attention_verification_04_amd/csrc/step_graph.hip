// The verify step as one call, and as a HIP graph captured once and replayed.
//
// Page "视觉语言模型加速：ViSpec框架与推测解码优化", §3.2: the verification flow is
// captured whole in a graph, so no interpreter or host code runs between its
// kernels.  Here the flow is the step's three calls (tree index, tree attention,
// acceptance); the graph replays them on buffers fixed at capture, which the
// caller refreshes in place.  None of the three enqueues a memset or a copy (their
// counter words reset themselves), so the graph holds kernel nodes only.
#include <new>

#include "attn.h"
#include "tv_common.h"

struct tree_verify_graph {
  hipGraphExec_t exec;
  int device;
};

extern "C" size_t tree_verify_step_args_size(void) { return sizeof(tree_verify_step_args); }

extern "C" int tree_verify_step(const tree_verify_step_args* a, void* stream) {
  tv::clear_error();
  if (a == nullptr) return tv::fail(TV_EINVAL, "tree_verify_step: null args");
  int st = tree_build_index(a->parent, a->cu_nodes, a->batch, a->total_nodes, a->max_nodes,
                            a->prefix_len, a->anc_bits, a->words, a->depth, a->pos, a->err, stream);
  if (st != TV_OK) return st;
  st = tree_verify_attention(a->q, a->k_cache, a->v_cache, a->num_blocks, a->block_table,
                             a->max_blocks, a->prefix_len, a->k_tree, a->v_tree, a->cu_nodes,
                             a->anc_bits, a->words, a->batch, a->total_nodes, a->max_nodes,
                             a->max_prefix, a->hq, a->hkv, a->head_dim, a->dtype, a->softmax_scale,
                             a->out, a->lse, a->attn_workspace, a->attn_workspace_bytes, a->err,
                             stream);
  if (st != TV_OK) return st;
  return tree_accept(a->p_target, a->p_draft, a->token, a->u_accept, a->u_resample, a->parent,
                     a->cu_nodes, a->p_own, a->own_row, a->own_rows, a->batch, a->total_nodes,
                     a->max_nodes, a->vocab, a->max_path, a->accept_len, a->path,
                     a->resample_node, a->resample_token, a->node_ok, a->accept_workspace,
                     a->accept_workspace_bytes, a->err, stream);
}

extern "C" int tree_verify_graph_create(const tree_verify_step_args* a, void* stream,
                                        tree_verify_graph** graph) {
  tv::clear_error();
  if (a == nullptr || graph == nullptr)
    return tv::fail(TV_EINVAL, "tree_verify_graph_create: null args or graph");
  *graph = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return tv::fail(TV_EHIP, "tree_verify_graph_create: no device");
  // kernel attributes are not stream work: set them before the capture
  tv::set_attn_mfma_attributes();
  tv::set_attn_long_attributes();
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool own_stream = s == nullptr;  // the null stream cannot be captured
  if (own_stream && hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess)
    return tv::fail(TV_EHIP, "tree_verify_graph_create: stream creation failed");
  auto release_stream = [&]() {
    if (own_stream) (void)hipStreamDestroy(s);
  };
  hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    release_stream();
    tv::set_error("tree_verify_graph_create: capture failed to start: %s", hipGetErrorString(e));
    return TV_EHIP;
  }
  const int st = tree_verify_step(a, s);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(s, &g);  // always ended, also after a failed call
  if (st != TV_OK || e != hipSuccess || g == nullptr) {
    if (g != nullptr) (void)hipGraphDestroy(g);
    release_stream();
    if (st != TV_OK) return st;  // the failing call's reason stays in tree_last_error
    tv::set_error("tree_verify_graph_create: capture failed: %s", hipGetErrorString(e));
    return TV_EHIP;
  }
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  release_stream();
  if (e != hipSuccess) {
    tv::set_error("tree_verify_graph_create: instantiation failed: %s", hipGetErrorString(e));
    return TV_EHIP;
  }
  tree_verify_graph* h = new (std::nothrow) tree_verify_graph{exec, dev};
  if (h == nullptr) {
    (void)hipGraphExecDestroy(exec);
    return tv::fail(TV_EINVAL, "tree_verify_graph_create: out of host memory");
  }
  *graph = h;
  return TV_OK;
}

extern "C" int tree_verify_graph_launch(tree_verify_graph* graph, void* stream) {
  tv::clear_error();
  if (graph == nullptr) return tv::fail(TV_EINVAL, "tree_verify_graph_launch: null graph");
  const hipError_t e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    tv::set_error("tree_verify_graph_launch: %s", hipGetErrorString(e));
    return TV_EHIP;
  }
  return TV_OK;
}

extern "C" int tree_verify_graph_destroy(tree_verify_graph* graph) {
  tv::clear_error();
  if (graph == nullptr) return TV_OK;
  const hipError_t e = hipGraphExecDestroy(graph->exec);
  delete graph;
  if (e != hipSuccess) {
    tv::set_error("tree_verify_graph_destroy: %s", hipGetErrorString(e));
    return TV_EHIP;
  }
  return TV_OK;
}
