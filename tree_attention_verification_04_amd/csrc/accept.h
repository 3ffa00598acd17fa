// Internal interface between the acceptance entry points and their kernel.
#pragma once

#include "tv_common.h"

namespace tv {

// Above this vocabulary the launch is chunked and uses the workspace.
constexpr int kAcceptFusedVocab = 65536;

// Bytes of the finish-ticket words at the start of the workspace (one 128-byte line
// per sequence, rounded up to 256 bytes).
size_t accept_ticket_bytes(int batch);

// Argument checks and the one acceptance launch shared by tree_accept and
// tree_accept_noalloc (workspace: the ticket words and chunk sums of the chunked
// launch, see tree_accept_workspace_size).
int accept_launch(const char* fn, const float* p_target, const float* p_draft,
                  const int32_t* token, const float* u_accept, const float* u_resample,
                  const int32_t* parent, const int32_t* cu_nodes, const float* p_own,
                  const int32_t* own_row, int32_t own_rows, int32_t batch, int32_t total_nodes,
                  int32_t max_nodes, int32_t vocab, int32_t max_path, int32_t* accept_len,
                  int32_t* path, int32_t* resample_node, int32_t* resample_token,
                  uint8_t* node_ok, void* workspace, size_t workspace_bytes, int32_t* err,
                  void* stream);

}  // namespace tv
