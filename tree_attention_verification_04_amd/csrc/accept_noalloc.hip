// tree_accept_noalloc: tree_accept for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The scratch the chunked acceptance launch needs (ticket words and
// per-chunk sums) lives in a fixed device array of this library, one copy per GPU,
// held until the process ends; nothing is allocated per call.
#include <mutex>

#include "accept.h"

namespace tv {

namespace {

// Largest scratch one call may use: tickets for 1024 sequences (a 128-byte line each,
// 128 KiB) plus their chunk sums at the largest vocabulary (1024 x 64 chunks x 16 B =
// 1 MiB).
constexpr int kMaxSequences = 1024;
constexpr size_t kTicketBytes = size_t{kMaxSequences} * 128;
constexpr size_t kScratchBytes = kTicketBytes + (size_t{1} << 20);
constexpr int kMaxDevices = 64;

// Zero when the code object is loaded; every call leaves its ticket words zero again.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each GPU, once looked up

__global__ void k_zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The device address of this GPU's scratch array (looked up once per device, with
// that device current, and its ticket words cleared then), or null with the status
// in *status.
void* scratch_for_current_device(hipStream_t s, int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = fail(TV_EHIP, "tree_accept_noalloc: no current device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      set_error("tree_accept_noalloc: hipGetSymbolAddress failed: %s", hipGetErrorString(e));
      *status = TV_EHIP;
      return nullptr;
    }
    // the first 128 KiB hold the ticket words: clear them once, by a kernel (not a
    // memset node) so that a call under graph capture stays valid
    constexpr int kWords = static_cast<int>(kTicketBytes / 4);
    hipLaunchKernelGGL(k_zero_words, dim3(kWords / 256), dim3(256), 0, s,
                       static_cast<uint32_t*>(ptr), kWords);
    const int st = check_launch("tree_accept_noalloc/clear");
    if (st != TV_OK) {
      *status = st;
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  *status = TV_OK;
  return g_scratch[dev];
}

}  // namespace

}  // namespace tv

extern "C" int tree_accept_noalloc(const float* p_target, const float* p_draft,
                                   const int32_t* token, const float* u_accept,
                                   const float* u_resample, const int32_t* parent,
                                   const int32_t* cu_nodes, const float* p_own,
                                   const int32_t* own_row, int32_t own_rows, int32_t batch,
                                   int32_t total_nodes, int32_t max_nodes, int32_t vocab,
                                   int32_t max_path, int32_t* accept_len, int32_t* path,
                                   int32_t* resample_node, int32_t* resample_token,
                                   uint8_t* node_ok, int32_t* err, void* stream) {
  tv::clear_error();
  const size_t need = tree_accept_workspace_size(batch, vocab);
  if (vocab > tv::kAcceptFusedVocab &&
      (need > tv::kScratchBytes || batch > tv::kMaxSequences ||
       tv::accept_ticket_bytes(batch) > tv::kTicketBytes))
    return tv::fail(TV_EUNSUPPORTED,
                    "tree_accept_noalloc: batch x vocabulary chunks exceed the fixed scratch "
                    "(at most 1024 sequences; 1 MiB of chunk sums)");
  int status = TV_OK;
  void* ws = nullptr;
  if (batch > 0 && vocab > 0) {
    ws = tv::scratch_for_current_device(static_cast<hipStream_t>(stream), &status);
    if (ws == nullptr) return status;
  }
  return tv::accept_launch("tree_accept_noalloc", p_target, p_draft, token, u_accept, u_resample,
                           parent, cu_nodes, p_own, own_row, own_rows, batch, total_nodes,
                           max_nodes, vocab, max_path, accept_len, path, resample_node,
                           resample_token, node_ok, ws, tv::kScratchBytes, err, stream);
}
