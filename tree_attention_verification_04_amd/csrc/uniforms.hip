// Counter-based uniforms for the acceptance draws.
//
// Page "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力机制与显存碎片整理联合加速"
// (ufo.work/2026/537), §8.2: all ranks must draw identical numbers for a tree node, so
// the draws come from a counter-based generator whose input is built from the request,
// the tree level, the node index and the step, with no state and nothing broadcast.
//
// Generator: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11).  Counter of local node j of sequence b = (j, depth[j] as
// 32-bit unsigned, step, request_id[b]); key = (seed, purpose).  Output word 0 gives
// the node's acceptance uniform, word 1 its resample uniform, each as its top 24 bits
// times 2^-24 (exact in fp32, in [0, 1 - 2^-24]).  One thread per node; the 64x64-bit
// products are split by the compiler into 32-bit multiplies.
#include "tv_common.h"

namespace tv {
namespace {

// round multipliers and key (Weyl) increments of Philox4x64
constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;
constexpr int kUniformThreads = 256;

__global__ void __launch_bounds__(kUniformThreads)
    k_uniforms(uint64_t seed, uint64_t purpose, uint64_t step, const int64_t* __restrict__ request_id,
               const int32_t* __restrict__ depth, const int32_t* __restrict__ cu_nodes, int batch,
               int total, float* __restrict__ u_accept, float* __restrict__ u_resample) {
  const int n = blockIdx.x * kUniformThreads + threadIdx.x;
  if (n >= total) return;
  const int b = seq_of_node(cu_nodes, batch, n);
  uint64_t c0 = static_cast<uint64_t>(static_cast<int64_t>(n) - cu_nodes[b]);
  uint64_t c1 = static_cast<uint32_t>(depth[n]);
  uint64_t c2 = step;
  uint64_t c3 = static_cast<uint64_t>(request_id[b]);
  uint64_t k0 = seed, k1 = purpose;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t hi0 = __umul64hi(kPhiloxM0, c0), lo0 = kPhiloxM0 * c0;
    const uint64_t hi1 = __umul64hi(kPhiloxM1, c2), lo1 = kPhiloxM1 * c2;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  if (u_accept != nullptr) u_accept[n] = static_cast<float>(static_cast<uint32_t>(c0 >> 40)) * 0x1p-24f;
  if (u_resample != nullptr)
    u_resample[n] = static_cast<float>(static_cast<uint32_t>(c1 >> 40)) * 0x1p-24f;
}

}  // namespace
}  // namespace tv

extern "C" int tree_uniforms(uint64_t seed, uint64_t purpose, uint64_t step,
                             const int64_t* request_id, const int32_t* depth,
                             const int32_t* cu_nodes, int32_t batch, int32_t total_nodes,
                             float* u_accept, float* u_resample, void* stream) {
  tv::clear_error();
  if (batch < 0 || total_nodes < 0) return tv::fail(TV_EINVAL, "tree_uniforms: negative size");
  if (total_nodes == 0) return TV_OK;
  if (batch == 0) return tv::fail(TV_EINVAL, "tree_uniforms: nodes without sequences");
  if (request_id == nullptr || depth == nullptr || cu_nodes == nullptr)
    return tv::fail(TV_EINVAL, "tree_uniforms: null request_id, depth or cu_nodes");
  if (u_accept == nullptr && u_resample == nullptr) return TV_OK;
  const int blocks = tv::ceil_div(total_nodes, tv::kUniformThreads);
  hipLaunchKernelGGL(tv::k_uniforms, dim3(blocks), dim3(tv::kUniformThreads), 0,
                     static_cast<hipStream_t>(stream), seed, purpose, step, request_id, depth,
                     cu_nodes, batch, total_nodes, u_accept, u_resample);
  return tv::check_launch("tree_uniforms");
}
