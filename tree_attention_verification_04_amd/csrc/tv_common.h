// Internal helpers shared by the HIP sources of the tree-verification library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "treeverify.h"

namespace tv {

// thread-local error message behind tree_last_error()
void set_error(const char* fmt, ...);
void clear_error();

inline int fail(int status, const char* msg) {
  set_error("%s", msg);
  return status;
}

inline int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return TV_EHIP;
  }
  return TV_OK;
}

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- device side

// Sequence that owns flattened node `node`: the b with cu[b] <= node < cu[b+1].
__device__ __forceinline__ int seq_of_node(const int32_t* __restrict__ cu, int batch, int node) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= node) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Streaming (non-temporal) stores for whole 16-byte pieces that no workgroup of the
// same launch reads back: they go out as the kernel runs instead of sitting dirty in
// the die's L2 until the write-back at the end of the launch.
typedef float stream_f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_stream4(float* p, float x, float y, float z, float w) {
  const stream_f32x4_t v = {x, y, z, w};
  __builtin_nontemporal_store(v, reinterpret_cast<stream_f32x4_t*>(p));
}
__device__ __forceinline__ void store_stream(float* p, float v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace tv
