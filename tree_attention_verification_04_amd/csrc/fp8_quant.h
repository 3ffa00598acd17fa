// E4M3 rows with power-of-two (E8M0) row scales: the scale rule shared by the row
// quantizer and the FP8 matrix-core attention (which quantizes Q in its own kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tv {

// s of the row scale 2^s: the smallest power of two with amax <= 448 * 2^s, in
// [-127, 127]; 0 for amax = 0.  With amax = m * 2^E (1 <= m < 2): s = E - 8, plus one
// when m > 1.75 (448 = 1.75 * 2^8); small and subnormal amax are clamped to -127.
__device__ __forceinline__ int e8m0_shift(float amax) {
  const uint32_t bits = __float_as_uint(amax);
  const int expo = static_cast<int>((bits >> 23) & 0xffu);
  const uint32_t mant = bits & 0x7fffffu;
  if (expo == 0) return mant == 0 ? 0 : -127;
  const int s = (expo - 127) - 8 + (mant > 0x600000u ? 1 : 0);
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// codes [rows][128] and exps [rows] from x [rows][128] (bf16 or fp32)
int launch_quant_rows(const void* x, int dtype, long rows, uint8_t* codes, uint8_t* exps,
                      hipStream_t stream);
// two row sets of the same size and dtype in one launch (x1 null: the first only)
int launch_quant_rows2(const void* x0, uint8_t* codes0, uint8_t* exps0, const void* x1,
                       uint8_t* codes1, uint8_t* exps1, int dtype, long rows, hipStream_t stream);

}  // namespace tv
