// Rows of 128 elements -> OCP E4M3 codes with one power-of-two scale per row, stored
// as an E8M0 byte (value 2^(e - 127)).
//
// Page "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力机制与显存碎片整理联合加速"
// (ufo.work/2026/537), §9.2: Q, K and V in FP8 E4M3 with one scale per block of 128
// elements.  The scale of a row is the smallest power of two 2^s with
// max|x| <= 448 * 2^s (s in [-127, 127]; 0 for an all-zero row), so the codes are the
// round-to-nearest-even E4M3 values of x * 2^-s, which the scaled FP8 matrix
// instructions take back with the exponent byte at no cost.
//
// 16 threads per row, 8 elements each; the row maximum by a 16-lane butterfly.
#include "fp8_quant.h"
#include "tv_common.h"

namespace tv {
namespace {

constexpr int kQuantThreads = 256;

// Two row sets in one launch (blockIdx.y selects x / codes / exps of set 0 or 1).
struct QuantSets {
  const void* x[2];
  uint8_t* codes[2];
  uint8_t* exps[2];
};

template <bool kBf16>
__global__ void __launch_bounds__(kQuantThreads)
    k_quant_rows(QuantSets sets, long rows) {
  const void* __restrict__ x = sets.x[blockIdx.y];
  uint8_t* __restrict__ codes = sets.codes[blockIdx.y];
  uint8_t* __restrict__ exps = sets.exps[blockIdx.y];
  const long t = static_cast<long>(blockIdx.x) * kQuantThreads + threadIdx.x;
  const long row = t >> 4;
  const int part = static_cast<int>(t & 15);
  const bool live = row < rows;
  const long r = live ? row : rows - 1;  // dead lanes of the last block repeat a row
  float v[8];
  if constexpr (kBf16) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + r * 128 + 8 * part);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(ww[j] << 16);
      v[2 * j + 1] = __uint_as_float(ww[j] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + r * 128 + 8 * part);
    const float4 a = p[0], b = p[1];
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
  const int s = e8m0_shift(amax);
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], -s), ldexpf(v[1], -s), lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], -s), ldexpf(v[3], -s), lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4], -s), ldexpf(v[5], -s), hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[6], -s), ldexpf(v[7], -s), hi, true);
  if (live) {
    *reinterpret_cast<uint2*>(codes + row * 128 + 8 * part) = make_uint2(lo, hi);
    if (part == 0) exps[row] = static_cast<uint8_t>(s + 127);
  }
}

}  // namespace

int launch_quant_rows(const void* x, int dtype, long rows, uint8_t* codes, uint8_t* exps,
                      hipStream_t stream) {
  return launch_quant_rows2(x, codes, exps, nullptr, nullptr, nullptr, dtype, rows, stream);
}

int launch_quant_rows2(const void* x0, uint8_t* codes0, uint8_t* exps0, const void* x1,
                       uint8_t* codes1, uint8_t* exps1, int dtype, long rows, hipStream_t stream) {
  if (rows <= 0) return TV_OK;
  const long threads = rows * 16;
  const long blocks = (threads + kQuantThreads - 1) / kQuantThreads;
  if (blocks > 0x7fffffffL) return fail(TV_EUNSUPPORTED, "quantize: too many rows");
  const QuantSets sets{{x0, x1}, {codes0, codes1}, {exps0, exps1}};
  const dim3 grid(static_cast<unsigned>(blocks), x1 != nullptr ? 2 : 1);
  if (dtype == TV_DTYPE_BF16)
    hipLaunchKernelGGL(k_quant_rows<true>, grid, dim3(kQuantThreads), 0, stream, sets, rows);
  else
    hipLaunchKernelGGL(k_quant_rows<false>, grid, dim3(kQuantThreads), 0, stream, sets, rows);
  return check_launch("quantize rows");
}

}  // namespace tv

extern "C" int tree_quantize_rows_e4m3(const void* x, int32_t dtype, int64_t rows, uint8_t* codes,
                                       uint8_t* exps, void* stream) {
  tv::clear_error();
  if (rows < 0) return tv::fail(TV_EINVAL, "tree_quantize_rows_e4m3: negative rows");
  if (dtype != TV_DTYPE_F32 && dtype != TV_DTYPE_BF16)
    return tv::fail(TV_EUNSUPPORTED, "tree_quantize_rows_e4m3: dtype must be F32 or BF16");
  if (rows == 0) return TV_OK;
  if (x == nullptr || codes == nullptr || exps == nullptr)
    return tv::fail(TV_EINVAL, "tree_quantize_rows_e4m3: null x, codes or exps");
  return tv::launch_quant_rows(x, dtype, rows, codes, exps, static_cast<hipStream_t>(stream));
}
