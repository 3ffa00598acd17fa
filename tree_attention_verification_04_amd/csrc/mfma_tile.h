// Shared pieces of the matrix-core tree-attention kernels: operand types, the
// swizzled LDS layout of a K/V tile, global -> register -> LDS staging of a tile.
#pragma once

#include "attn.h"

namespace tv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kD = 128;
constexpr int kKT = 64;                           // keys per tile
constexpr int kTileBytes = kKT * kD * 2;          // 16 KB per K (or V) tile
constexpr int kStageBytes = 2 * kTileBytes;       // K then V
constexpr int kAncBytes = kMfmaRowsPerWG * 8;     // ancestor words of the rows, per stage
constexpr int kAncOff = 3 * kStageBytes;
constexpr int kSmemBytes = 3 * kStageBytes + 3 * kAncBytes + 64;  // three stages + scalars
constexpr int kChunks = kKT * kD * 2 / 16;        // 16-byte chunks per tile (1024)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// MFMA row m of a 32-key sub-tile reads key perm(m): swaps 4-row groups 1<->2, 5<->6.
__device__ __forceinline__ int key_perm(int m) {
  const int grp = m >> 2;
  const int swapped = (grp & 3) == 1 ? grp + 1 : ((grp & 3) == 2 ? grp - 1 : grp);
  return (swapped << 2) | (m & 3);
}

// byte offset of (key, 16-byte chunk c) inside a K tile / a V tile
__device__ __forceinline__ int k_off(int key, int c) { return key * 256 + ((c ^ (key & 15)) << 4); }
__device__ __forceinline__ int v_off(int key, int c) { return key * 256 + ((c ^ ((key & 3) << 2)) << 4); }

struct TileSrc {
  const uint16_t* k;    // first row of the tile
  const uint16_t* v;
  long row_stride;      // 16-bit units between consecutive keys
  int nvalid;           // rows [0, nvalid) exist; later rows are zero-filled
  const uint64_t* anc;  // ancestor word of this thread's row for the tile (tree tiles)
  const float* ks;      // FP8 tile: per-key scales of K and V (null: a bf16 tile)
  const float* vs;
};

template <int THREADS>
struct TileRegsT {
  uint4 k[kChunks / THREADS];  // bf16 chunks; an FP8 tile holds its bytes in k[0] / v[0]
  uint4 v[kChunks / THREADS];  // and the K / V scales of this thread's key in k[1].x / v[1].x
  uint64_t anc;
  bool f8;
};

// Rows at or past nvalid are read from row nvalid - 1 (always inside the source
// array) and zeroed when the tile is written to LDS, so the loads need no branch.
// An FP8 tile (kFp8 and src.ks set) has 128-byte rows: thread t loads bytes
// 16 (t % 8) .. + 15 of row t / 8, and its K and V scales.
template <int THREADS, bool kFp8 = false>
__device__ __forceinline__ void load_tile_t(const TileSrc& src, int tid, TileRegsT<THREADS>& r) {
  r.f8 = kFp8 && src.ks != nullptr;
  if (kFp8 && src.ks != nullptr) {
    static_assert(!kFp8 || THREADS == 512, "FP8 tiles are staged by 512 threads");
    const int key = min(tid >> 3, max(src.nvalid - 1, 0)), c8 = tid & 7;
    const long off = key * src.row_stride + c8 * 8;
    r.k[0] = *reinterpret_cast<const uint4*>(src.k + off);
    r.v[0] = *reinterpret_cast<const uint4*>(src.v + off);
    r.k[1].x = __float_as_uint(src.ks[key]);
    r.v[1].x = __float_as_uint(src.vs[key]);
  } else {
#pragma unroll
    for (int i = 0; i < kChunks / THREADS; ++i) {
      const int ci = tid + THREADS * i;
      const int key = min(ci >> 4, max(src.nvalid - 1, 0)), c = ci & 15;
      const long off = key * src.row_stride + c * 8;
      r.k[i] = *reinterpret_cast<const uint4*>(src.k + off);
      r.v[i] = *reinterpret_cast<const uint4*>(src.v + off);
    }
  }
  r.anc = *src.anc;
}

// Eight E4M3 bytes (two dwords, byte order) times a scale, as eight bf16 (round to
// nearest even); the products are exact in fp32 before that rounding.
__device__ __forceinline__ uint4 fp8x8_to_bf16(uint32_t w0, uint32_t w1, float scale) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
  const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false), d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
  return make_uint4(pack2_bf16(a.x * scale, a.y * scale), pack2_bf16(b.x * scale, b.y * scale),
                    pack2_bf16(c.x * scale, c.y * scale), pack2_bf16(d.x * scale, d.y * scale));
}

// The ancestor words of the workgroup's 256 rows go to a small LDS slot per stage.
// An FP8 tile is dequantized here (byte * scale, rounded to bf16), so LDS always
// holds the bf16 layout.
template <int THREADS, bool kFp8 = false>
__device__ __forceinline__ void store_tile_t(char* stage, uint64_t* anc_slot, int tid,
                                             TileRegsT<THREADS>& r, int nvalid) {
  if (tid < kMfmaRowsPerWG) anc_slot[tid] = r.anc;
  if (kFp8 && r.f8) {
    const int key = tid >> 3, c8 = tid & 7;
    const float sk = __uint_as_float(r.k[1].x), sv = __uint_as_float(r.v[1].x);
    uint4 k0 = fp8x8_to_bf16(r.k[0].x, r.k[0].y, sk), k1 = fp8x8_to_bf16(r.k[0].z, r.k[0].w, sk);
    uint4 v0 = fp8x8_to_bf16(r.v[0].x, r.v[0].y, sv), v1 = fp8x8_to_bf16(r.v[0].z, r.v[0].w, sv);
    if (nvalid < kKT && key >= nvalid) k0 = k1 = v0 = v1 = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(stage + k_off(key, 2 * c8)) = k0;
    *reinterpret_cast<uint4*>(stage + k_off(key, 2 * c8 + 1)) = k1;
    *reinterpret_cast<uint4*>(stage + kTileBytes + v_off(key, 2 * c8)) = v0;
    *reinterpret_cast<uint4*>(stage + kTileBytes + v_off(key, 2 * c8 + 1)) = v1;
    return;
  }
#pragma unroll
  for (int i = 0; i < kChunks / THREADS; ++i) {
    const int ci = tid + THREADS * i;
    const int key = ci >> 4, c = ci & 15;
    if (nvalid < kKT && key >= nvalid) {  // nvalid is uniform: the branch is rare
      r.k[i] = make_uint4(0, 0, 0, 0);
      r.v[i] = make_uint4(0, 0, 0, 0);
    }
    *reinterpret_cast<uint4*>(stage + k_off(key, c)) = r.k[i];
    *reinterpret_cast<uint4*>(stage + kTileBytes + v_off(key, c)) = r.v[i];
  }
}

typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

// LDS transpose read of 4 bf16 (p points into the workgroup's LDS)
__device__ __forceinline__ bf16x4_t ds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

}  // namespace tv
