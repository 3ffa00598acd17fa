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
  long row_stride;      // elements between consecutive keys
  int nvalid;           // rows [0, nvalid) exist; later rows are zero-filled
  const uint64_t* anc;  // ancestor word of this thread's row for the tile (tree tiles)
};

template <int THREADS>
struct TileRegsT {
  uint4 k[kChunks / THREADS];
  uint4 v[kChunks / THREADS];
  uint64_t anc;
};

// Rows at or past nvalid are read from row nvalid - 1 (always inside the source
// array) and zeroed when the tile is written to LDS, so the loads need no branch.
template <int THREADS>
__device__ __forceinline__ void load_tile_t(const TileSrc& src, int tid, TileRegsT<THREADS>& r) {
#pragma unroll
  for (int i = 0; i < kChunks / THREADS; ++i) {
    const int ci = tid + THREADS * i;
    const int key = min(ci >> 4, max(src.nvalid - 1, 0)), c = ci & 15;
    const long off = key * src.row_stride + c * 8;
    r.k[i] = *reinterpret_cast<const uint4*>(src.k + off);
    r.v[i] = *reinterpret_cast<const uint4*>(src.v + off);
  }
  r.anc = *src.anc;
}

// The ancestor words of the workgroup's 256 rows go to a small LDS slot per stage.
template <int THREADS>
__device__ __forceinline__ void store_tile_t(char* stage, uint64_t* anc_slot, int tid,
                                             TileRegsT<THREADS>& r, int nvalid) {
  if (tid < kMfmaRowsPerWG) anc_slot[tid] = r.anc;
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
