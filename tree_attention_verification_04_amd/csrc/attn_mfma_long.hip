// Matrix-core tree attention for gfx950, pipelined for long work items (many 64-key
// tiles per workgroup).
//
// Same computation and operand layout as k_attn_mfma (scores transposed, S^T = K Q^T;
// O^T = V^T P^T with V read through the LDS transpose read; online softmax; tree mask
// M_tree of page "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力机制与显存碎片
// 整理联合加速" (ufo.work/2026/537), §2.2.2 and appendix B).  A workgroup owns 256 rows;
// each wavefront owns G groups of 32 rows (G = 1: 8 wavefronts, two per SIMD; G = 2:
// 4 wavefronts, one per SIMD, every LDS operand read feeding two MFMAs).
//
// Tiles reach LDS by direct global->LDS loads (global_load_lds_dwordx4), so no
// registers or vector instructions are spent on staging: each lane fetches the
// 16-byte chunk that belongs at its LDS position, which applies the XOR swizzle of
// the chunks on the global side; rows past the end of a partial tile repeat its last
// row (they are masked).
//
// Software pipeline over 32-key halves of a tile.  Half-step h issues, in a fixed
// order, the score MFMAs of half h+1 and the P.V MFMAs of half h-1; between them the
// vector ALU turns the scores of half h into bf16 probabilities and finally takes
// the max of the new scores, so matrix and vector work overlap (within a wavefront,
// and across the two wavefronts of a SIMD).  K and V have rings of their own,
// because K of a tile is read one half-step before its softmax and V one after:
//   K(t) and the ancestor words of tile t are loaded in iteration t-3 (4 K slots,
//   4 ancestor slots); V(t) is loaded in iteration t-2 (4 V slots).
// Every iteration issues the same loads per lane, so "all but the loads of this
// iteration done" (s_waitcnt vmcnt) before the barrier means that everything the
// next iteration reads has landed.
//
// The running max is raised lazily: the accumulators are rescaled only when a row's
// maximum grows by more than 2^8 in probability (or on its first visible key), so
// probabilities stay below 256 and most halves skip the rescale; the result is the
// same softmax, normalised by the same running sum (the sum of the bf16
// probabilities that enter the P.V product).
#include "mfma_tile.h"

namespace tv {

namespace {

constexpr float kLazy = 8.0f;         // log2 of the largest unnormalised probability
constexpr int kKRing = 4;             // K slots
constexpr int kVRing = 4;             // V slots
constexpr int kAncRing = 4;
constexpr int kAncSlotBytes = kMfmaRowsPerWG * 8;  // per 32-row group: 32 low, 32 high words
constexpr int kVOff = kKRing * kTileBytes;
constexpr int kAncOffL = kVOff + kVRing * kTileBytes;
constexpr int kMaskOff = kAncOffL + kAncRing * kAncSlotBytes;
constexpr int kSmemL = kMaskOff + 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Direct global->LDS loads.  Lane l of a load writes LDS at M0 + 16 l (4 l for the
// dword form), so the LDS base is wave-uniform; the global address is an SGPR base
// plus a per-lane 32-bit offset (an instruction offset would move the LDS address
// too, so none is used).  They are inline assembly so that the compiler does not
// see LDS stores it cannot order: every wait on them is explicit
// (wait_loads_and_barrier).  M0 is saved and restored; one wait state separates
// each M0 write from the load that reads it.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  typedef __attribute__((address_space(3))) const char lds_char_t;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_t*)(p)));
}
// two 16-byte loads, LDS lds and lds + 8192
__device__ __forceinline__ void dma_rows(const void* base, const uint32_t (&off)[2], uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[lds]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[o0], %[b]\n\t"
      "s_add_u32 m0, m0, 0x2000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[o1], %[b]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [o0] "v"(off[0]), [o1] "v"(off[1]), [b] "s"(base), [lds] "s"(lds)
      : "memory");
}
// four 16-byte loads, LDS lds + 4096 j
__device__ __forceinline__ void dma_rows(const void* base, const uint32_t (&off)[4], uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[lds]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[o0], %[b]\n\t"
      "s_add_u32 m0, m0, 0x1000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[o1], %[b]\n\t"
      "s_add_u32 m0, m0, 0x1000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[o2], %[b]\n\t"
      "s_add_u32 m0, m0, 0x1000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[o3], %[b]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [o0] "v"(off[0]), [o1] "v"(off[1]), [o2] "v"(off[2]), [o3] "v"(off[3]), [b] "s"(base),
        [lds] "s"(lds)
      : "memory");
}
// one dword load per 32-row group: LDS lds + 256 k + 4 l
__device__ __forceinline__ void dma_anc(const void* base, const uint32_t (&off)[1], uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[lds]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %[o0], %[b]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [o0] "v"(off[0]), [b] "s"(base), [lds] "s"(lds)
      : "memory");
}
__device__ __forceinline__ void dma_anc(const void* base, const uint32_t (&off)[2], uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[lds]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %[o0], %[b]\n\t"
      "s_add_u32 m0, m0, 0x100\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %[o1], %[b]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [o0] "v"(off[0]), [o1] "v"(off[1]), [b] "s"(base), [lds] "s"(lds)
      : "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0), then s_barrier; the empty asm statements keep the
// compiler from moving LDS accesses across the barrier
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// pin a value: the computation that produces it stays before this point
__device__ __forceinline__ void pin(uint32_t v) { asm volatile("" : : "v"(v)); }
__device__ __forceinline__ void pin(float v) { asm volatile("" : : "v"(v)); }

}  // namespace

template <int G>
__global__ void __launch_bounds__(512 / G, G == 1 ? 2 : 1) k_attn_long(AttnArgs a) {
  constexpr int kWaves = 8 / G;
  constexpr int kT = 64 * kWaves;
  constexpr int kRowLoads = 16 / kWaves;                  // 16-byte K (or V) loads per lane
  constexpr int kLoadsPerIter = 2 * kRowLoads + G;         // K, V and the ancestor words
  static_assert(kWaves * 32 * G == kMfmaRowsPerWG, "256 rows per workgroup");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint32_t* s_tree_mask = reinterpret_cast<uint32_t*>(smem + kMaskOff);

  // ---- work item (XCD-aware: consecutive work indices share an XCD)
  const int per_xcd = gridDim.x / 8;
  const int work = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (work >= a.total_work) return;
  const int tile = work % a.row_tiles;
  const int rest = work / a.row_tiles;
  const int split = rest % a.splits;
  const int pair = rest / a.splits;
  const int g = pair % a.hkv;
  const int b = pair / a.hkv;

  const int n0 = a.cu_nodes[b];
  int count = a.cu_nodes[b + 1] - n0;
  int plen = a.prefix_len[b];
  const int tid = threadIdx.x;
  if (count > a.max_nodes) {
    if (tid == 0 && tile == 0 && split == 0) atomicOr(a.err, TV_ERR_TOO_MANY_NODES);
    count = a.max_nodes;
  }
  if (plen < 0 || plen > a.max_prefix || plen > a.max_blocks * 64) {
    if (tid == 0 && tile == 0 && split == 0) atomicOr(a.err, TV_ERR_BLOCK);
    plen = max(0, min(plen, min(a.max_prefix, a.max_blocks * 64)));
  }
  const int rows = a.group * count;
  const int r0 = tile * kMfmaRowsPerWG;
  if (r0 >= rows) return;

  const int nblk = (plen + kKT - 1) / kKT;
  const int kb0 = split * a.blocks_per_split;
  const int kb1 = min(nblk, kb0 + a.blocks_per_split);
  const int n_prefix_tiles = max(0, kb1 - kb0);
  const bool do_tree = split == a.splits - 1;

  // ---- rows: wavefront w owns the 32-row groups G w .. G w + G - 1
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  int rl[G];
  bool ok[G];
  long grow[G];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    rl[k] = 32 * (G * wave + k) + col;
    ok[k] = r0 + rl[k] < rows;
    const int r = ok[k] ? r0 + rl[k] : r0;
    grow[k] = static_cast<long>(n0 + r / a.group) * a.hq + g * a.group + r % a.group;
  }
  const bool wave_live = r0 + 32 * G * wave < rows;
  bf16x8_t q[G][8];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + grow[k] * kD + half * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      q[k][s] = as_bf16x8(ok[k] ? *reinterpret_cast<const uint4*>(qp + s * 16) : make_uint4(0, 0, 0, 0));
  }

  // ---- which 64-node tree tiles any row of this workgroup can see
  if (tid == 0) *s_tree_mask = 0;
  __syncthreads();
  const int ntw = (count + 63) / 64;
  if (do_tree) {
    const int lo = r0 / a.group;
    const int hi = (min(rows, r0 + kMfmaRowsPerWG) - 1) / a.group;
    const int pairs_n = (hi - lo + 1) * ntw;
    uint32_t m = 0;
    for (int i = tid; i < pairs_n; i += kT) {
      const int nd = lo + i / ntw, t = i % ntw;
      if (a.anc[static_cast<long>(n0 + nd) * a.words + t] != 0) m |= 1u << t;
    }
    if (m) atomicOr(s_tree_mask, m);
  }
  __syncthreads();
  const uint32_t tree_mask = do_tree ? *s_tree_mask : 0u;
  const int n_tiles = n_prefix_tiles + __popc(tree_mask);

  f32x16_t acc[G][4];
#pragma unroll
  for (int k = 0; k < G; ++k)
#pragma unroll
    for (int d = 0; d < 4; ++d) acc[k][d] = f32x16_t{};
  float m_out[G], l[G];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    m_out[k] = -INFINITY;
    l[k] = 0.0f;
  }

  if (n_tiles > 0) {
    const char* kc = static_cast<const char*>(a.k_cache);
    const char* vc = static_cast<const char*>(a.v_cache);
    const char* kt = static_cast<const char*>(a.k_tree);
    const char* vt = static_cast<const char*>(a.v_tree);
    auto tile_kind = [&](int it, int& kind, int& base) __attribute__((always_inline)) {
      if (it < n_prefix_tiles) {
        kind = 0;
        base = (kb0 + it) * kKT;
      } else {
        uint32_t m = tree_mask;
        for (int j = it - n_prefix_tiles; j > 0; --j) m &= m - 1;
        kind = 1;
        base = __ffs(m) - 1;
      }
    };
    const __attribute__((address_space(4))) int32_t* bt_row =
        (const __attribute__((address_space(4))) int32_t*)(a.block_table) +
        static_cast<long>(b) * a.max_blocks;
    // staging lanes: load j of wave w covers tile rows 4 (kWaves j + w) .. +3, lane l
    // the row 4 (kWaves j + w) + l / 16 and LDS chunk l % 16; the ancestor load of a
    // 32-row group takes the low word in lanes 0-31 and the high word in lanes 32-63
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int lrow = 4 * wave + (lane >> 4);
    const int kcb = (((lane & 15) ^ (lrow & 15)) << 4);        // K: chunk c at c ^ (key & 15)
    const int vcb = (((lane & 15) ^ ((lrow & 3) << 2)) << 4);  // V: chunk c at c ^ ((key & 3) << 2)
    uint32_t koff_full[kRowLoads], voff_full[kRowLoads];
#pragma unroll
    for (int j = 0; j < kRowLoads; ++j) {
      koff_full[j] = (4 * kWaves * j + lrow) * 256 + kcb;
      voff_full[j] = (4 * kWaves * j + lrow) * 256 + vcb;
    }
    const char* anc_base = reinterpret_cast<const char*>(a.anc + static_cast<long>(n0) * a.words);
    uint32_t anc_lane[G];
#pragma unroll
    for (int k = 0; k < G; ++k)
      anc_lane[k] = static_cast<uint32_t>(
          min((r0 + 32 * (G * wave + k) + col) / a.group, count - 1) * a.words * 8 + 4 * half);
    const uint32_t lds0 = lds_addr(smem);

    struct Src {
      const char* k;
      const char* v;
      int stride;  // bytes between consecutive keys
      int nvalid;  // rows [0, nvalid) exist; later rows repeat row nvalid - 1 (masked)
      int anc;     // byte offset of the tile's word in a node's ancestor bitset
    };
    auto tile_src = [&](int it) __attribute__((always_inline)) -> Src {
      int kind, base;
      tile_kind(min(it, n_tiles - 1), kind, base);
      Src s;
      if (kind == 0) {
        s.anc = 0;
        s.stride = kD * 2;
        const int blk = bt_row[base / kKT];
        if (blk < 0 || blk >= a.num_blocks) {
          if (tid == 0) atomicOr(a.err, TV_ERR_BLOCK);
          s.k = kc;  // block 0 stands in; the sequence is flagged
          s.v = vc;
          s.nvalid = 1;
          return s;
        }
        const long off = (static_cast<long>(blk) * a.hkv + g) * kKT * kD * 2;
        s.k = kc + off;
        s.v = vc + off;
        s.nvalid = min(kKT, plen - base);
      } else {
        s.anc = base * 8;
        s.stride = a.hkv * kD * 2;
        const long off = (static_cast<long>(n0 + base * 64) * a.hkv + g) * kD * 2;
        s.k = kt + off;
        s.v = vt + off;
        s.nvalid = min(64, count - base * 64);
      }
      return s;
    };
    auto rows_of = [&](const Src& s, int cb, const uint32_t (&full)[kRowLoads],
                       uint32_t (&o)[kRowLoads]) __attribute__((always_inline)) {
      if (s.nvalid == kKT && s.stride == kD * 2) {
#pragma unroll
        for (int j = 0; j < kRowLoads; ++j) o[j] = full[j];
      } else {
#pragma unroll
        for (int j = 0; j < kRowLoads; ++j)
          o[j] = min(4 * kWaves * j + lrow, s.nvalid - 1) * s.stride + cb;
      }
    };
    auto load_k = [&](int t) __attribute__((always_inline)) {  // K rows and ancestor words
      const Src s = tile_src(t);
      uint32_t o[kRowLoads];
      rows_of(s, kcb, koff_full, o);
      dma_rows(s.k, o, lds0 + (t % kKRing) * kTileBytes + wave_u * 1024);
      uint32_t ao[G];
#pragma unroll
      for (int k = 0; k < G; ++k) ao[k] = anc_lane[k] + s.anc;
      dma_anc(anc_base, ao, lds0 + kAncOffL + (t % kAncRing) * kAncSlotBytes + wave_u * 256 * G);
    };
    auto load_v = [&](int t) __attribute__((always_inline)) {
      const Src s = tile_src(t);
      uint32_t o[kRowLoads];
      rows_of(s, vcb, voff_full, o);
      dma_rows(s.v, o, lds0 + kVOff + (t % kVRing) * kTileBytes + wave_u * 1024);
    };

    const float c2 = a.scale * kLog2e;
    const int krow0 = key_perm(col);
    const int k_xor = krow0 & 15;
    int k_base[2];
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) k_base[sg] = (32 * sg + krow0) * 256;
    const int grp = lane >> 4, jg = lane & 15, hh = grp >> 1;
    const int low = 2 * (grp & 1) + ((jg & 3) >> 1);
    int v_base[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      v_base[dt] = (8 * hh + (jg >> 2)) * 256 + ((((dt ^ (jg >> 2)) << 2) + low) << 4) + 8 * (jg & 1);

    // visibility of the 32 keys this lane holds in a tile, per row group, compressed
    // so that bit 16 sg + v belongs to register v of half sg (key 32sg + 16(v/8) +
    // 8 half + v%8); returns true for a whole prefix block (no mask)
    auto tile_vis = [&](int it, uint32_t (&w)[G]) __attribute__((always_inline)) -> bool {
      int kind, base;
      tile_kind(min(it, n_tiles - 1), kind, base);
      if (kind == 0 && plen - base >= kKT) return true;
      const uint32_t* slot =
          reinterpret_cast<const uint32_t*>(smem + kAncOffL + (it % kAncRing) * kAncSlotBytes);
      const uint64_t pvis = (kind == 0) ? (1ull << (plen - base)) - 1ull : 0ull;
#pragma unroll
      for (int k = 0; k < G; ++k) {
        uint32_t lo, hi;
        if (kind == 0) {
          lo = static_cast<uint32_t>(pvis);
          hi = static_cast<uint32_t>(pvis >> 32);
        } else {
          const int gi = G * wave + k;
          lo = ok[k] ? slot[64 * gi + col] : 0u;
          hi = ok[k] ? slot[64 * gi + 32 + col] : 0u;
        }
        const int sh = 8 * half;
        w[k] = ((lo >> sh) & 0xffu) | (((lo >> (16 + sh)) & 0xffu) << 8) |
               (((hi >> sh) & 0xffu) << 16) | (((hi >> (16 + sh)) & 0xffu) << 24);
      }
      return false;
    };
    auto mask = [&](f32x16_t& sc, uint32_t w) __attribute__((always_inline)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[v] = ((w >> v) & 1u) ? sc[v] : -INFINITY;
    };

    // Online softmax state per row group.  Half h (32 keys) is scored in half-step
    // h-1; at the end of that half-step its max sets the reference mr (raised
    // lazily), mc = mr * c2, and the factor al that the accumulators take before the
    // P.V of half h; half-step h turns its scores into bf16 probabilities.
    float mr[G], mc[G], al[G], al_next[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      mr[k] = -INFINITY;
      mc[k] = 0.0f;
      al[k] = 1.0f;
      al_next[k] = 1.0f;
    }
    auto max16 = [&](const f32x16_t& sc) __attribute__((always_inline)) -> float {
      float mx = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
      for (int v = 3; v < 15; v += 2) mx = fmaxf(fmaxf(mx, sc[v]), sc[v + 1]);
      return fmaxf(mx, sc[15]);
    };
    // a row's two halves of keys sit in lanes l and l ^ 32 (permlane32 swap)
    auto bump = [&](float mx, int k) __attribute__((always_inline)) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const bool up = mr[k] == -INFINITY ? mx != -INFINITY : (mx - mr[k]) * c2 > kLazy;
      const float m_new = up ? mx : mr[k];
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      al_next[k] = up ? __builtin_amdgcn_exp2f((mr[k] - m_use) * c2) : 1.0f;
      mc[k] = m_use * c2;
      mr[k] = m_new;
    };
    const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    // probabilities of registers v, v+1: bf16 pair into pk, its sum into sum
    auto exp2_pair = [&](const f32x16_t& sc, int v, float mck, float& sum, uint32_t (&pk)[8])
        __attribute__((always_inline)) {
      const float p0 = __builtin_amdgcn_exp2f(sc[v] * c2 - mck);
      const float p1 = __builtin_amdgcn_exp2f(sc[v + 1] * c2 - mck);
      pk[v >> 1] = pack2_bf16(p0, p1);
      sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[v >> 1]), ones, sum, false);
      pin(pk[v >> 1]);
      pin(sum);
    };
    auto rescale = [&]() __attribute__((always_inline)) {
      bool any = false;
#pragma unroll
      for (int k = 0; k < G; ++k) any = any || al[k] != 1.0f;
      if (__ballot(any)) {
#pragma unroll
        for (int k = 0; k < G; ++k)
#pragma unroll
          for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[k][d][v] *= al[k];
      }
    };

    // One half-step h, in an explicit issue order of 16 MFMA slots (one MFMA per row
    // group, the groups sharing the LDS operand): the 8 score MFMAs of half h+1 (K slot
    // tn, 32-key half hn) into n, interleaved with the 8 P.V MFMAs of half h-1 (V slot
    // tp, half hp, probabilities pp).  LDS operands are read four slots ahead.  Between
    // the MFMAs the vector ALU turns the scores of half h (c) into probabilities pc;
    // at the end the new scores are masked (when masked) and their max taken.
    auto half_step = [&](f32x16_t (&n)[G], int tn, int hn, const uint32_t (&pp)[G][8], int tp,
                         int hp, const f32x16_t (&c)[G], uint32_t (&pc)[G][8], bool masked,
                         const uint32_t (&w)[G], int wsh) __attribute__((always_inline)) {
      const char* ks = smem + (tn % kKRing) * kTileBytes + k_base[hn];
      const char* vs = smem + kVOff + (tp % kVRing) * kTileBytes + 32 * hp * 256;
      uint4 kr[8];
      bf16x4_t vr[8][2];
      auto read = [&](int r) __attribute__((always_inline)) {  // operand r of 16, in use order
        if (r < 8) {
          kr[r] = *reinterpret_cast<const uint4*>(ks + (((2 * r + half) ^ k_xor) << 4));
        } else {
          const int qq = r - 8;
          const char* p = vs + v_base[qq & 3] + 16 * (qq >> 2) * 256;
          vr[qq][0] = ds_read_tr(p);
          vr[qq][1] = ds_read_tr(p + 4 * 256);
        }
      };
      auto mfma = [&](int r) __attribute__((always_inline)) {
        if (r < 8) {
          const bf16x8_t kf = as_bf16x8(kr[r]);
#pragma unroll
          for (int k = 0; k < G; ++k)
            n[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, q[k][r], r == 0 ? f32x16_t{} : n[k], 0, 0, 0);
        } else {
          const int qq = r - 8, jj = qq >> 2, dt = qq & 3;
          const bf16x8_t vf = {vr[qq][0][0], vr[qq][0][1], vr[qq][0][2], vr[qq][0][3],
                               vr[qq][1][0], vr[qq][1][1], vr[qq][1][2], vr[qq][1][3]};
#pragma unroll
          for (int k = 0; k < G; ++k) {
            const bf16x8_t f = as_bf16x8(
                make_uint4(pp[k][4 * jj], pp[k][4 * jj + 1], pp[k][4 * jj + 2], pp[k][4 * jj + 3]));
            acc[k][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, f, acc[k][dt], 0, 0, 0);
          }
        }
      };
      float sum[G], mx[G];
#pragma unroll
      for (int k = 0; k < G; ++k) sum[k] = 0.0f;
      // issue order: S0 S1 P0 S2 P1 ... S7 P6 P7 (S = score step, P = P.V step), so
      // consecutive steps of the dependent score chain are two MFMAs apart and the
      // last score leaves two MFMAs before its max is taken
      constexpr int kOrder[16] = {0, 1, 8, 2, 9, 3, 10, 4, 11, 5, 12, 6, 13, 7, 14, 15};
      constexpr int kAhead = 4;  // LDS operands are read this many MFMAs ahead
#pragma unroll
      for (int r = 0; r < kAhead; ++r) read(kOrder[r]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        mfma(kOrder[r]);
        if (r + kAhead < 16) read(kOrder[r + kAhead]);
        __builtin_amdgcn_sched_barrier(0);
        // probability pairs spread over the slots: pair p = group p / 8, registers
        // 2 (p % 8), +1
        if (G == 2 || (r & 1) == 0) {
          const int pi = G == 1 ? r / 2 : r;
          const int k = pi / 8, v = 2 * (pi % 8);
          exp2_pair(c[k], v, mc[k], sum[k], pc[k]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // the new scores of half h+1: mask, max; half h is done: l takes its factor and
      // sum, and the reference moves to half h+1
      if (masked) {
#pragma unroll
        for (int k = 0; k < G; ++k) mask(n[k], w[k] >> wsh);
      }
#pragma unroll
      for (int k = 0; k < G; ++k) {
        mx[k] = max16(n[k]);
        l[k] = l[k] * al[k] + sum[k];
        m_out[k] = mr[k];
        bump(mx[k], k);
      }
      rescale();
#pragma unroll
      for (int k = 0; k < G; ++k) al[k] = al_next[k];
    };

    f32x16_t s0[G], s1[G];                  // scores of two consecutive halves
    uint32_t px[G][8], py[G][8];            // probabilities of two halves
#pragma unroll
    for (int k = 0; k < G; ++k)
#pragma unroll
      for (int v = 0; v < 8; ++v) px[k][v] = 0u;

    // tile iteration i = half-steps 2i and 2i+1; the visibility of tile i+1 is read
    // from its ancestor slot, which landed one iteration earlier
    uint32_t wc[G], wn[G];
#pragma unroll
    for (int k = 0; k < G; ++k) wc[k] = wn[k] = ~0u;
    bool full_c = true;
    auto body = [&](int i) __attribute__((always_inline)) {
      load_k(i + 3);
      load_v(i + 2);
      if (wave_live) {
        const bool full_n = tile_vis(i + 1, wn);
        // probabilities of tile i half 0, scores of tile i half 1, P.V of tile i-1 half 1
        half_step(s1, i, 1, px, i + 3, 1, s0, py, !full_c, wc, 16);
        // probabilities of tile i half 1, scores of tile i+1 half 0, P.V of tile i half 0
        half_step(s0, i + 1, 0, py, i, 0, s1, px, !full_n, wn, 0);
#pragma unroll
        for (int k = 0; k < G; ++k) wc[k] = wn[k];
        full_c = full_n;
      }
      wait_loads_and_barrier<kLoadsPerIter>();
    };

    // prologue: K(0), K(1) with their ancestor words and V(0), then the loads an
    // iteration -1 would have issued (K(2), V(1)); V slot 3, read as "tile -1" by
    // the first half-step with zero probabilities, is cleared
    load_k(0);
    load_k(1);
    load_v(0);
    load_k(2);
    load_v(1);
    {
      uint4* vz = reinterpret_cast<uint4*>(smem + kVOff + 3 * kTileBytes);
#pragma unroll
      for (int j = 0; j < kTileBytes / 16 / kT; ++j) vz[tid + kT * j] = make_uint4(0, 0, 0, 0);
    }
    wait_loads_and_barrier<kLoadsPerIter>();
    if (wave_live) {  // scores, mask and max of tile 0 half 0
      full_c = tile_vis(0, wc);
      const char* ks = smem + k_base[0];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const bf16x8_t kf =
            as_bf16x8(*reinterpret_cast<const uint4*>(ks + (((2 * r + half) ^ k_xor) << 4)));
#pragma unroll
        for (int k = 0; k < G; ++k)
          s0[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, q[k][r], r == 0 ? f32x16_t{} : s0[k], 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < G; ++k) {
        if (!full_c) mask(s0[k], wc[k]);
        bump(max16(s0[k]), k);
        al[k] = al_next[k];
      }
    }
    for (int i = 0; i < n_tiles; ++i) body(i);
    if (wave_live) {  // P.V of the last half (tile n-1, half 1)
      const char* vs = smem + kVOff + ((n_tiles - 1) % kVRing) * kTileBytes + 32 * 256;
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) {
        const int jj = qq >> 2, dt = qq & 3;
        const char* p = vs + v_base[dt] + 16 * jj * 256;
        const bf16x4_t lo = ds_read_tr(p);
        const bf16x4_t hi = ds_read_tr(p + 4 * 256);
        const bf16x8_t vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int k = 0; k < G; ++k) {
          const bf16x8_t f = as_bf16x8(
              make_uint4(px[k][4 * jj], px[k][4 * jj + 1], px[k][4 * jj + 2], px[k][4 * jj + 3]));
          acc[k][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, f, acc[k][dt], 0, 0, 0);
        }
      }
    }
    wait_loads_and_barrier<0>();
  }

  // ---- epilogue (each lane holds half of its row's sum)
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const float l_tot = l[k] + __shfl_xor(l[k], 32, 64);
    if (!ok[k]) continue;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse = l_tot > 0.0f ? m_out[k] * a.scale + logf(l_tot) : -INFINITY;
    if (a.splits == 1) {
      uint16_t* out = static_cast<uint16_t*>(a.out) + grow[k] * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int d = 32 * dt + 8 * qd + 4 * half;
          *reinterpret_cast<uint2*>(out + d) =
              make_uint2(pack2_bf16(acc[k][dt][4 * qd] * inv, acc[k][dt][4 * qd + 1] * inv),
                         pack2_bf16(acc[k][dt][4 * qd + 2] * inv, acc[k][dt][4 * qd + 3] * inv));
        }
      if (a.lse != nullptr && half == 0) a.lse[grow[k]] = lse;
    } else {
      float* po = a.part_o + (static_cast<long>(split) * a.total_rows + grow[k]) * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int d = 32 * dt + 8 * qd + 4 * half;
          *reinterpret_cast<float4*>(po + d) =
              make_float4(acc[k][dt][4 * qd] * inv, acc[k][dt][4 * qd + 1] * inv,
                          acc[k][dt][4 * qd + 2] * inv, acc[k][dt][4 * qd + 3] * inv);
        }
      if (half == 0) a.part_lse[static_cast<long>(split) * a.total_rows + grow[k]] = lse;
    }
  }
}

template <int G>
static int launch_long(const AttnArgs& a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_long<G>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kSmemL);
    attr_set = true;
  }
  const int grid = 8 * ceil_div(a.total_work, 8);
  hipLaunchKernelGGL(k_attn_long<G>, dim3(grid), dim3(512 / G), kSmemL, s, a);
  const int st = check_launch("tree_verify_attention/long");
  if (st != TV_OK || a.splits == 1) return st;
  return launch_attn_combine(a, s);
}

int launch_attn_long(const AttnArgs& a, int rows_per_wave, hipStream_t s) {
  return rows_per_wave == 64 ? launch_long<2>(a, s) : launch_long<1>(a, s);
}

}  // namespace tv
