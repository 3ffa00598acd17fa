// Matrix-core tree attention for gfx950, pipelined for long work items (many 64-key
// tiles per workgroup).
//
// Same computation and operand layout as k_attn_mfma (scores transposed, S^T = K Q^T;
// O^T = V^T P^T with V read through the LDS transpose read; online softmax; tree mask
// M_tree of page "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力机制与显存碎片
// 整理联合加速" (ufo.work/2026/537), §2.2.2 and appendix B).  A workgroup owns 256 rows,
// 8 wavefronts of 32 rows, two wavefronts per SIMD.
//
// Tiles reach LDS by direct global->LDS loads (global_load_lds_dwordx4), so no
// registers or vector instructions are spent on staging: each lane fetches the
// 16-byte chunk that belongs at its LDS position, which applies the XOR swizzle of
// the chunks on the global side; rows past the end of a partial tile repeat its last
// row (they are masked).
//
// Software pipeline over 32-key halves of a tile.  Half-step h first takes the max
// of the scores of half h (computed one half-step earlier), then issues, in a fixed
// order, the score MFMAs of half h+1 and the P.V MFMAs of half h-1, and between them
// turns the scores of half h into bf16 probabilities on the vector ALU; matrix and
// vector work overlap within a wavefront and across the two wavefronts of a SIMD.
// K and V have rings of their own, because K of a tile is read one half-step before
// its softmax and V one after:
//   K(t) and the ancestor words of tile t are loaded in iteration t-3 (4 K slots,
//   4 ancestor slots); V(t) is loaded in iteration t-2 (4 V slots).
// Every iteration issues the same 5 loads per lane, so "all but the last 5 loads
// done" (s_waitcnt vmcnt(5)) before the barrier means that everything the next
// iteration reads has landed.  The tile loop is unrolled by the ring length, so
// every LDS operand address is a per-lane base plus an instruction offset.
//
// The running max is raised lazily: the accumulators are rescaled only when a row's
// maximum grows by more than 2^8 in probability (or on its first visible key), so
// probabilities stay below 256 and most halves skip the rescale; the result is the
// same softmax, normalised by the same running sum (the sum of the bf16
// probabilities that enter the P.V product).
#include <mutex>

#include "fp8_quant.h"
#include "mfma_tile.h"

namespace tv {

namespace {

constexpr int kWavesL = 8;
constexpr int kTL = 64 * kWavesL;
constexpr float kLazy = 8.0f;         // log2 of the largest unnormalised probability
constexpr int kRing = 4;              // slots of the K, V and ancestor rings
constexpr int kMaxPieces = kMaxTailPieces;  // tail pieces of one work item
constexpr int kVOff = kRing * kTileBytes;
constexpr int kAncSlotBytes = kMfmaRowsPerWG * 8;  // per wavefront: 32 low, 32 high words
constexpr int kAncOffL = kVOff + kRing * kTileBytes;
constexpr int kMaskOff = kAncOffL + kRing * kAncSlotBytes;
constexpr int kSmemL = kMaskOff + 64;
// LDS of the FP8 matrix-core mode: E4M3 K ring, bf16 V ring, E4M3 V staging ring,
// ancestor ring, exponent ring (per tile: K exponents in dwords 0-63, V in 64-127)
constexpr int kTile8Bytes = kKT * kD;  // 64 keys x 128 E4M3 bytes
constexpr int kExpSlotBytes = 512;
constexpr int kVOff8 = kRing * kTile8Bytes;
constexpr int kV8Off = kVOff8 + kRing * kTileBytes;
constexpr int kAncOff8 = kV8Off + kRing * kTile8Bytes;
constexpr int kExpOff = kAncOff8 + kRing * kAncSlotBytes;
constexpr int kMaskOff8 = kExpOff + kRing * kExpSlotBytes;
constexpr int kSmem8 = kMaskOff8 + 64;
static_assert(kSmem8 <= 160 * 1024, "LDS of the FP8 matrix-core mode");
// modes of the pipelined kernel
constexpr int kModeBf16 = 0;   // bf16 cache, tiles by direct loads
constexpr int kModeFp8 = 1;    // E4M3 cache with fp32 row scales, tiles through registers
constexpr int kModeMma8 = 2;   // E4M3 Q, K, V with power-of-two row scales, FP8 matrix cores
template <int kMode>
struct Layout {
  static constexpr int v_off = kMode == kModeMma8 ? kVOff8 : kVOff;
  static constexpr int anc_off = kMode == kModeMma8 ? kAncOff8 : kAncOffL;
  static constexpr int mask_off = kMode == kModeMma8 ? kMaskOff8 : kMaskOff;
  static constexpr int smem = kMode == kModeMma8 ? kSmem8 : kSmemL;
};
constexpr int kLoadsPerIter = 5;      // per lane: 2 K chunks, 1 ancestor dword, 2 V chunks
// A computing wavefront issues the K group of an iteration's loads after the first
// score MFMA of the iteration's first half-step and the V group after the first of
// the second, so the matrix cores have work while the loads are issued (serving
// shapes 257-262 -> 253 us, others unchanged); a wavefront with no live rows issues
// both groups at the start of the iteration.
constexpr int kIssueAt = 0;
static_assert(kWavesL * 32 == kMfmaRowsPerWG, "256 rows per workgroup");

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef int v8i_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  typedef __attribute__((address_space(3))) const char lds_char_t;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_t*)(p)));
}

// The loads of one iteration, in two groups: K rows of one tile (2 x 16 B per lane,
// LDS lds_k and lds_k + 8192) with the ancestor dword of this lane's row (LDS lds_a);
// V rows of another tile (LDS lds_v, lds_v + 8192).  Lane l of a load writes LDS at M0 + 16 l (4 l for
// the dword); the global address is an SGPR base plus a per-lane 32-bit offset (an
// instruction offset would move the LDS address too, so none is used).  Inline
// assembly, so that the compiler does not see LDS stores it cannot order: every wait
// on them is explicit (wait_loads_and_barrier).  M0 is saved and restored; one wait
// state separates each M0 write from the load that reads it.
__device__ __forceinline__ void issue_k_loads(const void* kb, uint32_t ko0, uint32_t ko1,
                                              uint32_t lds_k, const void* ab, uint32_t ao,
                                              uint32_t lds_a) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[lk]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[k0], %[kb]\n\t"
      "s_add_u32 m0, m0, 0x2000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[k1], %[kb]\n\t"
      "s_mov_b32 m0, %[la]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %[a0], %[ab]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [k0] "v"(ko0), [k1] "v"(ko1), [kb] "s"(kb), [lk] "s"(lds_k), [a0] "v"(ao), [ab] "s"(ab),
        [la] "s"(lds_a)
      : "memory");
}

__device__ __forceinline__ void issue_v_loads(const void* vb, uint32_t vo0, uint32_t vo1,
                                              uint32_t lds_v) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[lv]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[v0], %[vb]\n\t"
      "s_add_u32 m0, m0, 0x2000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[v1], %[vb]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [v0] "v"(vo0), [v1] "v"(vo1), [vb] "s"(vb), [lv] "s"(lds_v)
      : "memory");
}

// The FP8 matrix-core mode's K group: one 16-byte chunk of the E4M3 K tile (LDS
// lds_k + 16 l), in wavefront 0 the K exponent byte of key l and in wavefront 1 the V
// exponent byte (byte-wide direct loads: lane l's byte lands zero-extended in dword
// l of lds_e), the ancestor dword.  Four loads per lane in wavefronts 0 and 1, three
// in the others.  (Dword loads of a prefix tile's 64 contiguous exponents, read back
// a byte per key, made the calls slower.)
template <bool kExp>
__device__ __forceinline__ void issue_k8_loads(const void* kb, uint32_t ko, uint32_t lds_k,
                                               const void* eb, uint32_t eo, uint32_t lds_e,
                                               const void* ab, uint32_t ao, uint32_t lds_a) {
  uint32_t saved;
  if constexpr (kExp) {
    asm volatile(
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[lk]\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %[k0], %[kb]\n\t"
        "s_mov_b32 m0, %[le]\n\t"
        "s_nop 0\n\t"
        "global_load_lds_ubyte %[e0], %[eb]\n\t"
        "s_mov_b32 m0, %[la]\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %[a0], %[ab]\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [k0] "v"(ko), [kb] "s"(kb), [lk] "s"(lds_k), [e0] "v"(eo), [eb] "s"(eb),
          [le] "s"(lds_e), [a0] "v"(ao), [ab] "s"(ab), [la] "s"(lds_a)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[lk]\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %[k0], %[kb]\n\t"
        "s_mov_b32 m0, %[la]\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %[a0], %[ab]\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [k0] "v"(ko), [kb] "s"(kb), [lk] "s"(lds_k), [a0] "v"(ao), [ab] "s"(ab),
          [la] "s"(lds_a)
        : "memory");
  }
}

// ... and its V group: one 16-byte chunk of the E4M3 V tile into the staging ring.
__device__ __forceinline__ void issue_v8_load(const void* vb, uint32_t vo, uint32_t lds_v) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[lv]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[v0], %[vb]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [v0] "v"(vo), [vb] "s"(vb), [lv] "s"(lds_v)
      : "memory");
}

// 8 E4M3 bytes (w0, w1) times the power of two `scale` to 8 bf16: the conversion
// instruction applies the exponent of its fp32 scale operand, exactly
__device__ __forceinline__ uint4 fp8x8_to_bf16_pow2(uint32_t w0, uint32_t w1, float scale) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false);
  const bf16x2v b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true);
  const bf16x2v c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false);
  const bf16x2v d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

// The ancestor dword of this lane's row alone (the FP8 pipeline's one direct load per
// iteration; its tiles come through registers).
__device__ __forceinline__ void issue_anc_load(const void* ab, uint32_t ao, uint32_t lds_a) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[la]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %[a0], %[ab]\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [a0] "v"(ao), [ab] "s"(ab), [la] "s"(lds_a)
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

// a pointer that is the same in every lane, moved to scalar registers
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// pin a value: the computation that produces it stays before this point
__device__ __forceinline__ void pin(uint32_t v) { asm volatile("" : : "v"(v)); }
__device__ __forceinline__ void pin(float v) { asm volatile("" : : "v"(v)); }

template <int V>
struct Slot {
  static constexpr int value = V;
};

}  // namespace

// One work item: slot k_slot of die xcd's list.  kFp8: the paged prefix cache holds
// E4M3 bytes with a scale per (block, KV head, position); every tile then reaches LDS
// through registers, two tiles ahead of its use: the registers of tile t are loaded in
// iteration t - 4 and written to the bf16 rings in iteration t - 2 (an FP8 prefix tile
// dequantized on the way, byte x scale rounded to bf16; a tree tile copied), so the
// rest of the kernel is the bf16 one.  Each iteration still issues five loads per lane
// (four register loads and the ancestor dword), so the same wait holds.
template <int kMode>
__device__ __forceinline__ void long_item(const AttnArgs& a, const int xcd, const int k_slot) {
  constexpr bool kFp8 = kMode == kModeFp8;
  constexpr bool kMma8 = kMode == kModeMma8;
  using L = Layout<kMode>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint32_t* s_tree_mask = reinterpret_cast<uint32_t*>(smem + L::mask_off);

  // ---- work item.  Pair rank r (in pair_order, longest first, when given) goes to
  // die r % 8; the m = row_tiles * splits work items of a pair get consecutive
  // slots of that die's list, so they run together and share its L2.  With tail
  // balancing (splits == 1), the die's items past tail_whole are each cut into
  // tail_pieces consecutive slots, one prefix range per piece.
  const int m_items = fetch_args(a) + a.row_tiles * a.splits;
  int item = k_slot / m_items, member = k_slot % m_items, piece = 0, pieces = 1, tail_slot = -1;
  if (a.tail_pieces > 1 && k_slot >= a.tail_whole) {
    const int t = k_slot - a.tail_whole;
    const int idx = a.tail_whole + t / a.tail_pieces;
    item = idx / a.row_tiles;
    member = idx % a.row_tiles;
    piece = t % a.tail_pieces;
    pieces = a.tail_pieces;
    tail_slot = xcd * a.tail_items + t / a.tail_pieces;
  }
  const int rank = kXCDs * item + xcd;
  if (rank >= a.batch * a.hkv) return;
  const int pair = a.pair_order != nullptr ? a.pair_order[rank] : rank;
  const int tile = member % a.row_tiles;
  const int split = member / a.row_tiles;
  const int g = pair % a.hkv;
  const int b = pair / a.hkv;
  const bool first_piece = split == 0 && piece == 0;

  // the sequence's scalars and the block ids of the split's first tiles, requested
  // together (the pipeline re-reads the ids; this brings their line in); a tail
  // piece's range depends on the prefix length, so its guess uses max_prefix
  const int kb0_guess = pieces > 1 ? piece * ceil_div(ceil_div(a.max_prefix, kKT), pieces)
                                   : split * a.blocks_per_split;
  const int32_t* bt_first = a.max_blocks > 0 ? a.block_table + static_cast<long>(b) * a.max_blocks
                                             : a.cu_nodes;  // any readable word
  const int bt_last = max(a.max_blocks - 1, 0);
  int n0, n1, plen, blk0, blk1, blk2;
  load_words6(a.cu_nodes + b, a.cu_nodes + b + 1, a.prefix_len + b,
              bt_first + min(kb0_guess, bt_last), bt_first + min(kb0_guess + 1, bt_last),
              bt_first + min(kb0_guess + 2, bt_last), n0, n1, plen, blk0, blk1, blk2);
  (void)blk0, (void)blk1, (void)blk2;
  int count = n1 - n0;
  const int tid = threadIdx.x;
  if (count > a.max_nodes) {
    if (tid == 0 && tile == 0 && first_piece) atomicOr(a.err, TV_ERR_TOO_MANY_NODES);
    count = a.max_nodes;
  }
  if (plen < 0 || plen > a.max_prefix || plen > a.max_blocks * 64) {
    if (tid == 0 && tile == 0 && first_piece) atomicOr(a.err, TV_ERR_BLOCK);
    plen = max(0, min(plen, min(a.max_prefix, a.max_blocks * 64)));
  }
  const int rows = a.group * count;
  const int r0 = tile * kMfmaRowsPerWG;
  if (r0 >= rows) return;

  const int nblk = (plen + kKT - 1) / kKT;
  const int span = pieces > 1 ? ceil_div(nblk, pieces) : a.blocks_per_split;
  const int kb0 = pieces > 1 ? piece * span : split * a.blocks_per_split;
  const int kb1 = min(nblk, kb0 + span);
  const int n_prefix_tiles = max(0, kb1 - kb0);
  const bool do_tree = split == a.splits - 1 && piece == pieces - 1;

  // ---- rows: wavefront w owns rows 32 w .. 32 w + 31 of the tile
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  const int rl = 32 * wave + col;
  const bool row_ok = r0 + rl < rows;
  const int rr = row_ok ? r0 + rl : r0;
  const long grow = static_cast<long>(n0 + rr / a.group) * a.hq + g * a.group + rr % a.group;
  const bool wave_live = r0 + 32 * wave < rows;
  bf16x8_t q[8];
  v8i_t q8[2];         // FP8 matrix-core mode: E4M3 codes of d = 64 m + 32 half + 0..31
  int q_exp = 127;     // and the row's E8M0 exponent
  uint4 qw[8];         // FP8 matrix-core mode: the bf16 row, quantized after the tile loads
  if constexpr (kMma8) {
    const uint16_t* qr = static_cast<const uint16_t*>(a.q) + grow * kD + 32 * half;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      qw[j] = row_ok ? *reinterpret_cast<const uint4*>(qr + 64 * (j >> 2) + 8 * (j & 3))
                     : make_uint4(0, 0, 0, 0);
  } else {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + grow * kD + half * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      q[s] = as_bf16x8(row_ok ? *reinterpret_cast<const uint4*>(qp + s * 16) : make_uint4(0, 0, 0, 0));
  }

  uint32_t tree_mask = 0u;            // set by the tree-mask pass below
  int n_tiles = n_prefix_tiles;

  f32x16_t acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) acc[d] = f32x16_t{};
  float m_out = -INFINITY, l = 0.0f;

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
  // staging lanes: load j (0, 1) of wave w covers tile rows 32 j + 4 w .. +3, lane l
  // the row 32 j + 4 w + l / 16 and LDS chunk l % 16; the ancestor load takes the
  // low word of row 32 w + l in lanes 0-31 and the high word in lanes 32-63
  const int lrow = 4 * wave + (lane >> 4);
  const int kcb = (((lane & 15) ^ (lrow & 15)) << 4);        // K: chunk c at c ^ (key & 15)
  const int vcb = (((lane & 15) ^ ((lrow & 3) << 2)) << 4);  // V: chunk c at c ^ ((key & 3) << 2)
  const char* anc_base = reinterpret_cast<const char*>(a.anc + static_cast<long>(n0) * a.words);
  const uint32_t anc_lane =
      static_cast<uint32_t>(min((r0 + rl) / a.group, count - 1) * a.words * 8 + 4 * half);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds_kv = lds_addr(smem) + wave_u * 1024;
  const uint32_t lds_anc = lds_addr(smem) + L::anc_off + wave_u * 256;

  // source of tile it (clamped to the last tile)
  struct Src {
    const char* k;
    const char* v;
    uint32_t o0, o1;  // byte offsets of this lane's two rows (before the chunk offset)
    uint32_t anc;     // this lane's byte offset of the tile's ancestor dword
  };
  // the physical block of tile it (clamped to the last tile) when it is a prefix
  // tile, else 0: one scalar load, read ahead of its use by the loop below
  auto tile_blk = [&](int it) __attribute__((always_inline)) -> int {
    int kind, base;
    tile_kind(min(it, n_tiles - 1), kind, base);
    return kind == 0 ? bt_row[base / kKT] : 0;
  };
  // source of tile it given its block (tile_blk(it))
  auto tile_src_b = [&](int it, int blk) __attribute__((always_inline)) -> Src {
    int kind, base;
    tile_kind(min(it, n_tiles - 1), kind, base);
    Src s;
    int stride, nvalid;
    if (kind == 0) {
      s.anc = anc_lane;
      stride = kD * 2;
      nvalid = min(kKT, plen - base);
      if (blk < 0 || blk >= a.num_blocks) {
        if (tid == 0) atomicOr(a.err, TV_ERR_BLOCK);
        s.k = kc;  // block 0 stands in; the sequence is flagged
        s.v = vc;
        nvalid = 1;
      } else {
        const long off = (static_cast<long>(blk) * a.hkv + g) * kKT * kD * 2;
        s.k = kc + off;
        s.v = vc + off;
      }
    } else {
      s.anc = anc_lane + base * 8;
      stride = a.hkv * kD * 2;
      const long off = (static_cast<long>(n0 + base * 64) * a.hkv + g) * kD * 2;
      s.k = kt + off;
      s.v = vt + off;
      nvalid = min(64, count - base * 64);
    }
    s.o0 = min(lrow, nvalid - 1) * stride;
    s.o1 = min(32 + lrow, nvalid - 1) * stride;
    return s;
  };
  auto tile_src = [&](int it) __attribute__((always_inline)) -> Src {
    return tile_src_b(it, tile_blk(it));
  };
  // the loads of one iteration: K and ancestor words of the tile of sk, V of sv
  auto issue_k = [&](const Src& sk, int slot_k) __attribute__((always_inline)) {
    issue_k_loads(sk.k, sk.o0 + kcb, sk.o1 + kcb, lds_kv + slot_k * kTileBytes, anc_base, sk.anc,
                  lds_anc + slot_k * kAncSlotBytes);
  };
  auto issue_v = [&](const Src& sv, int slot_v) __attribute__((always_inline)) {
    issue_v_loads(sv.v, sv.o0 + vcb, sv.o1 + vcb, lds_kv + kVOff + slot_v * kTileBytes);
  };
  auto issue = [&](const Src& sk, int slot_k, const Src& sv, int slot_v)
      __attribute__((always_inline)) {
    issue_k(sk, slot_k);
    issue_v(sv, slot_v);
  };

  // ---- FP8 matrix-core mode: tiles of E4M3 rows (64 keys x 128 bytes), all by direct
  // loads, K and V of a tile in the same iteration.  Chunk p = 64 w + l of a tile (16
  // bytes) is lane l of wave w: K row p / 8 at stored position p % 8, which holds the
  // row's global chunk (p % 8) ^ ((row / 2) % 8) (so that the 32 lanes reading one
  // chunk position of 32 rows spread over the banks); V row p / 8, chunk p % 8 as is
  // (converted in place order).  Exponent lane l: key l.  Rows past a partial tile
  // repeat its last row.
  struct Src8 {
    const char* k;
    const char* v;
    const uint8_t* ke;
    const uint8_t* ve;
    uint32_t ko, vo, eo, anc;
  };
  const int p8 = 64 * wave + lane;
  const int row8 = p8 >> 3;
  const int kch8 = (p8 & 7) ^ ((row8 >> 1) & 7);
  const int vch8 = p8 & 7;
  auto tile_src8 = [&](int it) __attribute__((always_inline)) -> Src8 {
    int kind, base;
    tile_kind(min(it, n_tiles - 1), kind, base);
    Src8 s8;
    int stride, estride, nvalid;
    if (kind == 0) {
      s8.anc = anc_lane;
      const int blk = bt_row[base / kKT];
      nvalid = min(kKT, plen - base);
      long row0 = static_cast<long>(g) * kKT;  // block 0 stands in for a bad id
      if (blk < 0 || blk >= a.num_blocks) {
        if (tid == 0) atomicOr(a.err, TV_ERR_BLOCK);
        nvalid = 1;
      } else {
        row0 = (static_cast<long>(blk) * a.hkv + g) * kKT;
      }
      s8.k = kc + row0 * kD;
      s8.v = vc + row0 * kD;
      s8.ke = a.k_exp + row0;
      s8.ve = a.v_exp + row0;
      stride = kD;
      estride = 1;
    } else {
      s8.anc = anc_lane + base * 8;
      nvalid = min(64, count - base * 64);
      const long row0 = static_cast<long>(n0 + base * 64) * a.hkv + g;
      s8.k = reinterpret_cast<const char*>(a.kt8) + row0 * kD;
      s8.v = reinterpret_cast<const char*>(a.vt8) + row0 * kD;
      s8.ke = a.kt_e + row0;
      s8.ve = a.vt_e + row0;
      stride = a.hkv * kD;
      estride = a.hkv;
    }
    s8.k = uniform_ptr(s8.k);  // (uniform: block id, sequence and head are)
    s8.v = uniform_ptr(s8.v);
    s8.ke = uniform_ptr(s8.ke);
    s8.ve = uniform_ptr(s8.ve);
    s8.ko = min(row8, nvalid - 1) * stride + 16 * kch8;
    s8.vo = min(row8, nvalid - 1) * stride + 16 * vch8;
    s8.eo = min(lane, nvalid - 1) * estride;
    return s8;
  };
  const uint32_t lds_k8 = lds_addr(smem) + wave_u * 1024;
  const uint32_t lds_v8 = lds_addr(smem) + kV8Off + wave_u * 1024;
  const uint32_t lds_e8 = lds_addr(smem) + kExpOff;
  auto issue_k8 = [&](const Src8& t, int slot) __attribute__((always_inline)) {
    if (wave_u < 2)
      issue_k8_loads<true>(t.k, t.ko, lds_k8 + slot * kTile8Bytes, wave_u == 0 ? t.ke : t.ve, t.eo,
                           lds_e8 + slot * kExpSlotBytes + 256 * wave_u, anc_base, t.anc,
                           lds_anc + slot * kAncSlotBytes);
    else
      issue_k8_loads<false>(t.k, t.ko, lds_k8 + slot * kTile8Bytes, nullptr, 0u, 0u, anc_base, t.anc,
                            lds_anc + slot * kAncSlotBytes);
  };
  auto issue_v8 = [&](const Src8& t, int slot) __attribute__((always_inline)) {
    issue_v8_load(t.v, t.vo, lds_v8 + slot * kTile8Bytes);
  };
  // V tile of staging slot `slot` to bf16 in the V ring's slot `slot`: thread t takes
  // key t / 8, bytes 16 (t % 8) .. +15, times the key's power-of-two scale
  auto convert_v = [&](int slot) __attribute__((always_inline)) {
    const int key = tid >> 3, c8 = tid & 7;
    const uint4 w = *reinterpret_cast<const uint4*>(smem + kV8Off + slot * kTile8Bytes + 16 * tid);
    const uint32_t e =
        *reinterpret_cast<const uint32_t*>(smem + kExpOff + slot * kExpSlotBytes + 256 + 4 * key);
    const float sc = __uint_as_float(e << 23);
    char* vst = smem + kVOff8 + slot * kTileBytes;
    *reinterpret_cast<uint4*>(vst + v_off(key, 2 * c8)) = fp8x8_to_bf16_pow2(w.x, w.y, sc);
    *reinterpret_cast<uint4*>(vst + v_off(key, 2 * c8 + 1)) = fp8x8_to_bf16_pow2(w.z, w.w, sc);
  };

  // ---- FP8 pipeline: a tile's registers.  FP8 prefix tile: thread t holds the 16
  // E4M3 bytes 16 (t % 8) .. of key t / 8 of K (a) and V (b) and that key's scales
  // (c.x, d.x); bf16 tree tile: chunks t and t + 512 of K (a, b) and V (c, d).
  struct Regs {
    uint4 a, b, c, d;
  };
  const uint8_t* k8 = static_cast<const uint8_t*>(a.k_cache);
  const uint8_t* v8 = static_cast<const uint8_t*>(a.v_cache);
  auto load_regs = [&](int it, Regs& r) __attribute__((always_inline)) {
    int kind, base;
    tile_kind(min(it, n_tiles - 1), kind, base);
    if (kind == 0) {
      int blk = bt_row[base / kKT];
      int nvalid = min(kKT, plen - base);
      if (blk < 0 || blk >= a.num_blocks) {
        if (tid == 0) atomicOr(a.err, TV_ERR_BLOCK);
        blk = 0;  // block 0 stands in; the sequence is flagged
        nvalid = 1;
      }
      const long row0 = (static_cast<long>(blk) * a.hkv + g) * kKT;
      const long key = row0 + min(tid >> 3, nvalid - 1);
      r.a = *reinterpret_cast<const uint4*>(k8 + key * kD + 16 * (tid & 7));
      r.b = *reinterpret_cast<const uint4*>(v8 + key * kD + 16 * (tid & 7));
      r.c.x = __float_as_uint(a.k_scale[key]);
      r.d.x = __float_as_uint(a.v_scale[key]);
    } else {
      const int nvalid = min(64, count - base * 64);
      const long row0 = static_cast<long>(n0 + base * 64);
      const int key0 = min(tid >> 4, nvalid - 1), key1 = min((tid + kTL) >> 4, nvalid - 1);
      const long o0 = ((row0 + key0) * a.hkv + g) * kD * 2 + 16 * (tid & 15);
      const long o1 = ((row0 + key1) * a.hkv + g) * kD * 2 + 16 * (tid & 15);
      r.a = *reinterpret_cast<const uint4*>(kt + o0);
      r.b = *reinterpret_cast<const uint4*>(kt + o1);
      r.c = *reinterpret_cast<const uint4*>(vt + o0);
      r.d = *reinterpret_cast<const uint4*>(vt + o1);
    }
  };
  auto store_regs = [&](int it, int slot, const Regs& r) __attribute__((always_inline)) {
    int kind, base;
    tile_kind(min(it, n_tiles - 1), kind, base);
    char* kst = smem + slot * kTileBytes;
    char* vst = smem + kVOff + slot * kTileBytes;
    if (kind == 0) {
      const int key = tid >> 3, c8 = tid & 7;
      const float sk = __uint_as_float(r.c.x), sv = __uint_as_float(r.d.x);
      *reinterpret_cast<uint4*>(kst + k_off(key, 2 * c8)) = fp8x8_to_bf16(r.a.x, r.a.y, sk);
      *reinterpret_cast<uint4*>(kst + k_off(key, 2 * c8 + 1)) = fp8x8_to_bf16(r.a.z, r.a.w, sk);
      *reinterpret_cast<uint4*>(vst + v_off(key, 2 * c8)) = fp8x8_to_bf16(r.b.x, r.b.y, sv);
      *reinterpret_cast<uint4*>(vst + v_off(key, 2 * c8 + 1)) = fp8x8_to_bf16(r.b.z, r.b.w, sv);
    } else {
      const int key0 = tid >> 4, key1 = (tid + kTL) >> 4, c = tid & 15;
      *reinterpret_cast<uint4*>(kst + k_off(key0, c)) = r.a;
      *reinterpret_cast<uint4*>(kst + k_off(key1, c)) = r.b;
      *reinterpret_cast<uint4*>(vst + v_off(key0, c)) = r.c;
      *reinterpret_cast<uint4*>(vst + v_off(key1, c)) = r.d;
    }
  };
  auto issue_anc = [&](int it, int slot) __attribute__((always_inline)) {
    int kind, base;
    tile_kind(min(it, n_tiles - 1), kind, base);
    issue_anc_load(anc_base, kind == 0 ? anc_lane : anc_lane + base * 8,
                   lds_anc + slot * kAncSlotBytes);
  };
  Regs rx{}, ry{};  // registers of even and odd tiles

  // The first three tiles' loads do not depend on the tree mask when they are all
  // prefix tiles: then they are issued before the mask pass, whose ancestor-word
  // loads overlap them (the tiles are older than those loads, so the compiler's
  // wait for the words also covers them).  V slot 3, read as "tile -1" by the first
  // half-step with zero probabilities, is cleared.
  Src sv{};  // V source of the next iteration's loads
  auto prologue = [&]() __attribute__((always_inline)) {
    if constexpr (kFp8) {
      // tiles 0 and 1 into the rings now, tiles 2 and 3 into registers; the
      // ancestor words of tiles 0, 1 and 2
      load_regs(0, rx);
      load_regs(1, ry);
      store_regs(0, 0, rx);
      store_regs(1, 1, ry);
      issue_anc(0, 0);
      issue_anc(1, 1);
      issue_anc(2, 2);
      load_regs(2, rx);
      load_regs(3, ry);
    } else if constexpr (kMma8) {
      // K, exponents, ancestor words and V of tiles 0, 1 and 2 (V(0) is converted
      // before the first iteration, V(t + 1) in iteration t)
      const Src8 t0 = tile_src8(0), t1 = tile_src8(1), t2 = tile_src8(2);
      issue_k8(t0, 0);
      issue_v8(t0, 0);
      issue_k8(t1, 1);
      issue_v8(t1, 1);
      issue_k8(t2, 2);
      issue_v8(t2, 2);
    } else {
      sv = tile_src(2);
      const Src t0 = tile_src(0), t1 = tile_src(1);
      issue(t0, 0, t0, 0);
      issue(t1, 1, t0, 0);
      issue(sv, 2, t1, 1);
    }
    uint4* vz = reinterpret_cast<uint4*>(smem + L::v_off + 3 * kTileBytes);
#pragma unroll
    for (int j = 0; j < kTileBytes / 16 / kTL; ++j) vz[tid + kTL * j] = make_uint4(0, 0, 0, 0);
  };
  const bool early = n_prefix_tiles >= (kFp8 ? 4 : 3);
  if (early) prologue();

  // ---- which 64-node tree tiles any row of this workgroup can see
  if (tid == 0) *s_tree_mask = 0;
  __syncthreads();
  const int ntw = (count + 63) / 64;
  if (do_tree) {
    const int lo = r0 / a.group;
    const int hi = (min(rows, r0 + kMfmaRowsPerWG) - 1) / a.group;
    const int pairs_n = (hi - lo + 1) * ntw;
    uint32_t m = 0;
    for (int i = tid; i < pairs_n; i += kTL) {
      const int nd = lo + i / ntw, t = i % ntw;
      if (a.anc[static_cast<long>(n0 + nd) * a.words + t] != 0) m |= 1u << t;
    }
    if (m) atomicOr(s_tree_mask, m);
  }
  __syncthreads();
  tree_mask = do_tree ? *s_tree_mask : 0u;
  n_tiles = n_prefix_tiles + __popc(tree_mask);

  if (n_tiles > 0) {
    if (!early) prologue();
    const float c2 = a.scale * kLog2e;
    // per-lane LDS bases of the MFMA operands; slot, half and step are instruction offsets
    const int krow0 = key_perm(col);
    const int k_xor = krow0 & 15;
    const char* kaddr[8];  // K operand of score step r in slot 0, keys 0-31
#pragma unroll
    for (int r = 0; r < 8; ++r) kaddr[r] = smem + krow0 * 256 + (((2 * r + half) ^ k_xor) << 4);
    if constexpr (kMma8) {
      // q's row quantized with the rule of the row quantizer (after the first tile
      // loads are on their way): its maximum from both halves (lanes col and col + 32
      // hold the row), bf16 magnitudes compared as integers
      uint32_t mb = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t ww[4] = {qw[j].x, qw[j].y, qw[j].z, qw[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) mb = max(mb, max(ww[e] & 0x7fffu, (ww[e] >> 16) & 0x7fffu));
      }
      const auto sw = __builtin_amdgcn_permlane32_swap(mb, mb, false, false);
      mb = max(sw[0], sw[1]);
      const int sh = e8m0_shift(__uint_as_float(mb << 16));
      q_exp = sh + 127;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t ww[4] = {qw[j].x, qw[j].y, qw[j].z, qw[j].w};
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = ldexpf(__uint_as_float(ww[e] << 16), -sh);
          f[2 * e + 1] = ldexpf(__uint_as_float(ww[e] & 0xffff0000u), -sh);
        }
        uint32_t c0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        c0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], c0, true);
        uint32_t c1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        c1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], c1, true);
        q8[j >> 2][2 * (j & 3)] = static_cast<int>(c0);
        q8[j >> 2][2 * (j & 3) + 1] = static_cast<int>(c1);
      }
    }
    // FP8 matrix-core mode: the E4M3 K operand of MFMA m (d = 64 m + 32 half + 0..31,
    // two chunks) in slot 0, keys 0-31, and this lane's key exponent
    const char* kaddr8[2][2];
    const int f8 = (krow0 >> 1) & 7;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < 2; ++j) kaddr8[m][j] = smem + krow0 * kD + (((4 * m + 2 * half + j) ^ f8) << 4);
    const char* keaddr = smem + kExpOff + 4 * krow0;
    const int grp = lane >> 4, jg = lane & 15, hh = grp >> 1;
    const int low = 2 * (grp & 1) + ((jg & 3) >> 1);
    const char* vaddr[4];  // V^T operand of d-tile dt in slot 0, keys 0-15
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      vaddr[dt] = smem + L::v_off + (8 * hh + (jg >> 2)) * 256 +
                  ((((dt ^ (jg >> 2)) << 2) + low) << 4) + 8 * (jg & 1);

    // visibility of the 32 keys this lane holds in a tile, compressed so that bit
    // 16 sg + v belongs to register v of half sg (key 32sg + 16(v/8) + 8 half + v%8);
    // returns true for a whole prefix block (no mask)
    auto tile_vis = [&](int it, int slot, uint32_t& w) __attribute__((always_inline)) -> bool {
      int kind, base;
      tile_kind(it, kind, base);
      if (kind == 0 && plen - base >= kKT) return true;
      uint32_t lo, hi;
      if (kind == 0) {
        const uint64_t pvis = (1ull << (plen - base)) - 1ull;
        lo = static_cast<uint32_t>(pvis);
        hi = static_cast<uint32_t>(pvis >> 32);
      } else {
        const uint32_t* s = reinterpret_cast<const uint32_t*>(smem + L::anc_off + slot * kAncSlotBytes);
        lo = row_ok ? s[64 * wave + col] : 0u;
        hi = row_ok ? s[64 * wave + 32 + col] : 0u;
      }
      const int sh = 8 * half;
      w = ((lo >> sh) & 0xffu) | (((lo >> (16 + sh)) & 0xffu) << 8) |
          (((hi >> sh) & 0xffu) << 16) | (((hi >> (16 + sh)) & 0xffu) << 24);
      return false;
    };
    auto mask = [&](f32x16_t& sc, uint32_t w) __attribute__((always_inline)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[v] = ((w >> v) & 1u) ? sc[v] : -INFINITY;
    };

    // online softmax state: reference max mr (raised lazily), mc = mr * c2
    // mr starts finite: the first visible key always raises it (rescale factor
    // exp2(-huge) = 0) and a half with no visible key (mx = -inf) never does, which
    // gives the references and factors of a start at -inf without its special cases
    float mr = -1.0e30f, mc = mr * c2;
    const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

    // One half-step h: mask and max of the scores c of half h, then 16 MFMAs in a
    // fixed order, S0 S1 P0 S2 P1 .. S7 P6 P7: the score steps of half h+1 (K slot
    // ks, 32-key half hn) into n and the P.V steps of half h-1 (V slot vs, half hp,
    // probabilities pp).  LDS operands are read four MFMAs ahead; between the MFMAs
    // the vector ALU turns c into probabilities pc, one per MFMA.  At the end, l
    // takes the rescale factor and the sum of half h, and so do the accumulators,
    // which then wait for the P.V of half h.
    auto half_step = [&](f32x16_t& n, int ks, int hn, const uint32_t (&pp)[8], int vs, int hp,
                         f32x16_t& c, uint32_t (&pc)[8], bool masked, uint32_t w, auto&& hook)
        __attribute__((always_inline)) {
      if (masked) mask(c, w);
      float mx = fmaxf(fmaxf(c[0], c[1]), c[2]);
#pragma unroll
      for (int v = 3; v < 15; v += 2) mx = fmaxf(fmaxf(mx, c[v]), c[v + 1]);
      mx = fmaxf(mx, c[15]);
      // a row's two halves of keys sit in lanes l and l ^ 32 (permlane32 swap)
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const bool up = (mx - mr) * c2 > kLazy;
      const float al_up = __builtin_amdgcn_exp2f((mr - mx) * c2);
      mr = up ? mx : mr;
      const float al = up ? al_up : 1.0f;
      mc = mr * c2;

      uint4 kr[8];
      uint4 kr8[2][2];
      uint32_t ke = 127u;
      bf16x4_t vr[8][2];
      constexpr int kOrder[16] = {0, 1, 8, 2, 9, 3, 10, 4, 11, 5, 12, 6, 13, 7, 14, 15};
      auto read = [&](int r) __attribute__((always_inline)) {  // operand of MFMA r
        if (r < 8) {
          if constexpr (kMma8) {
            if ((r & 3) == 0) {
              const int m = r >> 2;
              const int off = ks * kTile8Bytes + hn * 32 * kD;
              kr8[m][0] = *reinterpret_cast<const uint4*>(kaddr8[m][0] + off);
              kr8[m][1] = *reinterpret_cast<const uint4*>(kaddr8[m][1] + off);
              if (m == 0) ke = *reinterpret_cast<const uint32_t*>(keaddr + ks * kExpSlotBytes + hn * 128);
            }
          } else {
            kr[r] = *reinterpret_cast<const uint4*>(kaddr[r] + ks * kTileBytes + hn * 32 * 256);
          }
        } else {
          const int qq = r - 8;
          const char* p = vaddr[qq & 3] + vs * kTileBytes + (32 * hp + 16 * (qq >> 2)) * 256;
          vr[qq][0] = ds_read_tr(p);
          vr[qq][1] = ds_read_tr(p + 4 * 256);
        }
      };
      auto mfma = [&](int r) __attribute__((always_inline)) {
        if (r < 8) {
          if constexpr (kMma8) {
            if ((r & 3) == 0) {  // scores over d = 64 m .. 64 m + 63, scales applied inside
              const int m = r >> 2;
              const v8i_t a8 = {static_cast<int>(kr8[m][0].x), static_cast<int>(kr8[m][0].y),
                                static_cast<int>(kr8[m][0].z), static_cast<int>(kr8[m][0].w),
                                static_cast<int>(kr8[m][1].x), static_cast<int>(kr8[m][1].y),
                                static_cast<int>(kr8[m][1].z), static_cast<int>(kr8[m][1].w)};
              n = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  a8, q8[m], m == 0 ? f32x16_t{} : n, 0, 0, 0, static_cast<int>(ke), 0, q_exp);
            }
          } else {
            n = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[r]), q[r],
                                                        r == 0 ? f32x16_t{} : n, 0, 0, 0);
          }
        } else {
          const int qq = r - 8, jj = qq >> 2, dt = qq & 3;
          const bf16x8_t vf = {vr[qq][0][0], vr[qq][0][1], vr[qq][0][2], vr[qq][0][3],
                               vr[qq][1][0], vr[qq][1][1], vr[qq][1][2], vr[qq][1][3]};
          const bf16x8_t f =
              as_bf16x8(make_uint4(pp[4 * jj], pp[4 * jj + 1], pp[4 * jj + 2], pp[4 * jj + 3]));
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, f, acc[dt], 0, 0, 0);
        }
      };
      float sum = 0.0f;
      // one probability per MFMA slot, packed in pairs a slot later (each exp result
      // is used two instructions later or more), so every MFMA has a short block of
      // vector work behind it rather than four exponentials behind every fourth one
      // (long 1041 -> 1023 us, wide 367 -> 359, serving 251 -> 247)
      float pe[16];
      auto pack = [&](int k) __attribute__((always_inline)) {
        pc[k] = pack2_bf16(pe[2 * k], pe[2 * k + 1]);
        sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pc[k]), ones, sum, false);
        pin(pc[k]);
        pin(sum);
      };
      constexpr int kAhead = 4;
#pragma unroll
      for (int r = 0; r < kAhead; ++r) read(kOrder[r]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        mfma(kOrder[r]);
        if (r + kAhead < 16) read(kOrder[r + kAhead]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kMma8) {
          // (four every fourth slot here: this mode has two score MFMAs per half-step,
          // and one exponential per slot measured 2% slower)
          if ((r & 3) == 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) pe[r - 1 + e] = __builtin_amdgcn_exp2f(c[r - 1 + e] * c2 - mc);
            pack((r - 1) >> 1);
            pack(((r - 1) >> 1) + 1);
          }
        } else {
          pe[r] = __builtin_amdgcn_exp2f(c[r] * c2 - mc);
          if (r >= 2 && (r & 1) == 0) pack((r - 2) >> 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (r == kIssueAt) hook();
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!kMma8) pack(7);
      l = l * al + sum;
      m_out = mr;
      if (__ballot(al != 1.0f)) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[d][v] *= al;
      }
    };

    // end of an iteration: all but this iteration's loads done (per wavefront: the FP8
    // matrix-core mode issues four in wavefronts 0 and 1, three elsewhere), then the
    // barrier
    auto wait_iteration = [&]() __attribute__((always_inline)) {
      if constexpr (kMma8) {
        if (wave_u < 2)
          wait_loads_and_barrier<4>();
        else
          wait_loads_and_barrier<3>();
      } else {
        wait_loads_and_barrier<kLoadsPerIter>();
      }
    };
    f32x16_t s0, s1;         // scores of two consecutive halves
    uint32_t px[8], py[8];   // probabilities of two halves
#pragma unroll
    for (int v = 0; v < 8; ++v) px[v] = 0u;
    // bf16 mode: the block of the tile whose loads the next iteration issues, read
    // at the end of this one, so that the barrier's wait covers its scalar load (a
    // read at the top of the iteration stalled every iteration on it)
    int blk_ahead = 0;
    if constexpr (!kFp8 && !kMma8) blk_ahead = tile_blk(3);

    // tile iteration i (ring slot S = i % 4) = half-steps 2i and 2i+1
    auto body = [&](int i, auto slot) __attribute__((always_inline)) {
      constexpr int S = decltype(slot)::value;
      if constexpr (kFp8) {
        // tile i+2 from its registers into the rings, then the ancestor word of tile
        // i+3 and the registers of tile i+4 (the same registers, now free)
        Regs& r = (S % 2 == 0) ? rx : ry;
        store_regs(i + 2, (S + 2) % kRing, r);
        issue_anc(i + 3, (S + 3) % kRing);
        load_regs(i + 4, r);
      }
      if constexpr (kMma8) convert_v((S + 1) % kRing);  // V(i + 1), landed last iteration
      Src sk{};
      Src8 sk8{};
      if constexpr (kMma8) {
        sk8 = tile_src8(i + 3);
      } else if constexpr (!kFp8) {
        sk = tile_src_b(i + 3, blk_ahead);
      }
      // the K group of this iteration's loads, then the V group (see kIssueAt)
      const auto hk = [&]() __attribute__((always_inline)) {
        if constexpr (kMma8)
          issue_k8(sk8, (S + 3) % kRing);
        else if constexpr (!kFp8)
          issue_k(sk, (S + 3) % kRing);
      };
      const auto hv = [&]() __attribute__((always_inline)) {
        if constexpr (kMma8)
          issue_v8(sk8, (S + 3) % kRing);
        else if constexpr (!kFp8)
          issue_v(sv, (S + 2) % kRing);
      };
      if (!wave_live) {
        hk();
        hv();
      }
      if (wave_live) {
        uint32_t w = ~0u;
        const bool full = tile_vis(i, S, w);
        // probabilities of tile i half 0, scores of tile i half 1, P.V of tile i-1 half 1
        half_step(s1, S, 1, px, (S + 3) % kRing, 1, s0, py, !full, w, hk);
        // probabilities of tile i half 1, scores of tile i+1 half 0, P.V of tile i half 0
        half_step(s0, (S + 1) % kRing, 0, py, S, 0, s1, px, !full, w >> 16, hv);
      }
      if constexpr (!kFp8 && !kMma8) {
        sv = sk;
        blk_ahead = tile_blk(i + 4);  // lands by the barrier's wait
      }
      wait_iteration();
    };

    // prologue (issued above): three groups of loads in the iteration pattern, K(0),
    // K(1) and K(2) with their ancestor words and V(0), V(0), V(1)
    wait_iteration();
    if constexpr (kMma8) {  // V(0) to bf16 before the first iteration reads it
      convert_v(0);
      __syncthreads();
    }
    if (wave_live) {  // scores of tile 0 half 0
      if constexpr (kMma8) {
        const int ke0 = static_cast<int>(*reinterpret_cast<const uint32_t*>(keaddr));
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint4 x0 = *reinterpret_cast<const uint4*>(kaddr8[m][0]);
          const uint4 x1 = *reinterpret_cast<const uint4*>(kaddr8[m][1]);
          const v8i_t a8 = {static_cast<int>(x0.x), static_cast<int>(x0.y), static_cast<int>(x0.z),
                            static_cast<int>(x0.w), static_cast<int>(x1.x), static_cast<int>(x1.y),
                            static_cast<int>(x1.z), static_cast<int>(x1.w)};
          s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, q8[m], m == 0 ? f32x16_t{} : s0, 0,
                                                               0, 0, ke0, 0, q_exp);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r)
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(*reinterpret_cast<const uint4*>(kaddr[r])), q[r], r == 0 ? f32x16_t{} : s0, 0, 0, 0);
      }
    }
    int i = 0;
    for (; i + 4 <= n_tiles; i += 4) {
      body(i, Slot<0>{});
      body(i + 1, Slot<1>{});
      body(i + 2, Slot<2>{});
      body(i + 3, Slot<3>{});
    }
    if (i < n_tiles) body(i, Slot<0>{});
    if (i + 1 < n_tiles) body(i + 1, Slot<1>{});
    if (i + 2 < n_tiles) body(i + 2, Slot<2>{});
    if (wave_live) {  // P.V of the last half (tile n-1, half 1)
      const int vs = (n_tiles - 1) % kRing;
#pragma unroll
      for (int qq = 0; qq < 8; ++qq) {
        const int jj = qq >> 2, dt = qq & 3;
        const char* p = vaddr[dt] + vs * kTileBytes + (32 + 16 * jj) * 256;
        const bf16x4_t lo = ds_read_tr(p);
        const bf16x4_t hi = ds_read_tr(p + 4 * 256);
        const bf16x8_t vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8_t f =
            as_bf16x8(make_uint4(px[4 * jj], px[4 * jj + 1], px[4 * jj + 2], px[4 * jj + 3]));
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, f, acc[dt], 0, 0, 0);
      }
    }
    wait_loads_and_barrier<0>();
  }

  // ---- epilogue (each lane holds half of its row's sum and d = 32 dt + 8 qd + 4 half
  // + 0..3 of its row's output)
  const float l_tot = l + __shfl_xor(l, 32, 64);
  float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float lse = l_tot > 0.0f ? m_out * a.scale + logf(l_tot) : -INFINITY;
  if (pieces > 1) {
    // a piece of a tail item: store the piece's normalised output and log-sum-exp,
    // then take a ticket; the piece that takes the last one merges all pieces and
    // zeroes the ticket for the next call.  The others' stores are visible to it:
    // every lane's stores complete before the barrier, one thread then releases them
    // at device scope (the die's L2 is written back) and takes the ticket; the
    // merging piece's ticket thread acquires (caches invalidated) before the barrier
    // that starts the merge.  One fence per workgroup rather than per lane: each fence
    // writes back or invalidates the whole L2 of the die, which the other work items
    // of the pair are reading their K/V tiles from.  (Prefix splits of a short verify
    // are merged by k_attn_combine instead: there every workgroup runs at once and
    // such fences, one per workgroup, made the call slower than the extra launch.)
    const long p_base = static_cast<long>(tail_slot) * pieces * kMfmaRowsPerWG + rl;
    const long p_stride = kMfmaRowsPerWG;
    const int ticket = tail_slot, n_pieces = pieces, my_piece = piece;
    if (row_ok) {
      float* po = a.part_o + (p_base + my_piece * p_stride) * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<float4*>(po + 32 * dt + 8 * qd + 4 * half) =
              make_float4(acc[dt][4 * qd] * inv, acc[dt][4 * qd + 1] * inv,
                          acc[dt][4 * qd + 2] * inv, acc[dt][4 * qd + 3] * inv);
      if (half == 0) a.part_lse[p_base + my_piece * p_stride] = lse;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    int* s_last = reinterpret_cast<int*>(smem + L::mask_off + 4);
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const bool last = atomicAdd(a.tickets + ticket, 1) == n_pieces - 1;
      if (last) a.tickets[ticket] = 0;  // every piece has taken its ticket
      *s_last = last;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (*s_last == 0) return;
    if (!row_ok) return;
    // lse = log sum_p exp(lse_p), out = sum_p exp(lse_p - lse) out_p
    float lp[kMaxPieces];
    float mx = -INFINITY;
#pragma unroll
    for (int pc = 0; pc < kMaxPieces; ++pc) {
      lp[pc] = pc < n_pieces ? a.part_lse[p_base + pc * p_stride] : -INFINITY;
      mx = fmaxf(mx, lp[pc]);
    }
    const float mref = mx == -INFINITY ? 0.0f : mx;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16_t{};
    float w_sum = 0.0f;
#pragma unroll
    for (int pc = 0; pc < kMaxPieces; ++pc) {
      if (pc >= n_pieces) break;
      const float w = __builtin_amdgcn_exp2f((lp[pc] - mref) * kLog2e);
      w_sum += w;
      const float* po = a.part_o + (p_base + pc * p_stride) * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const float4 x = *reinterpret_cast<const float4*>(po + 32 * dt + 8 * qd + 4 * half);
          acc[dt][4 * qd] = fmaf(w, x.x, acc[dt][4 * qd]);
          acc[dt][4 * qd + 1] = fmaf(w, x.y, acc[dt][4 * qd + 1]);
          acc[dt][4 * qd + 2] = fmaf(w, x.z, acc[dt][4 * qd + 2]);
          acc[dt][4 * qd + 3] = fmaf(w, x.w, acc[dt][4 * qd + 3]);
        }
    }
    inv = w_sum > 0.0f ? 1.0f / w_sum : 0.0f;
    lse = w_sum > 0.0f ? mx + logf(w_sum) : -INFINITY;
  }
  if (!row_ok) return;
  // The split partials go out by streaming stores (LLaVA-like call 15.4 -> 14.5 us);
  // the bf16 output rows do not: 8-byte pieces of many rows per store instruction,
  // which a streaming store sends out as partial lines (wide tree 372 -> 400 us)
  if (a.splits > 1) {  // k_attn_combine merges the prefix splits after the kernel ends
    float* po = a.part_o + (static_cast<long>(split) * a.total_rows + grow) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        store_stream4(po + 32 * dt + 8 * qd + 4 * half, acc[dt][4 * qd] * inv,
                      acc[dt][4 * qd + 1] * inv, acc[dt][4 * qd + 2] * inv,
                      acc[dt][4 * qd + 3] * inv);
    if (half == 0) store_stream(a.part_lse + static_cast<long>(split) * a.total_rows + grow, lse);
    return;
  }
  uint16_t* out = static_cast<uint16_t*>(a.out) + grow * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d = 32 * dt + 8 * qd + 4 * half;
      *reinterpret_cast<uint2*>(out + d) =
          make_uint2(pack2_bf16(acc[dt][4 * qd] * inv, acc[dt][4 * qd + 1] * inv),
                     pack2_bf16(acc[dt][4 * qd + 2] * inv, acc[dt][4 * qd + 3] * inv));
    }
  if (a.lse != nullptr && half == 0) a.lse[grow] = lse;
}

// Work items as run_work_items hands them out (kQueued: persistent, from the queues).
template <bool kQueued, int kMode>
__global__ void __launch_bounds__(kTL, 2) k_attn_long(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  run_work_items<kQueued>(a, reinterpret_cast<int*>(smem + Layout<kMode>::mask_off + 8),
                 [](const AttnArgs& args, int die, int k_slot) __attribute__((always_inline)) {
                   long_item<kMode>(args, die, k_slot);
                 });
}

void set_attn_long_attributes() {
  // the dynamic LDS above 64 KB must be allowed once per function and device, before
  // the first launch (and outside any stream capture)
  static std::mutex mu;
  static uint32_t done = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 32) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (done & (1u << dev)) return;
  const void* fns[6] = {reinterpret_cast<const void*>(&k_attn_long<false, kModeBf16>),
                        reinterpret_cast<const void*>(&k_attn_long<true, kModeBf16>),
                        reinterpret_cast<const void*>(&k_attn_long<false, kModeFp8>),
                        reinterpret_cast<const void*>(&k_attn_long<true, kModeFp8>),
                        reinterpret_cast<const void*>(&k_attn_long<false, kModeMma8>),
                        reinterpret_cast<const void*>(&k_attn_long<true, kModeMma8>)};
  const int bytes[6] = {kSmemL, kSmemL, kSmemL, kSmemL, kSmem8, kSmem8};
  for (int i = 0; i < 6; ++i)
    (void)hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, bytes[i]);
  done |= 1u << dev;
}

int launch_attn_long(const AttnArgs& a, hipStream_t s) {
  set_attn_long_attributes();
  const bool queued = a.queue != nullptr;
  const int mode = a.kt8 != nullptr ? kModeMma8 : (a.k_scale != nullptr ? kModeFp8 : kModeBf16);
  const dim3 grid(queued ? kCUs : 8 * ceil_div(a.batch * a.hkv, 8) * a.row_tiles * a.splits);
  if (mode == kModeMma8) {
    if (queued)
      hipLaunchKernelGGL((k_attn_long<true, kModeMma8>), grid, dim3(kTL), kSmem8, s, a);
    else
      hipLaunchKernelGGL((k_attn_long<false, kModeMma8>), grid, dim3(kTL), kSmem8, s, a);
  } else if (mode == kModeFp8) {
    if (queued)
      hipLaunchKernelGGL((k_attn_long<true, kModeFp8>), grid, dim3(kTL), kSmemL, s, a);
    else
      hipLaunchKernelGGL((k_attn_long<false, kModeFp8>), grid, dim3(kTL), kSmemL, s, a);
  } else if (queued) {
    hipLaunchKernelGGL((k_attn_long<true, kModeBf16>), grid, dim3(kTL), kSmemL, s, a);
  } else {
    hipLaunchKernelGGL((k_attn_long<false, kModeBf16>), grid, dim3(kTL), kSmemL, s, a);
  }
  const int st = check_launch("tree_verify_attention/long");
  if (st != TV_OK || a.splits == 1) return st;
  return launch_attn_combine(a, s);
}

// ---- dispatch order of the long work items: the (sequence, KV head) pairs
// ranked by estimated cost, largest first (longest-processing-time-first list
// scheduling: each free compute unit takes the next item of its die's list).
// Cost of a pair = its tiles x its live 64-row units summed over its row tiles, from
// the same clamped lengths the attention kernel uses.  Key of pair p = cost << 32 |
// ~p: keys are distinct, so the position of p in the list (larger costs first, equal
// costs in index order) is the number of keys above its own.  Every workgroup puts
// all keys in LDS and four adjacent threads count for one pair, thread q of the four
// over keys q, q + 4, q + 8, ... (so a wavefront reads four adjacent keys per step,
// in different banks, each a broadcast to 16 lanes), eight loads in flight per
// thread; the four counts are summed across the lanes.  The ranks need no sort
// network and no barrier past the first.
constexpr int kOrderThreads = 256;
constexpr int kOrderSplit = 4;                                  // threads per pair
constexpr int kOrderPairsPerWG = kOrderThreads / kOrderSplit;   // pairs ranked per workgroup
static_assert(64 % kOrderSplit == 0 && kOrderThreads % 64 == 0, "a pair's threads share a wavefront");

__device__ __forceinline__ uint64_t pair_cost_key(const AttnArgs& a, int p) {
  const int b = p / a.hkv;
  const int n0 = a.cu_nodes[b];
  const int count = max(0, min(a.cu_nodes[b + 1] - n0, a.max_nodes));
  const int plen = max(0, min(a.prefix_len[b], min(a.max_prefix, a.max_blocks * 64)));
  const int tiles = (plen + kKT - 1) / kKT + (count + 63) / 64;
  const int rows = a.group * count;
  int units = 0;
  for (int t = 0; t < a.row_tiles; ++t) {
    const int live = rows - t * kMfmaRowsPerWG;
    if (live > 0) units += (min(live, kMfmaRowsPerWG) + 63) / 64;
  }
  const uint32_t cost = static_cast<uint32_t>(tiles) * static_cast<uint32_t>(units);
  return (static_cast<uint64_t>(cost) << 32) | static_cast<uint32_t>(~p);
}

__global__ void __launch_bounds__(kOrderThreads) k_attn_order(AttnArgs a, int* order) {
  __shared__ uint64_t s_key[kMaxOrderedPairs];
  const int pairs = a.batch * a.hkv;
  for (int p = threadIdx.x; p < pairs; p += kOrderThreads) s_key[p] = pair_cost_key(a, p);
  __syncthreads();
  const int q = threadIdx.x % kOrderSplit;
  const int p = blockIdx.x * kOrderPairsPerWG + threadIdx.x / kOrderSplit;
  const bool live = p < pairs;  // dead threads still take part in the lane sums below
  const uint64_t mine = s_key[live ? p : 0];
  int c0 = 0, c1 = 0;
  int i = q;
  for (; i + 7 * kOrderSplit < pairs; i += 8 * kOrderSplit) {
    uint64_t k[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) k[j] = s_key[i + j * kOrderSplit];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      c0 += k[j] > mine;
      c1 += k[j + 1] > mine;
    }
  }
  for (; i < pairs; i += kOrderSplit) c0 += s_key[i] > mine;
  int above = c0 + c1;
  above += __shfl_xor(above, 1);
  above += __shfl_xor(above, 2);
  if (live && q == 0) order[above] = p;
}

int launch_attn_order(const AttnArgs& a, int* order, hipStream_t s) {
  const int pairs = a.batch * a.hkv;
  if (pairs < 1 || pairs > kMaxOrderedPairs) return TV_EINVAL;
  hipLaunchKernelGGL(k_attn_order, dim3((pairs + kOrderPairsPerWG - 1) / kOrderPairsPerWG),
                     dim3(kOrderThreads), 0, s, a, order);
  return check_launch("tree_verify_attention/order");
}

}  // namespace tv
