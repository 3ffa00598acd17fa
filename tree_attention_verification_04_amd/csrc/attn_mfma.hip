// Matrix-core tree attention for gfx950: bf16 Q/K/V, head_dim 128, fp32 accumulation.
//
// Work unit: (sequence b, KV head g, row tile, prefix split).  The rows of one KV
// head are the G * N_b pairs (node, query head of the group), ordered node-major;
// a workgroup of 8 wavefronts takes 256 of them, 32 per wavefront.  It streams the
// prefix of sequence b through the block table, one 64-token paged block at a
// time, and then the 64-node tiles of the tree that any of its rows can see.  Each
// tile is staged once in LDS and used by all 256 rows: the shared prefix is read
// once per tile for every node of the tree (page "端侧多模态大模型推测解码草稿模型动态剪枝：
// 详解基于重要性采样的树形验证并行加速策略" (ufo.work/2026/500), §3.2: common prefix kept
// once and reused; all branches flattened into one launch).
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: a lane
// then holds 16 keys of a single row per 32-key sub-tile, so the row max needs one
// cross-lane exchange (lane ^ 32) and the row sum none until the end.  The K rows
// fed to the MFMA are permuted (4-row groups 1<->2 and 5<->6 of every 32) so that
// the accumulator registers of a lane hold 8 consecutive keys per 16-key step; the
// probabilities are packed to bf16 and used directly as the B operand of
// O^T = V^T P^T.  V stays in LDS as [key][d]; its A operand comes from the gfx950
// LDS transpose read (ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives
// element i%4 of the 8-byte loads of lanes i/4, 4+i/4, 8+i/4, 12+i/4), so each lane
// gets 4 consecutive keys of one d per read.  Online softmax with running max and
// sum in fp32 (page "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力机制与显存
// 碎片整理联合加速" (ufo.work/2026/537), appendix B: running max m, sum l, rescale by
// exp(m_old - m_new), bf16 probabilities into the P.V product); the tree mask M_tree
// (same page, §2.2.2) comes from the 64-bit ancestor word of the row's node.
//
// LDS holds two stages of (K tile, V tile), 64 rows of 256 B each, unpadded; the
// 16-byte chunks of a row are XOR-swizzled (K by key & 15, V by (key & 3) << 2) so
// that the MFMA operand reads and the staging writes are free of bank conflicts.
// Tiles are prefetched two ahead: tile it+2 is loaded into registers during
// iteration it, tile it+1 (loaded one iteration earlier) is written to the other
// stage after the matrix work; one barrier per tile.  Work indices are remapped so
// that the workgroups sharing a (sequence, KV head, split) land on the same XCD and
// hit its L2 for the shared K/V tiles.
#include <mutex>

#include "mfma_tile.h"

namespace tv {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
static_assert(kMfmaRowsPerWG == kWaves * 32, "row tile is 32 rows per wavefront");

using TileRegs = TileRegsT<kThreads>;

// kFp8: the paged prefix cache holds E4M3 bytes with one scale per (block, KV
// head, position); its tiles are dequantized to bf16 on their way into LDS and
// everything after that is the bf16 kernel.
template <bool kFp8>
__device__ __forceinline__ void mfma_item(const AttnArgs& a, const int die, const int k_slot) {
  auto load_tile = [](const TileSrc& src, int tid, TileRegs& r) __attribute__((always_inline)) {
    load_tile_t<kThreads, kFp8>(src, tid, r);
  };
  auto store_tile = [](char* stage, uint64_t* anc_slot, int tid, TileRegs& r, int nvalid)
      __attribute__((always_inline)) { store_tile_t<kThreads, kFp8>(stage, anc_slot, tid, r, nvalid); };
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint32_t* s_tree_mask = reinterpret_cast<uint32_t*>(smem + kAncOff + 3 * kAncBytes);
  int* s_simd_slots = reinterpret_cast<int*>(smem + kAncOff + 3 * kAncBytes + 16);  // [4]

  // ---- work item (XCD-aware: each die runs a contiguous range of work indices)
  const int work = die * a.die_slots + k_slot;
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

  // ---- this lane's row and its Q fragment (B operand of S^T = K Q^T); issued early
  // Waves map to (row group rg, key group kg): with R live 32-row groups in this
  // tile, wave w takes rows rg = w % R and key group kg = w / R.  The pipelined
  // path uses key group 0 only; short work items spread their tiles over the key
  // groups and merge the partial softmax states at the end.
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  const int n_rg = min(kWaves, (rows - r0 + 31) / 32);
  const int rg = wave % n_rg, kg = wave / n_rg;
  const int r = r0 + rg * 32 + col;
  const bool row_ok = r < rows;
  const int node = row_ok ? r / a.group : 0;
  const int head = g * a.group + (row_ok ? r % a.group : 0);
  const long grow = static_cast<long>(n0 + node) * a.hq + head;  // global row (node, head)
  bool wave_live = kg == 0;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + grow * kD + half * 8;
  bf16x8_t qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = as_bf16x8(row_ok ? *reinterpret_cast<const uint4*>(qp + s * 16) : make_uint4(0, 0, 0, 0));

  // ---- which 64-node tree tiles any row of this workgroup can see
  if (tid == 0) *s_tree_mask = 0;
  if (tid < 4) s_simd_slots[tid] = 0;
  __syncthreads();
  const int ntw = (count + 63) / 64;
  if (do_tree) {
    const int lo = r0 / a.group;
    const int hi = (min(rows, r0 + kMfmaRowsPerWG) - 1) / a.group;
    const int pairs_n = (hi - lo + 1) * ntw;
    uint32_t m = 0;
    for (int i = tid; i < pairs_n; i += kThreads) {
      const int nd = lo + i / ntw, t = i % ntw;
      if (a.anc[static_cast<long>(n0 + nd) * a.words + t] != 0) m |= 1u << t;
    }
    if (m) atomicOr(s_tree_mask, m);
  }
  __syncthreads();
  const uint32_t tree_mask = do_tree ? *s_tree_mask : 0u;
  const int n_tiles = n_prefix_tiles + __popc(tree_mask);

  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const uint16_t* kt = static_cast<const uint16_t*>(a.k_tree);
  const uint16_t* vt = static_cast<const uint16_t*>(a.v_tree);

  // tile it -> kind (0 prefix block, 1 tree tile) and base (first key, or tree word)
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
  // block-table entries through the scalar (constant) path: uniform, read-only
  const __attribute__((address_space(4))) int32_t* bt_row =
      (const __attribute__((address_space(4))) int32_t*)(a.block_table) +
      static_cast<long>(b) * a.max_blocks;
  // the ancestor-word row of this thread's staging row (tid & 255 of the 256 rows)
  const int stage_node = min((r0 + (tid & (kMfmaRowsPerWG - 1))) / a.group, count - 1);
  const uint64_t* stage_anc = a.anc + static_cast<long>(n0 + stage_node) * a.words;
  auto tile_src = [&](int it) __attribute__((always_inline)) -> TileSrc {
    int kind, base;
    tile_kind(it, kind, base);
    TileSrc s;
    s.anc = stage_anc + (kind == 1 ? base : 0);
    s.ks = nullptr;
    s.vs = nullptr;
    if (kind == 0) {
      // an FP8 row is 128 bytes: 64 16-bit units
      constexpr int kRowUnits = kFp8 ? kD / 2 : kD;
      const int blk = bt_row[base / kKT];
      if (kFp8) {
        s.ks = a.k_scale;
        s.vs = a.v_scale;
      }
      if (blk < 0 || blk >= a.num_blocks) {
        if (tid == 0) atomicOr(a.err, TV_ERR_BLOCK);
        s.k = kc;
        s.v = vc;
        s.row_stride = kRowUnits;
        s.nvalid = 0;
        return s;
      }
      const long row0 = (static_cast<long>(blk) * a.hkv + g) * kKT;  // first (block, head) row
      s.k = kc + row0 * kRowUnits;
      s.v = vc + row0 * kRowUnits;
      if (kFp8) {
        s.ks = a.k_scale + row0;
        s.vs = a.v_scale + row0;
      }
      s.row_stride = kRowUnits;
      s.nvalid = min(kKT, plen - base);
    } else {
      const long off = (static_cast<long>(n0 + base * 64) * a.hkv + g) * kD;
      s.k = kt + off;
      s.v = vt + off;
      s.row_stride = static_cast<long>(a.hkv) * kD;
      s.nvalid = min(64, count - base * 64);
    }
    return s;
  };

  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float c2 = a.scale * kLog2e;
  const int krow0 = key_perm(col);

  // per-lane LDS offsets of the S^T A operand (K) for the two 32-key sub-tiles
  int k_base[2];
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) k_base[sg] = (32 * sg + krow0) * 256;
  const int k_xor = krow0 & 15;  // (32 sg + krow0) & 15 == krow0 & 15
  // per-lane LDS offsets of the transposed V reads, one per 32-wide d-tile
  const int grp = lane >> 4, jg = lane & 15, hh = grp >> 1;
  const int low = 2 * (grp & 1) + ((jg & 3) >> 1);
  int v_base[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    v_base[dt] = kTileBytes + (8 * hh + (jg >> 2)) * 256 + ((((dt ^ (jg >> 2)) << 2) + low) << 4) +
                 8 * (jg & 1);

  f32x16_t sacc[2];   // S^T of the tile between its score MFMAs and its softmax
  uint32_t pk[2][8];  // bf16 probabilities between the softmax and the P.V MFMAs

  // scores of tile it: S^T = K Q^T
  auto mfma_scores = [&](const char* stage) __attribute__((always_inline)) {
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      sacc[sg] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int c = 2 * s + half;
        const bf16x8_t kf =
            as_bf16x8(*reinterpret_cast<const uint4*>(stage + k_base[sg] + ((c ^ k_xor) << 4)));
        sacc[sg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[sg], 0, 0, 0);
      }
    }
    // keep the K reads four MFMAs ahead of their use
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
  };
  // O^T += V^T P^T for the tile whose probabilities are in pk
  auto mfma_pv = [&](const char* stage) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sg = j >> 1, vb = (j & 1) * 4;
      const bf16x8_t pf =
          as_bf16x8(make_uint4(pk[sg][vb], pk[sg][vb + 1], pk[sg][vb + 2], pk[sg][vb + 3]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const char* p = stage + v_base[dt] + 16 * j * 256;
        const bf16x4_t lo = ds_read_tr(p);
        const bf16x4_t hi = ds_read_tr(p + 4 * 256);
        const bf16x8_t vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[dt], 0, 0, 0);
      }
    }
    // keep the transposed V reads four MFMAs ahead of their use
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  // mask, online-softmax update, bf16 probabilities of tile it
  auto softmax = [&](int kind, int base, const uint64_t* anc_slot) __attribute__((always_inline)) {
    // key index of register v of sub-tile sg is 32sg + 16(v/8) + 8*half + v%8
    const bool full = kind == 0 && plen - base >= kKT;
    if (!full) {
      const uint64_t vis = kind == 0 ? ((1ull << (plen - base)) - 1ull)
                                     : (row_ok ? anc_slot[rg * 32 + col] : 0ull);
      // the 32 keys this lane holds, compressed so that register (sg, v) is bit 16sg + v
      const uint32_t lo = static_cast<uint32_t>(vis), hi = static_cast<uint32_t>(vis >> 32);
      const int sh = 8 * half;
      const uint32_t w = ((lo >> sh) & 0xffu) | (((lo >> (16 + sh)) & 0xffu) << 8) |
                         (((hi >> sh) & 0xffu) << 16) | (((hi >> (16 + sh)) & 0xffu) << 24);
#pragma unroll
      for (int sg = 0; sg < 2; ++sg)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          sacc[sg][v] = ((w >> (16 * sg + v)) & 1u) ? sacc[sg][v] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sg = 0; sg < 2; ++sg)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[sg][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float mc = m_use * c2;
    if (__ballot(m_new != m_run)) {  // rescale only when some row's max moved
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] *= alpha;
    }
    m_run = m_new;
    float psum = 0.0f;
#pragma unroll
    for (int sg = 0; sg < 2; ++sg)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float p0 = __builtin_amdgcn_exp2f(sacc[sg][v] * c2 - mc);
        const float p1 = __builtin_amdgcn_exp2f(sacc[sg][v + 1] * c2 - mc);
        psum += p0 + p1;
        pk[sg][v >> 1] = pack2_bf16(p0, p1);
      }
    l_run += psum;
  };

  // ---- ping-pong schedule.  Waves 0-3 (group A) and 4-7 (group B) sit on the
  // same four SIMDs, one of each per SIMD.  Phases alternate: while one group
  // runs its matrix phase (P.V of tile i-1, then the scores of tile i) the other
  // runs the softmax of its previous tile on the vector ALU, so the two kinds of
  // work overlap on every SIMD.  Group A runs the matrix phase of tile i in phase
  // 2i and the softmax of tile i in phase 2i+1; group B runs one phase later.
  // Tile i lives in LDS stage i % 3 from phase 2i-2 (written) to phase 2i+3 (last
  // read).  Phase 2i writes tile i+1 from its registers; phase 2i+1 issues the
  // loads of tile i+3 into the register set just freed.  One barrier per phase.
  // One wave of each group per SIMD: waves take turns per SIMD (SIMD id from the
  // HW_ID register, bits 5:4); any assignment is correct, this one overlaps best.
  int slot = 0;
  if (lane == 0) slot = atomicAdd(&s_simd_slots[__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4) & 3], 1);
  const bool group_b = __shfl(slot, 0, 64) & 1;
  TileRegs r0s, r1s;       // register sets: set (i % 2) carries tiles i, i+2, ...
  int nv0 = 0, nv1 = 0;
  auto stage_of = [&](int i) __attribute__((always_inline)) -> char* { return smem + (i % 3) * kStageBytes; };
  auto anc_of = [&](int i) __attribute__((always_inline)) -> uint64_t* {
    return reinterpret_cast<uint64_t*>(smem + kAncOff + (i % 3) * kAncBytes);
  };
  auto matrix_phase = [&](int i) __attribute__((always_inline)) {  // P.V of tile i-1, scores of tile i
    if (i >= 1 && i - 1 < n_tiles) mfma_pv(stage_of(i - 1));
    __builtin_amdgcn_sched_barrier(0);  // keep the two MFMA chains' operand reads apart
    if (i < n_tiles) {
      mfma_scores(stage_of(i));
    }
  };
  auto vector_phase = [&](int i) __attribute__((always_inline)) {
    if (i >= 0 && i < n_tiles) {
      int kind, base;
      tile_kind(i, kind, base);
      softmax(kind, base, anc_of(i));
    }
  };
  auto compute_phase = [&](int p) __attribute__((always_inline)) {
    if (!wave_live) return;
    if (!group_b) {
      if ((p & 1) == 0) matrix_phase(p >> 1);
      else vector_phase(p >> 1);
    } else {
      if (p & 1) matrix_phase(p >> 1);
      else vector_phase((p >> 1) - 1);
    }
  };

  if (n_tiles > 0 && n_tiles <= 3) {
    // Short work items (a split of a short verify): all tiles fit the three
    // stages, so they are staged once and every live wave runs them back to back
    // with no further barrier.
    TileRegs r2s;  // all three tiles in flight at once: one memory round trip
    const TileSrc s0 = tile_src(0);
    const TileSrc s1 = tile_src(min(1, n_tiles - 1));
    const TileSrc s2 = tile_src(min(2, n_tiles - 1));
    load_tile(s0, tid, r0s);
    load_tile(s1, tid, r1s);
    load_tile(s2, tid, r2s);
    store_tile(stage_of(0), anc_of(0), tid, r0s, s0.nvalid);
    if (n_tiles > 1) store_tile(stage_of(1), anc_of(1), tid, r1s, s1.nvalid);
    if (n_tiles > 2) store_tile(stage_of(2), anc_of(2), tid, r2s, s2.nvalid);
    __syncthreads();
    const int n_kg = min(kWaves / n_rg, n_tiles);  // key groups that get a tile
    if (kg < n_kg) {
      for (int i = kg; i < n_tiles; i += n_kg) {
        int kind, base;
        tile_kind(i, kind, base);
        mfma_scores(stage_of(i));
        softmax(kind, base, anc_of(i));
        mfma_pv(stage_of(i));
      }
    }
    if (n_kg > 1) {
      // merge key groups 1.. into key group 0 through LDS (the stages are free now):
      //   m = max_k m_k,  l = sum_k l_k e^{m_k - m},  acc = sum_k acc_k e^{m_k - m}
      __syncthreads();
      float* slot = reinterpret_cast<float*>(smem) + ((kg - 1) * n_rg + rg) * (66 * 64);
      if (kg >= 1 && kg < n_kg) {
        slot[lane] = m_run;
        slot[64 + lane] = l_run;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) slot[128 + (dt * 16 + v) * 64 + lane] = acc[dt][v];
      }
      __syncthreads();
      if (kg == 0) {
        for (int k = 1; k < n_kg; ++k) {
          const float* o = reinterpret_cast<const float*>(smem) + ((k - 1) * n_rg + rg) * (66 * 64);
          const float mk = o[lane], lk = o[64 + lane];
          const float m_new = fmaxf(m_run, mk);
          const float m_use = m_new == -INFINITY ? 0.0f : m_new;
          const float a0 = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
          const float a1 = __builtin_amdgcn_exp2f((mk - m_use) * c2);
          l_run = l_run * a0 + lk * a1;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              acc[dt][v] = acc[dt][v] * a0 + o[128 + (dt * 16 + v) * 64 + lane] * a1;
          m_run = m_new;
        }
      }
    }
  } else if (n_tiles > 3) {
    const TileSrc s0 = tile_src(0);
    load_tile(s0, tid, r0s);
    nv0 = s0.nvalid;
    const TileSrc s1 = tile_src(min(1, n_tiles - 1));
    load_tile(s1, tid, r1s);
    nv1 = s1.nvalid;
    store_tile(stage_of(0), anc_of(0), tid, r0s, nv0);
    const TileSrc s2 = tile_src(min(2, n_tiles - 1));
    load_tile(s2, tid, r0s);
    nv0 = s2.nvalid;
    __syncthreads();
    // phases 4k .. 4k+3 cover tiles i = 2k (phases 4k, 4k+1) and 2k+1.  Every
    // iteration has the same memory operations in the same order (loads past the
    // last tile re-read it), so the waits before each LDS write cover only the
    // older register set; phases past the last one compute nothing.
    const int n_iter = (2 * n_tiles + 2 + 3) / 4;
    for (int k = 0; k < n_iter; ++k) {
      const int i0 = 2 * k, i1 = 2 * k + 1;
      if (i0 + 1 < n_tiles) store_tile(stage_of(i0 + 1), anc_of(i0 + 1), tid, r1s, nv1);
      compute_phase(4 * k);
      __syncthreads();
      {
        const TileSrc sn = tile_src(min(i0 + 3, n_tiles - 1));
        load_tile(sn, tid, r1s);
        nv1 = sn.nvalid;
      }
      compute_phase(4 * k + 1);
      __syncthreads();
      if (i1 + 1 < n_tiles) store_tile(stage_of(i1 + 1), anc_of(i1 + 1), tid, r0s, nv0);
      compute_phase(4 * k + 2);
      __syncthreads();
      {
        const TileSrc sn = tile_src(min(i1 + 3, n_tiles - 1));
        load_tile(sn, tid, r0s);
        nv0 = sn.nvalid;
      }
      compute_phase(4 * k + 3);
      __syncthreads();
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse = l_tot > 0.0f ? m_run * a.scale + logf(l_tot) : -INFINITY;
  // register v of d-tile dt holds d = 32dt + 8(v/4) + 4*half + v%4
  if (kg != 0) return;  // other key groups were merged into key group 0
  if (a.splits == 1) {
    if (!row_ok) return;
    uint16_t* out = static_cast<uint16_t*>(a.out) + grow * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d = 32 * dt + 8 * qd + 4 * half;
        const uint2 w = make_uint2(pack2_bf16(acc[dt][4 * qd] * inv, acc[dt][4 * qd + 1] * inv),
                                   pack2_bf16(acc[dt][4 * qd + 2] * inv, acc[dt][4 * qd + 3] * inv));
        *reinterpret_cast<uint2*>(out + d) = w;
      }
    if (a.lse != nullptr && half == 0) a.lse[grow] = lse;
    return;
  }

  // ---- split prefix: write this split's normalised partial and its log-sum-exp;
  // k_attn_combine merges the splits after the kernel ends
  if (!row_ok) return;
  float* po = a.part_o + (static_cast<long>(split) * a.total_rows + grow) * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d = 32 * dt + 8 * qd + 4 * half;
      store_stream4(po + d, acc[dt][4 * qd] * inv, acc[dt][4 * qd + 1] * inv,
                    acc[dt][4 * qd + 2] * inv, acc[dt][4 * qd + 3] * inv);
    }
  if (half == 0) store_stream(a.part_lse + static_cast<long>(split) * a.total_rows + grow, lse);
}

// Work items as run_work_items hands them out (kQueued: persistent, from the queues).
template <bool kFp8, bool kQueued>
__global__ void __launch_bounds__(kThreads) k_attn_mfma(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  run_work_items<kQueued>(a, reinterpret_cast<int*>(smem + kAncOff + 3 * kAncBytes + 48),
                 [](const AttnArgs& args, int die, int k_slot) __attribute__((always_inline)) {
                   mfma_item<kFp8>(args, die, k_slot);
                 });
}

// Merge of the prefix splits, one thread per (row, 4 consecutive d):
//   lse = log sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) * out_s
// All splits' values are loaded before any is used (one memory round trip); kS is
// the split count rounded up to an instance (2, 4, 5, 8 or 16; 5 is a short verify
// with a 17-block prefix), the loads past the last split re-read it and get weight
// zero.
template <int kS>
__global__ void __launch_bounds__(256) k_attn_combine(AttnArgs a) {
  int zero;
  asm("s_mov_b32 %0, 0"
      : "=s"(zero)
      : "s"(a.part_o), "s"(a.part_lse), "s"(a.out), "s"(a.lse), "s"(a.total_rows), "s"(a.splits));
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x + zero;
  if (idx >= static_cast<long>(a.total_rows) * (kD / 4)) return;
  const long gr = idx / (kD / 4);
  const int d4 = static_cast<int>(idx % (kD / 4));
  float ls[kS];
  float4 ps[kS];
#pragma unroll
  for (int sp = 0; sp < kS; ++sp) {
    const long at = static_cast<long>(min(sp, a.splits - 1)) * a.total_rows + gr;
    ls[sp] = a.part_lse[at];
    ps[sp] = *reinterpret_cast<const float4*>(a.part_o + at * kD + 4 * d4);
  }
#pragma unroll
  for (int sp = 0; sp < kS; ++sp)
    if (sp >= a.splits) ls[sp] = -INFINITY;
  float mx = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kS; ++sp) mx = fmaxf(mx, ls[sp]);
  const float mref = mx == -INFINITY ? 0.0f : mx;
  float w_sum = 0.0f;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int sp = 0; sp < kS; ++sp) {
    const float w = __builtin_amdgcn_exp2f((ls[sp] - mref) * kLog2e);
    w_sum += w;
    o.x = fmaf(w, ps[sp].x, o.x);
    o.y = fmaf(w, ps[sp].y, o.y);
    o.z = fmaf(w, ps[sp].z, o.z);
    o.w = fmaf(w, ps[sp].w, o.w);
  }
  const float wi = w_sum > 0.0f ? 1.0f / w_sum : 0.0f;
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + gr * kD + 4 * d4) =
      make_uint2(pack2_bf16(o.x * wi, o.y * wi), pack2_bf16(o.z * wi, o.w * wi));
  if (a.lse != nullptr && d4 == 0) a.lse[gr] = w_sum > 0.0f ? mx + logf(w_sum) : -INFINITY;
}

void set_attn_mfma_attributes() {
  // the dynamic LDS above 64 KB must be allowed once per function and device, before
  // the first launch (and outside any stream capture)
  static std::mutex mu;
  static uint32_t done = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 32) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (done & (1u << dev)) return;
  const void* fns[4] = {reinterpret_cast<const void*>(&k_attn_mfma<false, false>),
                          reinterpret_cast<const void*>(&k_attn_mfma<false, true>),
                          reinterpret_cast<const void*>(&k_attn_mfma<true, false>),
                          reinterpret_cast<const void*>(&k_attn_mfma<true, true>)};
  for (const void* f : fns)
    (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
  done |= 1u << dev;
}

int launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  set_attn_mfma_attributes();
  const bool fp8 = a.k_scale != nullptr, queued = a.queue != nullptr;
  const dim3 grid(queued ? kCUs : 8 * a.die_slots), block(kThreads);
  if (fp8 && queued)
    hipLaunchKernelGGL((k_attn_mfma<true, true>), grid, block, kSmemBytes, s, a);
  else if (fp8)
    hipLaunchKernelGGL((k_attn_mfma<true, false>), grid, block, kSmemBytes, s, a);
  else if (queued)
    hipLaunchKernelGGL((k_attn_mfma<false, true>), grid, block, kSmemBytes, s, a);
  else
    hipLaunchKernelGGL((k_attn_mfma<false, false>), grid, block, kSmemBytes, s, a);
  const int st = check_launch("tree_verify_attention/mfma");
  if (st != TV_OK || a.splits == 1) return st;
  return launch_attn_combine(a, s);
}

int launch_attn_combine(const AttnArgs& a, hipStream_t s) {
  const long items = static_cast<long>(a.total_rows) * (kD / 4);
  const dim3 grid(static_cast<int>((items + 255) / 256)), block(256);
  static_assert(kMaxSplits == 16, "combine instances cover up to 16 splits");
  if (a.splits <= 2)
    hipLaunchKernelGGL(k_attn_combine<2>, grid, block, 0, s, a);
  else if (a.splits <= 4)
    hipLaunchKernelGGL(k_attn_combine<4>, grid, block, 0, s, a);
  else if (a.splits <= 5)  // a single short verify (17-block prefix: 5 splits of 4)
    hipLaunchKernelGGL(k_attn_combine<5>, grid, block, 0, s, a);
  else if (a.splits <= 8)
    hipLaunchKernelGGL(k_attn_combine<8>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(k_attn_combine<16>, grid, block, 0, s, a);
  return check_launch("tree_verify_attention/combine");
}

}  // namespace tv
