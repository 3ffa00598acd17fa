// Internal interface between the tree-attention entry point and its kernels.
#pragma once

#include "tv_common.h"

namespace tv {

// Everything a tree-attention kernel reads, by value.
struct AttnArgs {
  const void* q;            // [total_nodes, hq, D]
  const void* k_cache;      // [num_blocks, hkv, 64, D]
  const void* v_cache;
  const int32_t* block_table;  // [batch, max_blocks]
  const int32_t* prefix_len;   // [batch]
  const void* k_tree;       // [total_nodes, hkv, D]
  const void* v_tree;
  const int32_t* cu_nodes;  // [batch + 1]
  const uint64_t* anc;      // [total_nodes, words]
  void* out;                // [total_nodes, hq, D]
  float* lse;               // [total_nodes, hq] or null
  float* part_o;            // [splits, total_rows, D] fp32 (split-KV partials)
  float* part_lse;          // [splits, total_rows]
  int32_t* err;
  const int* pair_order;    // [batch * hkv] (sequence, KV head) pairs, longest first; or null
  const float* k_scale;     // FP8 prefix cache: [num_blocks, hkv, 64] scales; null for bf16
  const float* v_scale;
  int* queue;               // persistent launch: [8] queue heads (one per die), exit count
  int* tickets;             // in-kernel merge: one finish ticket per cut work item
  int words, batch, total_nodes, total_rows, max_nodes, max_prefix;
  int num_blocks, max_blocks, hq, hkv, group;
  int splits, blocks_per_split, row_tiles, total_work;
  // tail balancing (pipelined kernel, splits == 1): per die, work items
  // [0, tail_whole) run whole and the next tail_items are cut into tail_pieces
  // prefix ranges each, merged by the piece that finishes last (1 = off)
  int tail_pieces, tail_whole, tail_items;
  int die_slots;            // queue slots per die (persistent launch)
  float scale;              // softmax scale (natural-exp units)
  // FP8 matrix-core mode (null otherwise): the paged cache's E8M0 row exponents and
  // the tree's K/V in the same format (E4M3 codes, E8M0 exponents)
  const uint8_t* k_exp;     // [num_blocks, hkv, 64]
  const uint8_t* v_exp;
  const uint8_t* kt8;       // [total_nodes, hkv, 128]
  const uint8_t* vt8;
  const uint8_t* kt_e;      // [total_nodes, hkv]
  const uint8_t* vt_e;
};

// Kernel arguments sit in memory, and each first use of a field would otherwise
// wait for its own scalar load; naming them all at entry requests them together,
// one memory round trip for the whole argument block.  The asm writes 0 (callers
// add it to an index) and has no memory effects, so later loads keep the scalar path.
__device__ __forceinline__ int fetch_args(const AttnArgs& a) {
  int zero;
  asm("s_mov_b32 %0, 0"
      : "=s"(zero)
      : "s"(a.q), "s"(a.k_cache), "s"(a.v_cache), "s"(a.block_table), "s"(a.prefix_len),
        "s"(a.k_tree), "s"(a.v_tree), "s"(a.cu_nodes), "s"(a.anc), "s"(a.err), "s"(a.pair_order),
        "s"(a.words), "s"(a.batch), "s"(a.max_nodes), "s"(a.max_prefix), "s"(a.num_blocks),
        "s"(a.max_blocks), "s"(a.hq), "s"(a.hkv), "s"(a.group), "s"(a.splits),
        "s"(a.blocks_per_split), "s"(a.row_tiles), "s"(a.total_work), "s"(a.scale),
        "s"(a.tail_pieces), "s"(a.tail_whole), "s"(a.tail_items), "s"(a.die_slots));
  return zero;
}

// Six 32-bit words through the scalar path, all six requests in flight at once
// (one memory round trip); the addresses must be uniform across the wavefront.
__device__ __forceinline__ void load_words6(const int32_t* p0, const int32_t* p1, const int32_t* p2,
                                            const int32_t* p3, const int32_t* p4, const int32_t* p5,
                                            int& v0, int& v1, int& v2, int& v3, int& v4, int& v5) {
  asm volatile(
      "s_load_dword %0, %6, 0x0\n\t"
      "s_load_dword %1, %7, 0x0\n\t"
      "s_load_dword %2, %8, 0x0\n\t"
      "s_load_dword %3, %9, 0x0\n\t"
      "s_load_dword %4, %10, 0x0\n\t"
      "s_load_dword %5, %11, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(v0), "=&s"(v1), "=&s"(v2), "=&s"(v3), "=&s"(v4), "=&s"(v5)
      : "s"(p0), "s"(p1), "s"(p2), "s"(p3), "s"(p4), "s"(p5)
      : "memory");
}

// How one launch is laid out; the same function sizes the workspace.
struct AttnPlan {
  bool mfma;          // bf16, head_dim 128: matrix-core kernel; else the vector kernel
  bool long_items;    // pipelined matrix-core kernel for work items of many tiles
  bool ordered;       // long items dispatched longest (sequence, KV head) first
  int splits;         // prefix split across workgroups (1 = no combine pass)
  int blocks_per_split;
  int row_tiles;      // row tiles per (sequence, kv head)
  long total_work;    // workgroups with work
  bool persistent;    // long items over several rounds: one workgroup per CU pulls items
  bool merge_in_kernel;  // cut items merged by the piece that finishes last (no combine pass)
  int die_slots;      // queue slots per die
  int tail_pieces;    // tail balancing: pieces per tail item (1 = off)
  int tail_whole;     // per die: work items that run whole
  int tail_items;     // per die: work items cut into tail_pieces pieces
  size_t workspace;   // bytes: counter words, partials, pair order
  size_t part_off, lse_off, order_off;  // workspace offsets
};

// cache formats of the matrix-core plans
constexpr int kKvBf16 = 0;    // the dtype of q
constexpr int kKvFp8 = 1;     // E4M3 with fp32 row scales
constexpr int kKvMma8 = 2;    // E4M3 with E8M0 row exponents, on the FP8 matrix cores

// Counter words at the start of the workspace (zero between calls).
constexpr int kCounterBytes = 2048;
constexpr int kQueueWord = 0;        // [8] queue heads, [8] exit count of a persistent launch
constexpr int kTicketWord = 16;      // finish tickets from here
constexpr int kMaxTickets = kCounterBytes / 4 - kTicketWord;

AttnPlan plan_attention(int batch, int total_nodes, int max_nodes, int max_prefix, int hq, int hkv,
                        int head_dim, int dtype, int kv_format);

int launch_attn_vec(const AttnArgs& a, int head_dim, int dtype, hipStream_t s);
int launch_attn_mfma(const AttnArgs& a, hipStream_t s);
// allow the matrix-core kernels' dynamic LDS on the current device (idempotent; the
// launchers call them too, but a stream capture must not be the first caller)
void set_attn_mfma_attributes();
void set_attn_long_attributes();
int launch_attn_long(const AttnArgs& a, hipStream_t s);
int launch_attn_order(const AttnArgs& a, int* order, hipStream_t s);
int launch_attn_combine(const AttnArgs& a, hipStream_t s);

// Tail balancing: how many pieces to cut each of `tail` leftover work items into
// so that the last round on `cus` compute units ends soonest (1 = leave whole).
int tail_pieces_for(int tail, int cus);

constexpr int kMfmaRowsPerWG = 256;  // 8 waves x 32 rows
constexpr int kCUs = 256;
constexpr int kXCDs = 8;             // compute dies; workgroup i runs on die i % 8
constexpr int kCUsPerXCD = kCUs / kXCDs;
constexpr int kMaxTailPieces = 8;
constexpr int kMaxSplits = 16;       // prefix splits per (sequence, KV head, row tile)
// work items of at least this many 64-key tiles run the pipelined kernel
#ifndef TV_LONG_MIN_TILES
#define TV_LONG_MIN_TILES 4
#endif
constexpr int kLongMinTiles = TV_LONG_MIN_TILES;
constexpr int kMinSplitBlocks = 4;   // prefix blocks per split at least (when splitting)
constexpr int kMaxOrderedPairs = 2048;  // pairs the ordering kernel ranks (all keys in one LDS)

// Work items of a tree-attention launch.  Without a queue, workgroup i runs slot
// i / 8 of die i % 8's list (the hardware hands workgroups to dies round-robin in
// launch order).  With one (items over several rounds), one workgroup per compute
// unit takes slots from the queue of the die it runs on (the hardware die id) until
// it is empty, then from the other dies' queues: no unit idles while another die's
// dispatch waits, and no workgroup ever waits for another.  A slot is taken only
// when the workgroup is free (taking the next one ahead, while an item runs,
// reserves work for a busy unit: 64 sequences of 16-96 nodes, 267 -> 320 us).
// s_pull is one LDS word.
// kQueued false: the plain mapping only (no loop, so the item body keeps the
// registers it would have as a kernel of its own).
template <bool kQueued, class Item>
__device__ __forceinline__ void run_work_items(const AttnArgs& a, int* s_pull, Item item) {
  if constexpr (!kQueued) {
    item(a, static_cast<int>(blockIdx.x % kXCDs), static_cast<int>(blockIdx.x / kXCDs));
    return;
  }
  const bool queued = true;
  const int home = static_cast<int>(__builtin_amdgcn_s_getreg(20 | (3 << 11))) & (kXCDs - 1);
  int die = queued ? home : static_cast<int>(blockIdx.x % kXCDs);
  int k_slot = blockIdx.x / kXCDs, tried = 0;
  for (;;) {  // one call site of the item body (register pressure)
    if (queued) {
      if (threadIdx.x == 0) *s_pull = atomicAdd(a.queue + die, 1);
      __syncthreads();
      k_slot = *s_pull;
      __syncthreads();  // every lane has read the slot before lane 0 takes the next
      if (k_slot < 0 || k_slot >= a.die_slots) {
        if (++tried == kXCDs) break;
        die = (die + 1) & (kXCDs - 1);
        continue;
      }
    }
    // the item body reads its arguments afresh from the kernel-argument segment (the
    // pointer is opaque to the compiler), so that no argument stays in a scalar
    // register across items: the body alone needs nearly all of them
    const __attribute__((address_space(4))) char* ap =
        (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ap));
    const AttnArgs item_args = *(const AttnArgs*)ap;
    item(item_args, die, k_slot);
    if (!queued) break;
  }
  // the last workgroup to finish zeroes the queue heads and the exit count for the
  // next call (every other workgroup has taken its last slot before counting itself)
  if (queued && threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (atomicAdd(a.queue + kXCDs, 1) == static_cast<int>(gridDim.x) - 1) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      for (int d = 0; d <= kXCDs; ++d) a.queue[d] = 0;
    }
  }
}

}  // namespace tv
