"""Accepted-path KV commit oracle: the plain definition (a copy), per sequence.

After acceptance, the keys and values of the accepted path become prefix
positions of the sequence: the next verify round reuses them as shared prefix
instead of recomputing them (page [P537] "端云协同推测解码中草稿模型动态生成与验证并行化…",
§5.2, prefix caching: the KV from the root to the branch point overlaps the
previous round's accepted path, so it is updated incrementally), and the
tree's slots return to the pool right after verification (page [P525]
"端侧大模型推测解码草稿模型动态剪枝策略…", §2.3.2, dynamic KV pool; §8.1, the
verify op returns the accepted length and the new KV indices).

Readings taken where the pages are silent:
  * the path is the one the acceptance step returns, root-level node first; node
    path[j] (local index) holds the keys/values of depth j+1, i.e. of position
    P_b + j, so they are written to prefix position P_b + j unchanged;
  * the paged cache must already map every logical block the new positions fall
    in (the caller reserves them; no block is allocated here); the sequence's
    prefix length grows by the accepted length;
  * a sequence whose path is invalid (accepted length outside [0, max_path], a
    path entry outside its nodes) or whose new positions are not mapped to a
    valid block gets the error bit and is left untouched;
  * a block the new positions fall in must be the sequence's own: prefix blocks
    may be shared by several sequences for reading (page [P537] §2.3.3, shared
    prefix pool), but when another sequence's table row also maps a destination
    block (anywhere in that row), writing it would change that sequence's
    prefix, so the commit sets the block error bit and leaves the sequence
    untouched (copying a shared block before writing is the caller's job).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .tree import ERR_BLOCK, ERR_PATH

BLOCK = 64


def commit_kv(k_cache, v_cache, block_table, prefix_len, num_blocks: int, k_tree, v_tree,
              cu_nodes, accept_len, path, max_path: int):
    """Returns (k_cache', v_cache', prefix_len', err) — new arrays, inputs untouched.

    k_cache/v_cache [num_blocks, hkv, 64, d]; block_table [batch, max_blocks];
    k_tree/v_tree [total_nodes, hkv, d]; path [batch, max_path] local node ids.
    """
    kc, vc = k_cache.copy(), v_cache.copy()
    plen_out = np.asarray(prefix_len).copy()
    err = 0
    max_blocks = block_table.shape[1]
    for b in range(len(cu_nodes) - 1):
        n0, n1 = int(cu_nodes[b]), int(cu_nodes[b + 1])
        length = int(accept_len[b])
        p0 = int(prefix_len[b])
        if length < 0 or length > max_path:
            err |= ERR_PATH
            continue
        nodes = [int(path[b, j]) for j in range(length)]
        if any(n < 0 or n >= n1 - n0 for n in nodes):
            err |= ERR_PATH
            continue
        positions = range(p0, p0 + length)
        if p0 < 0 or p0 + length > max_blocks * BLOCK:
            err |= ERR_BLOCK
            continue
        blocks = [int(block_table[b, t // BLOCK]) for t in positions]
        if any(blk < 0 or blk >= num_blocks for blk in blocks):
            err |= ERR_BLOCK
            continue
        others = {int(x) for o in range(len(cu_nodes) - 1) if o != b for x in block_table[o]}
        if any(blk in others for blk in blocks):
            err |= ERR_BLOCK
            continue
        for j, t in enumerate(positions):
            kc[blocks[j], :, t % BLOCK, :] = k_tree[n0 + nodes[j]]
            vc[blocks[j], :, t % BLOCK, :] = v_tree[n0 + nodes[j]]
        plen_out[b] = p0 + length
    return kc, vc, plen_out, err
