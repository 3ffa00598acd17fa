"""Tree-attention oracle: the plain definition, in fp64.

Every draft-tree node is a query.  Node n of sequence b, query head h, sees
  * every prefix position t < P_b of its sequence — the shared prefix is
    kept once and reused by every branch (page [P500]
    "端侧多模态大模型推测解码草稿模型动态剪枝…", §3.2, common-prefix merge),
    read through the paged block table (page [P525]
    "端侧大模型推测解码草稿模型动态剪枝策略…", §2.3.1);
  * every tree node j with M_tree[n, j] = 0, i.e. j is n or an ancestor of n
    (page [P537] "端云协同推测解码中草稿模型动态生成与验证并行化…", §2.2.2,
    equation M_tree); all other tree nodes are masked with -inf.
Scores are scale * <q, k>, softmax over the visible set, output the
softmax-weighted sum of the visible values (page [P537], appendix B: scaled
QK^T, masked, softmax, times V).  Readings taken where the pages are silent:
the scale is passed by the caller (1/sqrt(D) by default); query head h reads
KV head h // (Hq/Hkv); the whole prefix is visible to every node.

The ancestor sets come from explicit parent walks — not from bitsets — so
this oracle is independent of the tree-index step.  Evaluation order: one
(sequence, query head) at a time, a matrix product for the scores (numpy),
row max subtracted before exp.
"""
from __future__ import annotations

import numpy as np

from .tree import ancestors_or_self

BLOCK = 64


def kv_head(h: int, hq: int, hkv: int) -> int:
    """KV head read by query head h: consecutive query heads share a KV head."""
    return h // (hq // hkv)


def gather_prefix(cache: np.ndarray, block_table_row: np.ndarray, plen: int) -> np.ndarray:
    """Rows 0..plen-1 of one sequence's prefix: [plen, hkv, d], via the block table."""
    t = np.arange(plen)
    blk = block_table_row[t // BLOCK]
    return cache[blk, :, t % BLOCK, :]


def tree_attention(q, k_cache, v_cache, block_table, prefix_len, k_tree, v_tree, cu_nodes,
                   parent, hq: int, hkv: int, scale: float, nodes=None):
    """Tree attention over a batch of sequences.

    All float inputs are fp64 arrays holding the exact stored values.
    `nodes`, if given, is a list (one entry per sequence) of local node
    indices to evaluate; other rows of the result are NaN.

    Returns (out [total, hq, d] fp64, lse [total, hq] fp64) where
    lse = log(sum over the visible set of exp(score)).
    """
    total, _, d = q.shape
    out = np.full((total, hq, d), np.nan)
    lse = np.full((total, hq), np.nan)
    for b in range(len(cu_nodes) - 1):
        n0, n1 = int(cu_nodes[b]), int(cu_nodes[b + 1])
        nb = n1 - n0
        if nb == 0:
            continue
        sel = np.arange(nb) if nodes is None else np.asarray(nodes[b], dtype=np.int64)
        if len(sel) == 0:
            continue
        plen = int(prefix_len[b])
        kp = gather_prefix(k_cache, block_table[b], plen)  # [plen, hkv, d]
        vp = gather_prefix(v_cache, block_table[b], plen)
        par = parent[n0:n1]
        # visible[i, j]: tree node j is i itself or an ancestor of i (M_tree == 0)
        visible = np.zeros((len(sel), nb), dtype=bool)
        for r, i in enumerate(sel):
            visible[r, ancestors_or_self(par, int(i))] = True
        for h in range(hq):
            g = kv_head(h, hq, hkv)
            qs = q[n0 + sel, h, :]                         # [r, d]
            s_pre = scale * (qs @ kp[:, g, :].T)            # [r, plen]
            s_tree = scale * (qs @ k_tree[n0:n1, g, :].T)   # [r, nb]
            s_tree = np.where(visible, s_tree, -np.inf)
            s = np.concatenate([s_pre, s_tree], axis=1)
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            l = w.sum(axis=1, keepdims=True)
            vals = np.concatenate([vp[:, g, :], v_tree[n0:n1, g, :]], axis=0)
            out[n0 + sel, h, :] = (w @ vals) / l
            lse[n0 + sel, h] = (m + np.log(l))[:, 0]
    return out, lse


def check_paging(block_table, prefix_len, num_blocks: int) -> int:
    """Error bit for a prefix that the block table cannot hold (ERR_BLOCK)."""
    from .tree import ERR_BLOCK
    err = 0
    max_blocks = block_table.shape[1]
    for b, plen in enumerate(prefix_len):
        nblk = (int(plen) + BLOCK - 1) // BLOCK
        if nblk > max_blocks:
            err |= ERR_BLOCK
            continue
        ids = block_table[b, :nblk]
        if np.any(ids < 0) or np.any(ids >= num_blocks):
            err |= ERR_BLOCK
    return err
