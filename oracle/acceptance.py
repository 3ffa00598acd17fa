"""Acceptance oracle: ratio test, walk to the longest accepted path, residual resample.

The steps follow page [P537] "端云协同推测解码中草稿模型动态生成与验证并行化…",
§2.2.3 (batch verification and acceptance inside one kernel):
  1. every node gets p_accept = min(1, p_target / p_draft) at its drafted token;
  2. uniforms r ~ U(0,1), one per node, give each node an accept bit;
  3. a depth-first walk from the root stops at the first rejected node of each
     branch and outputs the longest accepted path;
and page [P525] "端侧大模型推测解码草稿模型动态剪枝策略…", §1.2: at the
rejection point a token is resampled.  The residual distribution is the
normalised max(0, p_target - p_draft); if it has no mass, the target row is
sampled instead (page [P525], §7.2: fall back to plain target sampling).

Readings taken where the pages are silent (each also listed in the design notes):
  * Row i of p_target / p_draft is the pair of distributions that judged node
    i's drafted token (those at its parent's context).
  * The test is the strict u < min(1, pt/pd) (the pages' `u < accept_prob`,
    page [P500] §10.2), with gamma = 1 and no log clamp.  It is evaluated
    exactly as (double)u * (double)pd < (double)pt: the product of two fp32
    numbers is exact in fp64, and for u in [0,1) this equals u < min(1, pt/pd).
  * A node counts as accepted only if it and all its ancestors pass.  The
    longest path ends at the accepted node of largest depth; ties go to the
    smallest node index.  Nothing accepted -> length 0.
  * The rejection point is the smallest-index child of the path's last node
    (or the smallest-index node under the prefix if nothing was accepted).
  * Bonus token at a fully accepted leaf: the target's single forward pass over
    the tree gives a distribution at every node's own context (page [P537]
    §2.2.3: one forward pass yields logits at every node), so when the path's
    last node w has no child, the caller may pass p_target at w's own context
    (own_row[w], a row of p_own) and the extra token is drawn from it with
    u_resample[w]: the step then always emits accepted + 1 tokens, as plain
    speculative sampling does (page [P525] §1.2).  Without that row nothing is
    resampled (-1).  An own_row entry outside [-1, own_rows) sets ERR_ROW.
  * Sampling is an integer inverse CDF: weights q_k = floor(r_k * 2^40) with
    r_k = (double)pt_k - (double)pd_k (0 where r_k <= 0), Z = sum q_k, the
    uniform u = M * 2^E taken exactly, T = floor(M * Z * 2^E), token = the
    smallest k whose running sum of q exceeds T.  All sums are integers, so
    the result does not depend on summation order.
"""
from __future__ import annotations

import math

import numpy as np

from .probs import ERR_ROW
from .tree import (ERR_BAD_PARENT, ERR_PATH, ERR_TOKEN, ERR_UNIFORM, ERR_ZERO_MASS,
                   ancestors_or_self, parent_errors)

FIX_SHIFT = 40
TWO40 = float(1 << FIX_SHIFT)


def ratio_accepts(u: float, pd_tok: float, pt_tok: float) -> bool:
    """u < min(1, pt/pd), evaluated exactly for fp32 inputs and u in [0, 1)."""
    return float(np.float64(u) * np.float64(pd_tok)) < float(np.float64(pt_tok))


def uniform_ok(u) -> bool:
    u = float(u)
    return (not math.isnan(u)) and 0.0 <= u < 1.0


def fixed_weights(row_t: np.ndarray, row_d: np.ndarray | None) -> np.ndarray:
    """q_k = floor(r_k * 2^40) for r_k > 0, else 0 (uint64).

    r_k = (double)pt_k - (double)pd_k, or (double)pt_k alone when row_d is None.
    """
    r = row_t.astype(np.float64)
    if row_d is not None:
        r = r - row_d.astype(np.float64)
    q = np.where(r > 0.0, np.floor(r * TWO40), 0.0)
    return q.astype(np.uint64)


def threshold(u: float, z: int) -> int:
    """floor(u * Z) for u in [0, 1) taken exactly as M * 2^E."""
    if u == 0.0:
        return 0
    f, e = math.frexp(float(u))          # u = f * 2^e, f in [0.5, 1)
    m = int(f * (1 << 53))                # exact: u = m * 2^(e-53)
    shift = 53 - e
    return (m * z) >> shift


def residual_token(row_t: np.ndarray, row_d: np.ndarray, u: float):
    """Token drawn from norm(max(0, pt - pd)) (fallback: norm(pt)) with uniform u.

    Returns (token, err_bits); token = -1 when both masses are zero.
    """
    q = fixed_weights(row_t, row_d)
    z = int(q.sum(dtype=np.uint64))
    if z == 0:
        q = fixed_weights(row_t, None)
        z = int(q.sum(dtype=np.uint64))
        if z == 0:
            return -1, ERR_ZERO_MASS
    t = threshold(u, z)
    csum = np.cumsum(q, dtype=np.uint64)
    k = int(np.searchsorted(csum, np.uint64(t), side="right"))
    return k, 0


def target_token(row_t: np.ndarray, u: float):
    """Token drawn from norm(p_target row) with uniform u (the bonus token), by the
    same integer inverse CDF.  Returns (token, err_bits); -1 when the row has no mass."""
    q = fixed_weights(row_t, None)
    z = int(q.sum(dtype=np.uint64))
    if z == 0:
        return -1, ERR_ZERO_MASS
    t = threshold(u, z)
    csum = np.cumsum(q, dtype=np.uint64)
    return int(np.searchsorted(csum, np.uint64(t), side="right")), 0


def _dfs_accepted(parent: np.ndarray, acc: list[bool]) -> list[bool]:
    """Walk from the prefix down, entering a node only if it passed its test.

    A node is reached iff every node on its root path passed; the walk is cut
    below each rejected node.
    """
    n = len(parent)
    children: list[list[int]] = [[] for _ in range(n)]
    roots = []
    for i in range(n):
        (roots if parent[i] < 0 else children[parent[i]]).append(i)
    ok = [False] * n
    stack = list(reversed([r for r in roots if acc[r]]))
    while stack:
        v = stack.pop()
        ok[v] = True
        stack.extend(reversed([c for c in children[v] if acc[c]]))
    return ok


def accept_sequence(pt: np.ndarray, pd: np.ndarray, token: np.ndarray, u_acc: np.ndarray,
                    u_res: np.ndarray, parent: np.ndarray, vocab: int, max_path: int,
                    p_own=None, own_row=None):
    """Acceptance for one sequence; all arrays are that sequence's local slices.

    pt / pd may be any row-indexable [N, vocab] arrays.  p_own [R, vocab] and
    own_row [N] (row of p_own at each node's own context, -1 = none) are optional:
    with them a fully accepted leaf draws the bonus token.
    Returns dict(accept_len, path (list, -1 padded to max_path), resample_node,
    resample_token, node_ok (list of 0/1), err).
    """
    n = len(parent)
    err = parent_errors(parent)
    if err & ERR_BAD_PARENT:
        return dict(accept_len=0, path=[-1] * max_path, resample_node=-1, resample_token=-1,
                    node_ok=[0] * n, err=err)
    acc = []
    for i in range(n):
        tok = int(token[i])
        a = False
        if not (0 <= tok < vocab):
            err |= ERR_TOKEN
        elif not uniform_ok(u_acc[i]):
            err |= ERR_UNIFORM
        else:
            a = ratio_accepts(u_acc[i], pd[i][tok], pt[i][tok])
        acc.append(a)
    ok = _dfs_accepted(parent, acc)
    depth = [len(ancestors_or_self(parent, i)) for i in range(n)]
    w = -1
    for i in range(n):
        if ok[i] and (w < 0 or depth[i] > depth[w]):
            w = i
    accept_len = depth[w] if w >= 0 else 0
    path_nodes = list(reversed(ancestors_or_self(parent, w))) if w >= 0 else []
    if len(path_nodes) > max_path:
        err |= ERR_PATH
    path = (path_nodes + [-1] * max_path)[:max_path]
    c = next((i for i in range(n) if parent[i] == w), -1)
    rtok = -1
    if c >= 0:
        if not uniform_ok(u_res[c]):
            err |= ERR_UNIFORM
        else:
            rtok, e = residual_token(np.asarray(pt[c]), np.asarray(pd[c]), float(u_res[c]))
            err |= e
    elif w >= 0 and own_row is not None:
        # the path ends at a leaf: bonus token from p_target at w's own context
        r = int(own_row[w])
        if r < -1 or (p_own is not None and r >= len(p_own)) or (p_own is None and r >= 0):
            err |= ERR_ROW
        elif r >= 0:
            c = w
            if not uniform_ok(u_res[w]):
                err |= ERR_UNIFORM
            else:
                rtok, e = target_token(np.asarray(p_own[r]), float(u_res[w]))
                err |= e
    return dict(accept_len=accept_len, path=path, resample_node=c, resample_token=rtok,
                node_ok=[1 if o else 0 for o in ok], err=err)


def accept(p_target, p_draft, token, u_accept, u_resample, parent, cu_nodes, vocab: int,
           max_path: int, p_own=None, own_row=None):
    """Acceptance for a batch of flattened trees.

    p_own [R, vocab] / own_row [total] (global node indexing, -1 = none): optional
    own-context target rows for bonus tokens at fully accepted leaves.
    Returns dict of numpy arrays: accept_len [B], path [B, max_path],
    resample_node [B], resample_token [B], node_ok [total] uint8, err (int).
    resample_node is the rejection node c whose residual was sampled, or, for a
    bonus token, the path's last node w itself.
    """
    bsz = len(cu_nodes) - 1
    total = int(cu_nodes[-1])
    out = dict(accept_len=np.zeros(bsz, np.int32), path=np.full((bsz, max_path), -1, np.int32),
               resample_node=np.full(bsz, -1, np.int32), resample_token=np.full(bsz, -1, np.int32),
               node_ok=np.zeros(total, np.uint8), err=0)
    for b in range(bsz):
        n0, n1 = int(cu_nodes[b]), int(cu_nodes[b + 1])
        r = accept_sequence(p_target[n0:n1], p_draft[n0:n1], token[n0:n1], u_accept[n0:n1],
                            u_resample[n0:n1], parent[n0:n1], vocab, max_path, p_own,
                            None if own_row is None else own_row[n0:n1])
        out["accept_len"][b] = r["accept_len"]
        out["path"][b] = r["path"]
        out["resample_node"][b] = r["resample_node"]
        out["resample_token"][b] = r["resample_token"]
        out["node_ok"][n0:n1] = r["node_ok"]
        out["err"] |= r["err"]
    return out
