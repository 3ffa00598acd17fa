"""Draft-tree construction oracle: importance-sampled expansion with a
cumulative-mass soft truncation, one tree per sequence.

The pages grow the candidate tree from the draft model's distributions instead
of a fixed k-ary shape: at each expansion the top-K draft probabilities p give
importance weights w = p^beta / sum p^beta, and branches are kept and deepened
by sampling on w (page [P500] "端侧多模态大模型推测解码草稿模型动态剪枝…", §3.1,
steps 1-3).  Before that, the candidates of one context are truncated
breadth-first by cumulative probability mass: in descending order of p they are
kept until the kept mass reaches 1 - prune_ratio, and the kept probabilities are
renormalised by that mass (page [P525] "端侧大模型推测解码草稿模型动态剪枝策略…",
§2.1.2, steps 1-3).

Readings taken where the pages leave the procedure open (one sequence):
  * Inputs are the draft model's top-K probabilities per context, in
    descending order: row 0 is the context at the end of the prefix, row n + 1
    the context after node n (nodes are numbered in the order they are built).
  * Truncation keeps the shortest leading run of slots whose mass (summed in
    fp64, in slot order) reaches 1 - prune_ratio, at least one slot, at most K.
  * A kept candidate's weight is its importance weight times its parent's path
    weight (the product of importance weights from the prefix down); the
    importance weights are normalised over the kept candidates of the context.
  * Step i draws one candidate from all candidates not yet taken, with
    probability proportional to path weight, by inverse CDF with the uniform
    u[i] over the candidates in the order they were created: the first whose
    running sum exceeds u[i] * (sum of all).  The drawn candidate becomes node i
    (its parent: the context's node, -1 for the prefix); if its depth is below
    max_depth and row i + 1 exists, its kept children become candidates.
  * Building stops after n_max nodes or when no candidate has positive weight.
  * q_draft of a node = its probability divided by the kept mass of its
    context: the renormalised draft distribution the acceptance test must use
    for it.
  * A sequence with a probability outside [0, 1] or a uniform outside [0, 1)
    builds nothing and sets an error bit.
Arithmetic is fp64 (probabilities and uniforms are fp32 inputs, exact in fp64);
q_draft is returned rounded to fp32.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .tree import ERR_UNIFORM

ERR_DRAFT = 256  # a probability outside [0, 1] (or NaN) in a sequence's rows


def kept_count(p_row, prune_ratio: float) -> tuple[int, float]:
    """(m, kept mass): the shortest leading run of slots with mass >= 1 - prune_ratio."""
    target = 1.0 - float(np.float32(prune_ratio))
    mass = 0.0
    for j, p in enumerate(p_row):
        mass += float(p)
        if mass >= target:
            return j + 1, mass
    return len(p_row), mass


def importance_weights(p_row, m: int, beta: float) -> np.ndarray:
    """w_k = p_k^beta / sum_{j<m} p_j^beta over the kept slots (fp64); zeros if no mass."""
    b = float(np.float32(beta))
    pw = np.array([float(p) ** b if p > 0 else 0.0 for p in p_row[:m]], dtype=np.float64)
    s = 0.0
    for x in pw:
        s += x
    return pw / s if s > 0 else np.zeros(m)


def build_tree(probs, u, n_max: int, max_depth: int, beta: float, prune_ratio: float):
    """One sequence.  probs [rows, K] fp32, u [n_max] in [0, 1).
    Returns (parent, slot, depth, q_draft) arrays of the built nodes (length = count)
    and the draw margins (|u * total - nearest running-sum boundary| / total per step)."""
    probs = np.asarray(probs, dtype=np.float32)
    rows = probs.shape[0]
    parent, slot, depth, qd, margins = [], [], [], [], []
    # candidates: [path weight, context node, slot, depth, q] in creation order
    cand: list[list] = []

    def expand(row: int, ctx: int, ctx_depth: int, ctx_pw: float) -> None:
        m, mass = kept_count(probs[row], prune_ratio)
        w = importance_weights(probs[row], m, beta)
        for k in range(m):
            q = float(np.float32(float(probs[row][k]) / mass)) if mass > 0 else 0.0
            cand.append([ctx_pw * w[k], ctx, k, ctx_depth + 1, q])

    if rows > 0 and n_max > 0:
        expand(0, -1, 0, 1.0)
    for i in range(n_max):
        total = 0.0
        for c in cand:
            total += c[0]
        if not total > 0.0:
            break
        t = float(u[i]) * total
        run, pick = 0.0, -1
        bounds = []
        for j, c in enumerate(cand):
            run += c[0]
            bounds.append(run)
            if pick < 0 and run > t:
                pick = j
        margins.append(min(abs(t - b) for b in bounds) / total)
        c = cand[pick]
        parent.append(c[1])
        slot.append(c[2])
        depth.append(c[3])
        qd.append(c[4])
        pw = c[0]
        c[0] = 0.0  # taken: keeps its place in the creation order, weight zero
        if c[3] < max_depth and i + 1 < rows:
            expand(i + 1, i, c[3], pw)
    return (np.array(parent, np.int32), np.array(slot, np.int32), np.array(depth, np.int32),
            np.array(qd, np.float32), np.array(margins))


def build_trees(probs, u, n_max: int, max_depth: int, beta: float, prune_ratio: float):
    """Every sequence: probs [B, rows, K], u [B, n_max].  Returns padded
    (parent, slot, depth [B, n_max] int32 with -2 past the count; q_draft [B, n_max]
    fp32 with 0 past the count; count [B]; err)."""
    probs = np.asarray(probs, dtype=np.float32)
    batch = probs.shape[0]
    parent = np.full((batch, n_max), -2, np.int32)
    slot = np.full((batch, n_max), -2, np.int32)
    depth = np.full((batch, n_max), -2, np.int32)
    qd = np.zeros((batch, n_max), np.float32)
    count = np.zeros(batch, np.int32)
    err = 0
    u = np.asarray(u, dtype=np.float32)
    for b in range(batch):
        bad = 0
        if not np.all((probs[b] >= 0) & (probs[b] <= 1)):
            bad |= ERR_DRAFT
        if not np.all((u[b, :n_max] >= 0) & (u[b, :n_max] < 1)):
            bad |= ERR_UNIFORM
        if bad:
            err |= bad
            continue
        p, s, d, q, _ = build_tree(probs[b], u[b], n_max, max_depth, beta, prune_ratio)
        n = len(p)
        parent[b, :n], slot[b, :n], depth[b, :n], qd[b, :n] = p, s, d, q
        count[b] = n
    return parent, slot, depth, qd, count, err
