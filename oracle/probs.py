"""Target-logits -> probability-rows oracle: a row softmax, in fp64.

The target model's single forward pass over the whole tree gives one logits row
per context (page [P537] "端云协同推测解码中草稿模型动态生成与验证并行化…", §2.2.3: one
forward over the tree outputs every node's logits; the acceptance then compares
p_target with p_draft per node).  A drafted token is judged by the distribution
at its parent's context, so siblings share one row: output row i is the softmax
of logits row row_of[i] (row_of = identity when every node has its own row).
The pages compute log-probabilities as logits minus a log-sum-exp (page [P525]
"端侧大模型推测解码草稿模型动态剪枝策略…", §7.1, log-space chain with the
log-sum-exp trick); here the probabilities themselves are produced, with the row
maximum subtracted before exp.

Readings taken where the pages are silent: an optional inverse temperature t
multiplies the logits (t = 1: plain softmax); logits are fp32; the output is the
exact softmax (fp64 here, fp32 on the device); a row_of entry outside the
context rows sets the error bit and leaves that output row as zeros.

Kept-set rows (softmax_rows_kept).  Page [P525] "端侧大模型推测解码草稿模型动态剪枝策略…",
§2.2.1: pruning the draft keeps a set R of candidate tokens per context, so the
distribution the drafted tokens are actually drawn from is q~ = q * 1[x in R] / Z,
with Z the mass of R under q.  §2.2.2 writes this as a logits edit before the
softmax: log(1/Z) added to the logits of the kept tokens and minus infinity for
the others.  Reading taken here: that edit belongs to the draft's logits (it
yields q~, the distribution acceptance must divide by); added to the target's
logits it would change the distribution being sampled, so the target rows stay
the plain softmax.  The constant log(1/Z) cancels inside a softmax, so a kept
row is the softmax over R alone: p[k] = exp(t*l[k] - M_R) / sum_{k' in R}
exp(t*l[k'] - M_R) for k in R, 0 elsewhere, M_R the maximum over R.  keep[r] lists
context row r's kept token ids; -1 entries are padding, repeated ids count once;
an id outside [-1, vocab) sets ERR_TOKEN and an empty set ERR_ZERO_MASS, and
either leaves the output row as zeros.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .tree import ERR_TOKEN, ERR_ZERO_MASS

ERR_ROW = 128  # a context-row index outside [0, ctx_rows)


def softmax_rows(logits, row_of=None, inv_temperature: float = 1.0):
    """Returns (probs [R, V] fp64, err).  logits [C, V] fp32/fp64; row_of [R] or None."""
    lg = np.asarray(logits, dtype=np.float64)
    ctx_rows, vocab = lg.shape
    idx = np.arange(ctx_rows) if row_of is None else np.asarray(row_of, dtype=np.int64)
    out = np.zeros((len(idx), vocab), dtype=np.float64)
    err = 0
    t = float(inv_temperature)
    for i, r in enumerate(idx):
        if r < 0 or r >= ctx_rows:
            err |= ERR_ROW
            continue
        z = t * lg[r]
        z = z - z.max()
        e = np.exp(z)
        out[i] = e / e.sum()
    return out, err


def softmax_rows_kept(logits, keep, row_of=None, inv_temperature: float = 1.0):
    """Returns (probs [R, V] fp64, err): each output row the softmax over its context
    row's kept set (keep [C, K] int, -1 = padding), zero outside the set."""
    lg = np.asarray(logits, dtype=np.float64)
    ctx_rows, vocab = lg.shape
    kp = np.asarray(keep, dtype=np.int64).reshape(ctx_rows, -1)
    idx = np.arange(ctx_rows) if row_of is None else np.asarray(row_of, dtype=np.int64)
    out = np.zeros((len(idx), vocab), dtype=np.float64)
    err = 0
    t = float(inv_temperature)
    for i, r in enumerate(idx):
        if r < 0 or r >= ctx_rows:
            err |= ERR_ROW
            continue
        ids = kp[r]
        if np.any((ids < -1) | (ids >= vocab)):
            err |= ERR_TOKEN
            continue
        kept = sorted(set(int(k) for k in ids if k >= 0))
        if not kept:
            err |= ERR_ZERO_MASS
            continue
        z = t * lg[r, kept]
        e = np.exp(z - z.max())
        out[i, kept] = e / e.sum()
    return out, err
