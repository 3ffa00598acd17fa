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

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

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
