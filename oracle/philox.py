"""Counter-based uniforms for the acceptance draws — TEST INFRASTRUCTURE ONLY.

Page [P537] "端云协同推测解码中草稿模型动态生成与验证并行化…", §8.2 (consistent sampling
across nodes): every rank must draw the same random numbers for a tree node, so
the pages drop stateful device generators for a counter-based one (Philox or
Threefry) whose input is built from the request, the tree level, the node index
and the step.  No random numbers then need to be broadcast, and a restarted or
migrated request draws the same numbers again.

The generator here is Philox4x64-10 as published by Salmon, Moraes, Dror and
Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11): a 256-bit counter
(four 64-bit words) and a 128-bit key (two words) go through ten rounds; a round
multiplies words 0 and 2 by two fixed 64-bit constants, keeps the high and low
halves of both 128-bit products and mixes the high halves with words 1 and 3
and the key; between rounds the key words grow by two fixed Weyl increments.

Readings taken where the page is silent (each also listed in the design notes):
  * The "hash" of (request, tree level, node, step) is the cipher itself: the
    counter of local node j of sequence b is (j, depth[j], step, request_id[b])
    and the key is (seed, purpose), where purpose separates independent draw
    families of one step (for example 0 for the acceptance uniforms).
  * Depth enters as its 32-bit unsigned pattern and the request id as its
    64-bit two's-complement pattern.
  * Word 0 of the output block gives node j's acceptance uniform and word 1 its
    resample uniform; a uniform is the word's top 24 bits times 2^-24, which is
    exact in fp32 and lies in [0, 1 - 2^-24].

Parity pins (tests/test_oracle_philox.py): the cipher equals numpy's
independent Philox4x64-10 bit generator word for word; the counter layout and
the 24-bit mapping are checked on hand-built cases; a planted mistake in the
round function fails the numpy pin.
"""
from __future__ import annotations

import numpy as np

MASK32 = (1 << 32) - 1
MASK64 = (1 << 64) - 1

# round multipliers and key (Weyl) increments of Philox4x64 (Salmon et al., SC'11)
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
ROUNDS = 10


def philox4x64(counter, key, rounds: int = ROUNDS):
    """Philox4x64-R block: four 64-bit counter words and two key words (Python ints)
    in, four 64-bit output words out."""
    c0, c1, c2, c3 = (int(w) & MASK64 for w in counter)
    k0, k1 = (int(w) & MASK64 for w in key)
    for r in range(rounds):
        if r > 0:  # key schedule: the key grows by the Weyl increments between rounds
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        prod0 = PHILOX_M0 * c0  # exact 128-bit products
        prod1 = PHILOX_M1 * c2
        hi0, lo0 = prod0 >> 64, prod0 & MASK64
        hi1, lo1 = prod1 >> 64, prod1 & MASK64
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform24(word: int) -> float:
    """Top 24 bits of a 64-bit word times 2^-24: a uniform in [0, 1 - 2^-24]."""
    return (int(word) >> 40) / float(1 << 24)


def node_counter(local: int, depth: int, step: int, request_id: int):
    """Counter words of one node (page [P537] §8.2: request, tree level, node, step)."""
    return (int(local) & MASK64, int(depth) & MASK32, int(step) & MASK64, int(request_id) & MASK64)


def node_uniforms(seed: int, purpose: int, step: int, request_id, depth, cu_nodes):
    """Acceptance and resample uniforms of every node of a flattened batch of trees.

    request_id [batch] (int), depth [total_nodes] (int, from the tree index),
    cu_nodes [batch + 1].  Returns (u_accept, u_resample), float32 [total_nodes]."""
    cu = [int(x) for x in cu_nodes]
    total = cu[-1] if cu else 0
    u_acc = np.zeros(total, dtype=np.float32)
    u_res = np.zeros(total, dtype=np.float32)
    key = (int(seed) & MASK64, int(purpose) & MASK64)
    for b in range(len(cu) - 1):
        for n in range(cu[b], cu[b + 1]):
            x = philox4x64(node_counter(n - cu[b], int(depth[n]), step, int(request_id[b])), key)
            u_acc[n] = uniform24(x[0])
            u_res[n] = uniform24(x[1])
    return u_acc, u_res
