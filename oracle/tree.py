"""Tree index oracle: depth, ancestor-or-self sets and their bitsets.

A draft tree is flattened into a node array with a parent index per node,
-1 marking a node that hangs directly off the shared prefix (page [P537]
"端云协同推测解码中草稿模型动态生成与验证并行化…", appendix B, the
parent-index input of the tree kernel: -1 is the root).  Node i may see node j
iff j is i itself or an ancestor of i (page [P537], §2.2.2, equation M_tree).

Reading taken where the page is silent: parents precede their children
(parent[i] < i), and several nodes may hang off the prefix (a forest).

Error bits (OR-ed into one word, shared with the acceptance oracle):
"""
from __future__ import annotations

import numpy as np

ERR_BAD_PARENT = 1        # parent[i] >= i or parent[i] < -1
ERR_TOO_MANY_NODES = 2    # a sequence holds more nodes than max_nodes
ERR_TOKEN = 4             # drafted token outside [0, vocab)
ERR_BLOCK = 8             # block id outside the pool, or prefix longer than the table
ERR_ZERO_MASS = 16        # residual and target mass both zero at the rejection node
ERR_PATH = 32             # accepted path longer than the caller's path buffer
ERR_UNIFORM = 64          # a uniform outside [0, 1)


def ancestors_or_self(parent: np.ndarray, n: int) -> list[int]:
    """Anc*(n): n, parent(n), parent(parent(n)), ... up to the node under the prefix."""
    out = []
    i = int(n)
    while i >= 0:
        out.append(i)
        i = int(parent[i])
    return out


def parent_errors(parent: np.ndarray) -> int:
    err = 0
    for i, p in enumerate(parent):
        if p >= i or p < -1:
            err |= ERR_BAD_PARENT
    return err


def depths(parent: np.ndarray) -> np.ndarray:
    """Depth of each node: 1 for a node under the prefix, +1 per tree edge."""
    return np.array([len(ancestors_or_self(parent, i)) for i in range(len(parent))], dtype=np.int32)


def anc_bitsets(parent: np.ndarray, words: int) -> np.ndarray:
    """[N, words] uint64; bit j of row i (word j//64, bit j%64) set iff j in Anc*(i)."""
    n = len(parent)
    out = np.zeros((n, words), dtype=np.uint64)
    for i in range(n):
        for j in ancestors_or_self(parent, i):
            out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out


def build_index(parent: np.ndarray, cu_nodes: np.ndarray, max_nodes: int,
                prefix_len: np.ndarray | None = None):
    """What the tree-index step returns for a batch of flattened trees.

    Returns (anc [total, words] uint64, depth [total] int32, pos [total] int32
    or None, err).  pos = prefix_len + depth - 1 is the position id of a node
    (page [P500], §9.1, the static tree position tensor).  When err is
    non-zero the other outputs are unspecified.
    """
    words = max(1, (int(max_nodes) + 63) // 64)
    total = int(cu_nodes[-1])
    anc = np.zeros((total, words), dtype=np.uint64)
    dep = np.zeros(total, dtype=np.int32)
    pos = np.zeros(total, dtype=np.int32) if prefix_len is not None else None
    err = 0
    for b in range(len(cu_nodes) - 1):
        n0, n1 = int(cu_nodes[b]), int(cu_nodes[b + 1])
        if n1 - n0 > max_nodes:
            err |= ERR_TOO_MANY_NODES
            continue
        par = parent[n0:n1]
        e = parent_errors(par)
        err |= e
        if e:
            continue
        anc[n0:n1] = anc_bitsets(par, words)
        dep[n0:n1] = depths(par)
        if pos is not None:
            pos[n0:n1] = int(prefix_len[b]) + dep[n0:n1] - 1
    return anc, dep, pos, err
