"""Pins for the tree-index oracle (ancestor-or-self sets, bitsets, depth).

The oracle builds ancestor sets by walking parent pointers.  These tests pin
it to constructions that share nothing with that walk: an Euler-tour
interval test, a transitive closure by boolean matrix products, closed-form
depths of regular trees, and a hand-written fixture.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def euler_intervals(parent):
    """pre-order index and subtree size from an explicit DFS (children by index)."""
    n = len(parent)
    children = [[] for _ in range(n)]
    roots = []
    for i, p in enumerate(parent):
        (roots if p < 0 else children[p]).append(i)
    pre = [0] * n
    size = [1] * n
    counter = 0

    def dfs(v):
        nonlocal counter
        pre[v] = counter
        counter += 1
        for c in children[v]:
            dfs(c)
            size[v] += size[c]

    for r in roots:
        dfs(r)
    return pre, size


def closure_matrix(parent):
    """vis[i, j] = j in Anc*(i), via repeated boolean products of the parent relation."""
    n = len(parent)
    a = np.eye(n, dtype=bool)
    step = np.zeros((n, n), dtype=bool)
    for i, p in enumerate(parent):
        if p >= 0:
            step[i, p] = True
    reach = a.copy()
    frontier = a.copy()
    for _ in range(n):
        frontier = (frontier.astype(np.int64) @ step.astype(np.int64)) > 0
        if not frontier.any():
            break
        reach |= frontier
    return reach


def bit(anc, i, j):
    return bool((int(anc[i, j // 64]) >> (j % 64)) & 1)


TREES = {
    "heap15": W.tree_heap(15),
    "chain70": W.tree_chain(70),
    "star9": W.tree_star(9),
    "kary8x3": W.tree_kary_levels(8, 3),
    "long": W.tree_branch_then_chains(4, 3, 10, 256),
    "rand130": W.tree_random(np.random.default_rng(5), 130, 8),
    "importance": W.tree_importance_sampled(np.random.default_rng(6), 64, 8, 0.7, 6, 2000),
}


@pytest.mark.parametrize("name", sorted(TREES))
def test_bitsets_match_euler_intervals_and_closure(name):
    parent = TREES[name]
    n = len(parent)
    words = (n + 63) // 64
    anc = oracle.anc_bitsets(parent, words)
    pre, size = euler_intervals(list(parent))
    reach = closure_matrix(parent)
    for i in range(n):
        for j in range(n):
            euler = pre[j] <= pre[i] < pre[j] + size[j]
            assert bit(anc, i, j) == euler == bool(reach[i, j]), (i, j)
    # no bits beyond the node count
    for i in range(n):
        for j in range(n, words * 64):
            assert not bit(anc, i, j)


def test_depth_closed_forms():
    d = oracle.depths(W.tree_heap(15))
    assert list(d) == [int(np.floor(np.log2(i + 1))) + 1 for i in range(15)]
    d = oracle.depths(W.tree_kary_levels(8, 3))
    assert list(d) == [1] * 8 + [2] * 64 + [3] * 512
    d = oracle.depths(W.tree_chain(70))
    assert list(d) == list(range(1, 71))
    d = oracle.depths(W.tree_branch_then_chains(4, 3, 10, 256))
    assert d.max() == 10 and (d == 10).sum() == 24


def test_popcount_equals_depth():
    for parent in TREES.values():
        n = len(parent)
        anc = oracle.anc_bitsets(parent, (n + 63) // 64)
        pop = [sum(bin(int(w)).count("1") for w in row) for row in anc]
        assert pop == list(oracle.depths(parent))


def test_golden_small_tree():
    with open(os.path.join(GOLDEN, "tree_small.json")) as f:
        g = json.load(f)
    parent = np.array(g["parent"], dtype=np.int32)
    assert list(oracle.depths(parent)) == g["depth"]
    for i, expect in enumerate(g["ancestors_or_self"]):
        assert sorted(oracle.ancestors_or_self(parent, i)) == sorted(expect)
    anc = oracle.anc_bitsets(parent, 1)
    assert [int(x) for x in anc[:, 0]] == g["bitset_word0"]


def test_build_index_batch_and_pos():
    parents = [W.tree_heap(7), W.tree_star(3), np.zeros(0, np.int32), W.tree_chain(4)]
    cu = np.cumsum([0] + [len(p) for p in parents]).astype(np.int32)
    flat = np.concatenate(parents).astype(np.int32)
    plen = np.array([10, 0, 5, 64], np.int32)
    anc, dep, pos, err = oracle.build_index(flat, cu, 7, plen)
    assert err == 0
    assert list(dep) == [1, 2, 2, 3, 3, 3, 3, 1, 1, 1, 1, 2, 3, 4]
    assert list(pos) == [10, 11, 11, 12, 12, 12, 12, 0, 0, 0, 64, 65, 66, 67]
    # the star's bitsets hold only the node itself (local indices)
    assert [int(x) for x in anc[7:10, 0]] == [1, 2, 4]


@pytest.mark.parametrize("bad", [[-1, 1], [-1, 0, 5], [-2], [0]])
def test_bad_parent_flagged(bad):
    par = np.array(bad, np.int32)
    cu = np.array([0, len(bad)], np.int32)
    _, _, _, err = oracle.build_index(par, cu, 64)
    assert err & oracle.ERR_BAD_PARENT


def test_too_many_nodes_flagged():
    par = W.tree_chain(65)
    _, _, _, err = oracle.build_index(par, np.array([0, 65], np.int32), 64)
    assert err & oracle.ERR_TOO_MANY_NODES


def test_planted_mistake_is_caught(monkeypatch):
    """An ancestor walk that drops the node itself must fail the Euler pin."""
    import oracle.tree as T

    def no_self(parent, n):
        out = []
        i = int(parent[n])
        while i >= 0:
            out.append(i)
            i = int(parent[i])
        return out

    monkeypatch.setattr(T, "ancestors_or_self", no_self)
    parent = TREES["heap15"]
    anc = T.anc_bitsets(parent, 1)
    pre, size = euler_intervals(list(parent))
    mismatches = sum(bit(anc, i, j) != (pre[j] <= pre[i] < pre[j] + size[j])
                     for i in range(15) for j in range(15))
    assert mismatches > 0
