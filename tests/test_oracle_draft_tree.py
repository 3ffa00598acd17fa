"""Pins of the draft-tree construction oracle (CPU only): degenerate shapes with
closed forms, the truncation and weight formulas on hand rows, the draw
probabilities of the first two steps against hand-derived values over exhaustive
uniform grids, invariants, error cases and a planted mistake."""
import numpy as np
import pytest

import workloads as W
from oracle import ERR_UNIFORM
from oracle.draft_tree import (ERR_DRAFT, build_tree, build_trees, importance_weights,
                               kept_count)


def rows_of(p, rows):
    return np.tile(np.asarray(p, np.float32), (rows, 1))


def test_one_candidate_per_context_builds_a_chain():
    n = 12
    parent, slot, depth, q, _ = build_tree(rows_of([0.9], n + 1), np.full(n, 0.5), n, 99, 0.7, 0.1)
    assert list(parent) == [-1] + list(range(n - 1))
    assert list(depth) == list(range(1, n + 1)) and set(slot) == {0}
    assert np.all(q == 1.0)  # one kept candidate carries the whole kept mass


def test_depth_one_builds_a_star_of_the_kept_slots():
    p = [0.4, 0.3, 0.2, 0.05, 0.05]
    parent, slot, depth, _, _ = build_tree(rows_of(p, 9), np.linspace(0, 0.99, 8), 8, 1, 0.7, 0.1)
    m, _ = kept_count(np.float32(p), 0.1)
    assert m == 3 and len(parent) == 3            # the frontier empties after the kept slots
    assert set(parent) == {-1} and set(depth) == {1} and sorted(slot) == [0, 1, 2]


def test_stops_at_max_depth_on_a_single_branch():
    parent, _, depth, _, _ = build_tree(rows_of([0.9], 11), np.zeros(10), 10, 3, 0.7, 0.0)
    assert list(parent) == [-1, 0, 1] and list(depth) == [1, 2, 3]


@pytest.mark.parametrize("ratio,m", [(0.2, 2), (0.0, 4), (0.6, 1), (0.15, 3), (0.1, 3)])
def test_kept_count_closed_forms(ratio, m):
    p = np.float32([0.5, 0.3, 0.1, 0.05])  # masses 0.5, 0.8, 0.9, 0.95
    got, mass = kept_count(p, ratio)
    assert got == m
    assert mass == sum(float(x) for x in p[:m])


def test_importance_weight_closed_forms():
    p = np.float32([0.5, 0.3, 0.2])
    assert np.allclose(importance_weights(p, 3, 1.0), np.float64(p) / np.float64(p).sum(), rtol=0,
                       atol=1e-16)
    assert np.all(importance_weights(p, 3, 0.0) == 1.0 / 3)
    w = importance_weights(p, 2, 0.5)            # over the kept pair only
    a, b = np.sqrt(np.float64(p[0])), np.sqrt(np.float64(p[1]))
    assert np.allclose(w, [a / (a + b), b / (a + b)], rtol=1e-15)
    assert np.all(importance_weights(np.float32([0.0, 0.0]), 2, 0.7) == 0.0)


def test_first_draw_frequencies_on_a_uniform_grid():
    """Over the grid u = (j + 1/2) / N, node 0 takes root slot k for a fraction
    of the grid equal to its importance weight, to within 1/N."""
    p = np.float32([0.35, 0.3, 0.2, 0.1, 0.05])
    beta, N = 0.7, 4000
    w = np.float64(p) ** np.float64(np.float32(beta))
    w = w / w.sum()
    counts = np.zeros(5)
    for j in range(N):
        _, slot, _, _, _ = build_tree(rows_of(p, 2), [(j + 0.5) / N], 1, 6, beta, 0.0)
        counts[slot[0]] += 1
    assert np.abs(counts / N - w).max() <= 1.0 / N


def test_second_draw_uses_path_weights():
    """Two slots per context, two nodes.  After node 0 takes root slot a, the
    candidates are root slot b (weight w_b) and a's children (w_a * w'_0,
    w_a * w'_1): P(tree) is a product of these ratios, derived here by hand and
    matched over a grid of (u0, u1)."""
    p0 = np.float32([0.7, 0.3])      # root context
    pc = np.float32([0.6, 0.4])      # every later context
    probs = np.stack([p0, pc, pc])
    beta = 0.5
    w = np.sqrt(np.float64(p0)); w /= w.sum()
    v = np.sqrt(np.float64(pc)); v /= v.sum()
    want = {}
    for a in (0, 1):
        b = 1 - a
        rest = w[b] + w[a] * v[0] + w[a] * v[1]
        want[(a, "root", b)] = w[a] * w[b] / rest
        want[(a, "child", 0)] = w[a] * w[a] * v[0] / rest
        want[(a, "child", 1)] = w[a] * w[a] * v[1] / rest
    N = 300
    got = {k: 0 for k in want}
    for i in range(N):
        for j in range(N):
            parent, slot, _, _, _ = build_tree(probs, [(i + 0.5) / N, (j + 0.5) / N], 2, 2,
                                               beta, 0.0)
            a = int(slot[0])
            kind = "root" if parent[1] == -1 else "child"
            got[(a, kind, int(slot[1]))] += 1
    for k in want:
        assert abs(got[k] / N ** 2 - want[k]) <= 2.0 / N, (k, got[k] / N ** 2, want[k])


def test_planted_missing_path_weight_is_caught():
    """A build that gave children their own importance weight only (no parent
    factor) would shift a second-draw probability of the case above by more than
    0.05, far outside that test's grid tolerance (2/300), so it would fail there."""
    w = np.sqrt(np.float64([0.7, 0.3])); w /= w.sum()
    v = np.sqrt(np.float64([0.6, 0.4])); v /= v.sum()
    a, b = 0, 1
    right = w[a] * v[0] / (w[b] + w[a] * v[0] + w[a] * v[1])
    wrong = v[0] / (w[b] + v[0] + v[1])
    assert abs(right - wrong) > 0.05 > 2.0 / 300


def test_renormalised_draft_probabilities():
    rng = np.random.default_rng(4)
    probs = W.draft_rows(rng, 1, 65, 8)[0]
    parent, slot, depth, q, _ = build_tree(probs, W.grid_uniforms(rng, 64), 64, 6, 0.7, 0.1)
    for i in range(len(parent)):
        ctx_row = 0 if parent[i] < 0 else parent[i] + 1
        m, mass = kept_count(probs[ctx_row], 0.1)
        assert slot[i] < m
        assert q[i] == np.float32(float(probs[ctx_row][slot[i]]) / mass)
    # a context whose kept children were all built: their q sum to 1
    for ctx in set(parent.tolist()):
        kids = np.flatnonzero(parent == ctx)
        ctx_row = 0 if ctx < 0 else ctx + 1
        m, _ = kept_count(probs[ctx_row], 0.1)
        if len(kids) == m:
            assert abs(float(q[kids].astype(np.float64).sum()) - 1.0) < 1e-6
    assert np.all(parent < np.arange(len(parent)))     # parents precede children
    ok = np.where(parent < 0, 0, depth[np.maximum(parent, 0)])
    assert np.all(depth == ok + 1)


def test_errors_and_padding():
    rng = np.random.default_rng(5)
    probs = W.draft_rows(rng, 3, 9, 4)
    u = np.stack([W.grid_uniforms(rng, 8) for _ in range(3)])
    probs[1, 2, 1] = 1.5
    u[2, 3] = 1.0
    parent, slot, depth, q, count, err = build_trees(probs, u, 8, 4, 0.7, 0.1)
    assert err == ERR_DRAFT | ERR_UNIFORM
    assert count[1] == 0 and count[2] == 0 and count[0] > 0
    assert np.all(parent[1:] == -2) and np.all(q[1:] == 0)
    n = count[0]
    assert np.all(parent[0, n:] == -2)
