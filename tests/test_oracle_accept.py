"""Pins for the acceptance oracle (ratio test, walk, residual resample).

Pinned against: a hand-worked fixture; exhaustive enumeration of every
accept pattern on small trees, compared with an independent recursive
longest-path search; special cases of the ratio test; the speculative
sampling theorem on chains (Monte-Carlo: emitted tokens follow p_target and
the mean accepted length matches the closed form sum_k prod_{i<=k} alpha_i with
alpha = sum_x min(pt, pd)); and an exact sweep of the residual sampler over
all 2^24 grid uniforms.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

import oracle
import oracle.acceptance as OA
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return np.asarray(x, dtype=np.float32)


def test_golden_hand_worked():
    with open(os.path.join(GOLDEN, "accept_small.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        u_res = np.zeros(5, np.float32)
        u_res[4] = c["u_resample_node4"]
        r = OA.accept_sequence(f32(g["p_target"]), f32(g["p_draft"]), np.array(g["token"]),
                               f32(g["u_accept"]), u_res, np.array(g["parent"]), g["vocab"], 4)
        assert r["err"] == 0
        assert r["accept_len"] == c["accept_len"]
        assert r["path"] == c["path"] + [-1] * (4 - len(c["path"]))
        assert r["node_ok"] == c["node_ok"]
        assert r["resample_node"] == c["resample_node"]
        assert r["resample_token"] == c["resample_token"]


def test_ratio_special_cases():
    assert OA.ratio_accepts(0.0, 0.5, 1e-30)          # u = 0 accepts iff pt > 0
    assert not OA.ratio_accepts(0.0, 0.5, 0.0)        # pt = 0 always rejects
    assert not OA.ratio_accepts(0.0, 0.0, 0.0)
    assert OA.ratio_accepts(0.999, 0.0, 1e-30)        # pd = 0, pt > 0: ratio is infinite
    assert not OA.ratio_accepts(0.5, 0.5, 0.25)       # u equal to the ratio: strict test rejects
    assert OA.ratio_accepts(np.nextafter(np.float32(0.5), np.float32(0)), 0.5, 0.25)
    assert not OA.ratio_accepts(0.1, float("nan"), 0.5)
    assert not OA.ratio_accepts(0.1, 0.5, float("nan"))
    # the product form equals u < min(1, pt/pd) computed in exact rationals
    rng = np.random.default_rng(0)
    for _ in range(3000):
        u, pd, pt = (float(np.float32(x)) for x in rng.random(3) ** rng.integers(1, 30, 3))
        u = min(u, float(np.nextafter(np.float32(1), np.float32(0))))
        exact = Fraction(u) < min(Fraction(1), Fraction(pt) / Fraction(pd)) if pd > 0 else pt > 0
        assert OA.ratio_accepts(u, pd, pt) == exact


def recursive_longest(parent, acc):
    """Independent search: the deepest node whose whole root path passed.

    Returns (depth, node) maximising depth, ties to the smallest node index.
    """
    n = len(parent)
    kids = {i: [c for c in range(n) if parent[c] == i] for i in [-1] + list(range(n))}
    best = (0, -1)

    def go(v, d):
        nonlocal best
        if (d > best[0]) or (d == best[0] and v < best[1]):
            best = (d, v)
        for c in kids[v]:
            if acc[c]:
                go(c, d + 1)

    for r in kids[-1]:
        if acc[r]:
            go(r, 1)
    return best


def forced_rows(acc_bits, vocab=4):
    """Rows and uniforms that make node i pass its test iff acc_bits[i]."""
    n = len(acc_bits)
    pt = np.full((n, vocab), 0.25, np.float32)
    pd = np.full((n, vocab), 0.25, np.float32)
    tok = np.zeros(n, np.int32)
    for i, a in enumerate(acc_bits):
        if not a:
            pt[i] = [0.0, 0.5, 0.25, 0.25]   # pt at the drafted token is 0 -> reject
    return pt, pd, tok, np.full(n, 0.5, np.float32), np.full(n, 0.5, np.float32)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_exhaustive_accept_patterns(seed):
    rng = np.random.default_rng(seed)
    n = 9 if seed < 3 else 10
    parent = W.tree_random(rng, n, 4) if seed != 1 else W.tree_heap(n)
    for mask in range(1 << n):
        acc = [bool((mask >> i) & 1) for i in range(n)]
        pt, pd, tok, ua, ur = forced_rows(acc)
        r = OA.accept_sequence(pt, pd, tok, ua, ur, parent, 4, n)
        d, w = recursive_longest(list(parent), acc)
        assert r["accept_len"] == d
        path = []
        v = w
        while v >= 0:
            path.append(v)
            v = int(parent[v])
        assert r["path"] == path[::-1] + [-1] * (n - len(path))
        c = min([i for i in range(n) if parent[i] == w], default=-1)
        assert r["resample_node"] == c
        assert (r["resample_token"] >= 0) == (c >= 0)
        ok = [all(acc[j] for j in oracle.ancestors_or_self(parent, i)) for i in range(n)]
        assert r["node_ok"] == [int(o) for o in ok]


def test_equal_distributions_accept_everything():
    case = W.make_case("eq", [W.tree_random(np.random.default_rng(2), 40, 6)], [0], 1, 1, 8,
                       W.DT_F32, 300, 5)
    r = OA.accept_sequence(case.p_draft, case.p_draft, case.token, case.u_accept, case.u_resample,
                           case.parent, 300, 64)
    dep = oracle.depths(case.parent)
    assert r["node_ok"] == [1] * 40
    w = int(np.flatnonzero(dep == dep.max())[0])
    assert r["accept_len"] == dep.max() and r["path"][dep.max() - 1] == w
    assert r["resample_node"] == -1 and r["resample_token"] == -1   # w is a leaf


def test_sibling_rule_by_exact_enumeration():
    """Two drafted siblings judged independently: P(emit token 1) = 5/16, not
    p_target(1) = 1/4 (so only chains are distribution-preserving)."""
    pt = f32([[0.75, 0.25], [0.75, 0.25]])
    pd = f32([[0.5, 0.5], [0.5, 0.5]])
    grid = [(k + 0.5) / 16 for k in range(16)]
    total = Fraction(0)
    for ta in (0, 1):
        for tb in (0, 1):
            for ua in grid:
                for ub in grid:
                    r = OA.accept_sequence(pt, pd, np.array([ta, tb]), f32([ua, ub]), f32([0.5, 0.5]),
                                           np.array([-1, -1]), 2, 2)
                    emit = r["resample_token"] if r["accept_len"] == 0 else [ta, tb][r["path"][0]]
                    if emit == 1:
                        total += Fraction(1, 4 * 16 * 16)
    assert total == Fraction(5, 16)


def test_error_bits():
    pt = np.full((3, 4), 0.25, np.float32)
    par = np.array([-1, 0, 1])
    r = OA.accept_sequence(pt, pt, np.array([0, 4, 0]), f32([0.1] * 3), f32([0.1] * 3), par, 4, 3)
    assert r["err"] & oracle.ERR_TOKEN and r["accept_len"] == 1
    r = OA.accept_sequence(pt, pt, np.array([0, 0, 0]), f32([0.1, 1.0, 0.1]), f32([0.1] * 3), par, 4, 3)
    assert r["err"] & oracle.ERR_UNIFORM and r["accept_len"] == 1
    r = OA.accept_sequence(pt, pt, np.array([0, 0, 0]), f32([0.1] * 3), f32([0.1] * 3), par, 4, 2)
    assert r["err"] == oracle.ERR_PATH and r["accept_len"] == 3 and r["path"] == [0, 1]
    z = np.zeros((1, 4), np.float32)
    z[0, 0] = 1.0
    r = OA.accept_sequence(np.zeros((1, 4), np.float32), z, np.array([0]), f32([0.5]), f32([0.5]),
                           np.array([-1]), 4, 1)
    assert r["err"] == oracle.ERR_ZERO_MASS and r["resample_node"] == 0 and r["resample_token"] == -1
    r = OA.accept_sequence(pt, pt, np.array([0, 0, 0]), f32([0.1] * 3), f32([0.1] * 3),
                           np.array([-1, 1, 0]), 4, 3)
    assert r["err"] & oracle.ERR_BAD_PARENT


def test_fallback_to_target_when_residual_is_empty():
    pt = f32([[0.5, 0.5, 0.0]])
    pd = f32([[0.5, 0.5, 0.0]])
    # nothing left in max(0, pt - pd): sample from pt itself
    tok, err = OA.residual_token(pt[0], pd[0], 0.75)
    assert err == 0 and tok == 1
    tok, err = OA.residual_token(pt[0], pd[0], 0.25)
    assert err == 0 and tok == 0


def test_threshold_is_exact_floor():
    rng = np.random.default_rng(3)
    for _ in range(5000):
        u = np.float32(rng.random() ** rng.integers(1, 40))
        if u >= 1:
            continue
        z = int(rng.integers(1, 1 << 58, dtype=np.int64))
        assert OA.threshold(float(u), z) == int(Fraction(float(u)) * z)
    tiny = float(np.float32(1e-45))  # smallest subnormal
    assert OA.threshold(tiny, (1 << 58) - 1) == 0


def test_residual_sampler_exact_grid_sweep():
    rng = np.random.default_rng(11)
    vocab = 5
    pt = rng.random(vocab).astype(np.float32)
    pt /= pt.sum()
    pd = rng.random(vocab).astype(np.float32)
    pd /= pd.sum()
    q = OA.fixed_weights(pt, pd)
    z = int(q.sum())
    assert z > 0
    csum = np.cumsum(q).astype(np.uint64)
    m = np.arange(1 << 24, dtype=np.uint64)
    zh, zl = np.uint64(z >> 24), np.uint64(z & ((1 << 24) - 1))
    t = m * zh + ((m * zl) >> np.uint64(24))          # floor(m * z / 2^24)
    tok = np.searchsorted(csum, t, side="right")
    counts = np.bincount(tok, minlength=vocab)
    for k in range(vocab):
        assert abs(int(counts[k]) - int(q[k]) * (1 << 24) / z) <= 1.0
    # the sampled law is within the quantisation bound of norm(max(0, pt - pd))
    r = np.maximum(pt.astype(np.float64) - pd.astype(np.float64), 0)
    want = r / r.sum()
    assert np.abs(counts / float(1 << 24) - want).max() <= 2.0 ** -24 * 2 + vocab * 2.0 ** -40 / r.sum()
    # the oracle's own sampler agrees with the sweep, including at every boundary
    picks = list(rng.integers(0, 1 << 24, 300))
    for k in range(vocab):
        b = -(-int(csum[k]) * (1 << 24) // z)             # first m whose threshold reaches csum[k]
        picks += [b - 1, b, b + 1]
    for mm in picks:
        if 0 <= mm < (1 << 24):
            got, err = OA.residual_token(pt, pd, float(mm) * 2.0 ** -24)
            assert err == 0 and got == tok[mm]


def test_monte_carlo_chain_preserves_target():
    """Speculative sampling on a chain: the token emitted at depth k, given that
    depth k is reached, follows p_target_k; mean accepted length matches the
    closed form from alpha = E_{x~p_draft}[min(1, pt/pd)]."""
    rng = np.random.default_rng(2024)
    depth_n, vocab, trials = 3, 4, 40000
    pt = rng.dirichlet(np.ones(vocab), depth_n).astype(np.float32)
    pd = rng.dirichlet(np.ones(vocab), depth_n).astype(np.float32)
    parent = W.tree_chain(depth_n)
    alpha = np.minimum(pt.astype(np.float64), pd.astype(np.float64)).sum(axis=1)
    expect_len = sum(np.prod(alpha[:k + 1]) for k in range(depth_n))
    emitted = [[] for _ in range(depth_n)]
    lens = np.zeros(trials)
    cdf = np.cumsum(pd.astype(np.float64), axis=1)
    for t in range(trials):
        tok = np.array([min(int((cdf[k] <= rng.random() * cdf[k, -1]).sum()), vocab - 1)
                        for k in range(depth_n)], np.int32)
        ua = W.grid_uniforms(rng, depth_n)
        ur = W.grid_uniforms(rng, depth_n)
        r = OA.accept_sequence(pt, pd, tok, ua, ur, parent, vocab, depth_n)
        n_acc = r["accept_len"]
        lens[t] = n_acc
        for k in range(min(n_acc + 1, depth_n)):
            emitted[k].append(int(tok[k]) if k < n_acc else r["resample_token"])
    se = lens.std() / np.sqrt(trials)
    assert abs(lens.mean() - expect_len) < 5 * se + 1e-3
    for k in range(depth_n):
        obs = np.bincount(emitted[k], minlength=vocab)
        pk = pt[k].astype(np.float64)
        exp = pk / pk.sum() * len(emitted[k])
        p = stats.chisquare(obs, exp).pvalue
        assert p > 1e-4, (k, obs, exp, p)


def test_monte_carlo_catches_a_planted_mistake(monkeypatch):
    """Resampling from pt - pd without the max(0, .) clamp breaks the chi-square pin."""
    def unclamped(row_t, row_d):
        r = row_t.astype(np.float64) - (row_d.astype(np.float64) if row_d is not None else 0)
        return np.floor(np.abs(r) * OA.TWO40).astype(np.uint64)

    monkeypatch.setattr(OA, "fixed_weights", unclamped)
    rng = np.random.default_rng(5)
    pt = f32([[0.7, 0.2, 0.1]])
    pd = f32([[0.1, 0.2, 0.7]])
    tok_counts = np.zeros(3)
    for _ in range(4000):
        tok = np.array([min(int((np.cumsum(pd[0]) <= rng.random()).sum()), 2)], np.int32)
        r = OA.accept_sequence(pt, pd, tok, W.grid_uniforms(rng, 1), W.grid_uniforms(rng, 1),
                               np.array([-1]), 3, 1)
        emit = int(tok[0]) if r["accept_len"] else r["resample_token"]
        tok_counts[emit] += 1
    p0 = pt[0].astype(np.float64)
    p = stats.chisquare(tok_counts, p0 / p0.sum() * tok_counts.sum()).pvalue
    assert p < 1e-6
