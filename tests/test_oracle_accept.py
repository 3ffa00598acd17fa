"""Pins for the acceptance oracle (ratio test, walk, residual resample).

Pinned against: a hand-worked fixture; exhaustive enumeration of every
accept pattern on small trees, compared with an independent recursive
longest-path search; special cases of the ratio test; the speculative
sampling theorem on chains (Monte-Carlo over 10^6 steps: emitted tokens follow
p_target and the mean accepted length matches the closed form
sum_k prod_{i<=k} alpha_i with alpha = sum_x min(pt, pd)); exact sweeps of the
residual and target samplers over all 2^24 grid uniforms.  The bonus token at a
fully accepted leaf is pinned by hand-worked cases, the exhaustive patterns
(a bonus exactly when the winner is a leaf), the same Monte-Carlo law (every
step then emits accept_len + 1 tokens, the last following the leaf's own row)
and a planted mistake (bonus drawn as a residual) that the law rejects.
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
        # with every node's own-context row (row i = node i, a point mass on token
        # i % 4): a leaf winner draws the bonus from its own row, nothing else changes
        own = np.zeros((n, 4), np.float32)
        own[np.arange(n), np.arange(n) % 4] = 1.0
        rb = OA.accept_sequence(pt, pd, tok, ua, ur, parent, 4, n, own, np.arange(n))
        assert (rb["accept_len"], rb["path"], rb["node_ok"]) == (r["accept_len"], r["path"],
                                                                 r["node_ok"])
        if c >= 0 or w < 0:
            assert (rb["resample_node"], rb["resample_token"]) == (c, r["resample_token"])
        else:
            assert (rb["resample_node"], rb["resample_token"]) == (w, w % 4)


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
    # with own-context rows the leaf draws its bonus token: depth + 1 tokens in all
    rb = OA.accept_sequence(case.p_draft, case.p_draft, case.token, case.u_accept,
                            case.u_resample, case.parent, 300, 64, case.p_target,
                            np.arange(40, dtype=np.int32))
    want, _ = OA.target_token(case.p_target[w], float(case.u_resample[w]))
    assert (rb["resample_node"], rb["resample_token"]) == (w, want) and want >= 0


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


def _chain_trials(job):
    """Worker: `trials` draws of speculative sampling on a chain through the oracle.

    Tokens are drawn from p_draft row by row (inverse CDF of a float64 uniform),
    uniforms on the 2^-24 grid.  With p_own, the leaf (last node) has own-context
    row 0 of p_own, so a fully accepted chain emits a bonus token.  Returns the
    emitted-token counts per depth ([depth_n + 1, vocab]: row k = the token
    emitted at depth k + 1, given that depth was reached), the sum and the sum of
    squares of accept_len, and the number of steps that emitted no extra token."""
    seed, trials, pt, pd, p_own = job
    rng = np.random.default_rng(seed)
    depth_n, vocab = pt.shape
    parent = W.tree_chain(depth_n)
    own_row = None
    if p_own is not None:
        own_row = np.full(depth_n, -1, np.int32)
        own_row[-1] = 0
    cdf = np.cumsum(pd.astype(np.float64), axis=1)
    draws = rng.random((trials, depth_n))
    toks = np.stack([np.minimum((cdf[k][None, :] <= draws[:, k:k + 1] * cdf[k, -1]).sum(axis=1),
                                vocab - 1) for k in range(depth_n)], axis=1).astype(np.int32)
    ua = W.grid_uniforms(rng, trials * depth_n).reshape(trials, depth_n)
    ur = W.grid_uniforms(rng, trials * depth_n).reshape(trials, depth_n)
    counts = np.zeros((depth_n + 1, vocab), np.int64)
    s1 = s2 = no_extra = 0
    for t in range(trials):
        r = OA.accept_sequence(pt, pd, toks[t], ua[t], ur[t], parent, vocab, depth_n, p_own,
                               own_row)
        n_acc = r["accept_len"]
        s1 += n_acc
        s2 += n_acc * n_acc
        for k in range(n_acc):
            counts[k, toks[t, k]] += 1
        if r["resample_token"] >= 0:
            counts[n_acc, r["resample_token"]] += 1
        else:
            no_extra += 1
    return counts, s1, s2, no_extra


def run_chain_monte_carlo(pt, pd, p_own, trials: int, seed: int):
    """_chain_trials over a process pool (at most 8 workers), results summed."""
    import concurrent.futures as cf
    workers = max(1, min(8, os.cpu_count() or 1))
    per = -(-trials // workers)
    jobs = [(seed * 1000 + i, per, pt, pd, p_own) for i in range(workers)]
    with cf.ProcessPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(_chain_trials, jobs))
    counts = sum(p[0] for p in parts)
    return counts, sum(p[1] for p in parts), sum(p[2] for p in parts), sum(p[3] for p in parts), \
        per * workers


MC_TRIALS = 1_000_000


def check_chain_law(pt, pd, p_own, counts, s1, s2, n):
    """Emitted tokens follow the target at every reached depth (chi-square) and the
    mean accepted length is sum_k prod_{i<=k} alpha_i, alpha_i = sum_x min(pt_i, pd_i)."""
    depth_n, vocab = pt.shape
    alpha = np.minimum(pt.astype(np.float64), pd.astype(np.float64)).sum(axis=1)
    expect_len = sum(np.prod(alpha[:k + 1]) for k in range(depth_n))
    mean = s1 / n
    se = np.sqrt(max(s2 / n - mean * mean, 0.0) / n)
    assert abs(mean - expect_len) < 5 * se + 1e-4, (mean, expect_len, se)
    rows = list(pt.astype(np.float64))
    if p_own is not None:
        rows.append(p_own[0].astype(np.float64))
    for k, pk in enumerate(rows):
        obs = counts[k]
        exp = pk / pk.sum() * obs.sum()
        p = stats.chisquare(obs, exp).pvalue
        assert p > 1e-4, (k, obs, exp, p)


def chain_rows(seed: int, depth_n: int = 3, vocab: int = 4):
    rng = np.random.default_rng(seed)
    pt = rng.dirichlet(np.ones(vocab), depth_n).astype(np.float32)
    pd = rng.dirichlet(np.ones(vocab), depth_n).astype(np.float32)
    p_own = rng.dirichlet(np.ones(vocab), 1).astype(np.float32)
    return pt, pd, p_own


def test_monte_carlo_chain_preserves_target():
    """Speculative sampling on a chain, 10^6 steps through the oracle: the token
    emitted at depth k, given that depth k is reached, follows p_target_k; the mean
    accepted length matches the closed form from alpha = E_{x~p_draft}[min(1, pt/pd)].
    Power: with 10^6 steps the chi-square test at p = 1e-4 (3 degrees of freedom)
    detects a shift of about 1.3e-3 in any token's probability at depth 1."""
    pt, pd, _ = chain_rows(2024)
    counts, s1, s2, no_extra, n = run_chain_monte_carlo(pt, pd, None, MC_TRIALS, 1)
    check_chain_law(pt, pd, None, counts, s1, s2, n)
    # without own-context rows a fully accepted chain emits nothing extra
    assert counts[len(pt)].sum() == 0
    assert no_extra > 0


def test_monte_carlo_chain_with_bonus_token():
    """With the leaf's own-context target row, every step emits accept_len + 1
    tokens: the extra one is the residual at a rejection, or, once the whole chain
    is accepted, the bonus drawn from that row -- and it follows the row (10^6 steps)."""
    pt, pd, p_own = chain_rows(77)
    counts, s1, s2, no_extra, n = run_chain_monte_carlo(pt, pd, p_own, MC_TRIALS, 2)
    check_chain_law(pt, pd, p_own, counts, s1, s2, n)
    assert no_extra == 0
    alpha = np.minimum(pt.astype(np.float64), pd.astype(np.float64)).sum(axis=1)
    full = counts[len(pt)].sum() / n          # chains accepted to the leaf
    assert abs(full - np.prod(alpha)) < 5 * np.sqrt(np.prod(alpha) / n)


def test_monte_carlo_bonus_catches_a_planted_mistake(monkeypatch):
    """A bonus drawn as a residual against the leaf's draft row (reusing the
    rejection sampler) instead of from the own-context target row fails the law."""
    pt, pd, p_own = chain_rows(77)
    leaf_pd = pd[-1].copy()
    monkeypatch.setattr(OA, "target_token", lambda row, u: OA.residual_token(row, leaf_pd, u))
    counts, _, _, _ = _chain_trials((9, 60000, pt, pd, p_own))
    row = p_own[0].astype(np.float64)
    obs = counts[len(pt)]
    p = stats.chisquare(obs, row / row.sum() * obs.sum()).pvalue
    assert p < 1e-6


def test_bonus_hand_worked():
    """Hand-worked cases of the bonus token (pt = pd: every drafted token passes)."""
    rows = f32([[0.1, 0.2, 0.3, 0.4]] * 3)
    own = f32([[0.1, 0.2, 0.3, 0.4], [0.0, 0.0, 1.0, 0.0]])
    tok = np.array([1, 2, 3], np.int32)
    ua = f32([0.5, 0.5, 0.5])
    chain = np.array([-1, 0, 1], np.int32)
    # the cumulative target mass is 0.1, 0.3, 0.6, 1.0: u = 0.5 -> token 2, 0.05 -> 0, 0.95 -> 3
    for u, want in ((0.5, 2), (0.05, 0), (0.95, 3), (0.0, 0)):
        r = OA.accept_sequence(rows, rows, tok, ua, f32([0.9, 0.9, u]), chain, 4, 4, own,
                               np.array([-1, -1, 0], np.int32))
        assert (r["accept_len"], r["resample_node"], r["resample_token"], r["err"]) == (3, 2, want, 0)
    # a point mass: always that token
    r = OA.accept_sequence(rows, rows, tok, ua, f32([0.9, 0.9, 0.99]), chain, 4, 4, own,
                           np.array([-1, -1, 1], np.int32))
    assert (r["resample_node"], r["resample_token"]) == (2, 2)
    # the winner has a child: no bonus, the smallest child is the rejection node and
    # its residual max(0, pt - pd) = (0.1, 0.2, 0.3, 0) is sampled: u = 0.4 -> token 1
    star = np.array([-1, 0, 0], np.int32)
    rej = f32([0.5, 0.5, 0.5])
    pt = f32([[0.1, 0.2, 0.3, 0.4]] * 3)
    pd = f32([[0.1, 0.2, 0.3, 0.4], [0.0, 0.0, 0.0, 1.0], [0.0, 0.0, 0.0, 1.0]])
    r = OA.accept_sequence(pt, pd, np.array([1, 3, 3], np.int32), rej, f32([0.1, 0.4, 0.1]),
                           star, 4, 4, own, np.array([0, 0, 0], np.int32))
    assert (r["accept_len"], r["resample_node"], r["resample_token"]) == (1, 1, 1)
    # nothing accepted: the smallest root is the rejection node, own rows are not read
    pd0 = pd.copy()
    pd0[0] = pd[1]
    r = OA.accept_sequence(pt, pd0, np.array([3, 0, 0], np.int32), f32([0.99, 0.5, 0.5]),
                           f32([0.4, 0.5, 0.5]), star, 4, 4, own, np.array([7, 7, 7], np.int32))
    assert (r["accept_len"], r["resample_node"], r["resample_token"], r["err"]) == (0, 0, 1, 0)
    # own row -1 at the leaf: nothing; outside [-1, own_rows): error bit, nothing
    for rr, err in ((-1, 0), (2, OA.ERR_ROW), (-2, OA.ERR_ROW)):
        r = OA.accept_sequence(rows, rows, tok, ua, f32([0.9, 0.9, 0.5]), chain, 4, 4, own,
                               np.array([0, 0, rr], np.int32))
        assert (r["resample_node"], r["resample_token"], r["err"]) == (-1, -1, err)
    # a bad uniform at the leaf: the node is named, no token, the uniform bit
    r = OA.accept_sequence(rows, rows, tok, ua, f32([0.9, 0.9, 1.0]), chain, 4, 4, own,
                           np.array([-1, -1, 0], np.int32))
    assert (r["resample_node"], r["resample_token"], r["err"]) == (2, -1, OA.ERR_UNIFORM)
    # an all-zero own row: the node is named, no token, the zero-mass bit
    r = OA.accept_sequence(rows, rows, tok, ua, f32([0.9, 0.9, 0.5]), chain, 4, 4,
                           np.zeros((1, 4), np.float32), np.array([-1, -1, 0], np.int32))
    assert (r["resample_node"], r["resample_token"], r["err"]) == (2, -1, OA.ERR_ZERO_MASS)


def test_bonus_target_sampler_exact_grid_sweep():
    """The bonus sampler over all 2^24 grid uniforms: each token is drawn for exactly
    the floor-arithmetic share q_k 2^24 / Z of the grid (+-1), so the law is within
    V 2^-40 of norm(p_target); the sampler agrees with the sweep at every boundary."""
    rng = np.random.default_rng(12)
    vocab = 6
    pt = rng.random(vocab).astype(np.float32)
    pt[2] = 0.0
    pt /= pt.sum()
    q = OA.fixed_weights(pt, None)
    z = int(q.sum())
    csum = np.cumsum(q).astype(np.uint64)
    m = np.arange(1 << 24, dtype=np.uint64)
    zh, zl = np.uint64(z >> 24), np.uint64(z & ((1 << 24) - 1))
    t = m * zh + ((m * zl) >> np.uint64(24))
    tok = np.searchsorted(csum, t, side="right")
    counts = np.bincount(tok, minlength=vocab)
    assert counts[2] == 0
    for k in range(vocab):
        assert abs(int(counts[k]) - int(q[k]) * (1 << 24) / z) <= 1.0
    want = pt.astype(np.float64) / pt.astype(np.float64).sum()
    assert np.abs(counts / float(1 << 24) - want).max() <= 2.0 ** -23 + vocab * 2.0 ** -40
    picks = list(rng.integers(0, 1 << 24, 200))
    for k in range(vocab):
        b = -(-int(csum[k]) * (1 << 24) // z)
        picks += [b - 1, b, b + 1]
    for mm in picks:
        if 0 <= mm < (1 << 24):
            got, err = OA.target_token(pt, float(mm) * 2.0 ** -24)
            assert err == 0 and got == tok[mm]


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
