"""Pins of the probability-row oracle (CPU only): closed forms, a library routine,
invariances and planted mistakes."""
import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import oracle
from oracle.probs import ERR_ROW, softmax_rows


def test_uniform_and_two_valued_rows():
    v = 1000
    p, err = softmax_rows(np.zeros((1, v), np.float32))
    assert err == 0 and np.allclose(p, 1.0 / v, rtol=0, atol=1e-15)
    # logits a on k entries, b elsewhere: p = e^a / (k e^a + (v-k) e^b) (closed form)
    a, b, k = 3.0, -1.5, 7
    row = np.full(v, b, np.float32)
    row[:k] = a
    p, _ = softmax_rows(row[None])
    want_hi = np.exp(a) / (k * np.exp(a) + (v - k) * np.exp(b))
    want_lo = np.exp(b) / (k * np.exp(a) + (v - k) * np.exp(b))
    assert abs(p[0, 0] - want_hi) < 1e-15 and abs(p[0, -1] - want_lo) < 1e-17


def test_matches_library_softmax_and_sums_to_one():
    rng = np.random.default_rng(0)
    lg = (rng.standard_normal((5, 3001)) * np.sqrt(2.0)).astype(np.float32)
    p, _ = softmax_rows(lg)
    np.testing.assert_allclose(p, scipy_softmax(lg.astype(np.float64), axis=1), rtol=1e-13, atol=0)
    assert np.abs(p.sum(axis=1) - 1.0).max() < 1e-13


def test_shift_temperature_and_row_sharing():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((3, 500)).astype(np.float64)
    p, _ = softmax_rows(lg)
    q, _ = softmax_rows(lg + 123.25)                  # shift invariance
    assert np.abs(p - q).max() < 1e-14
    r, _ = softmax_rows(lg, inv_temperature=0.5)      # t scales the logits
    s, _ = softmax_rows(lg * 0.5)
    assert np.abs(r - s).max() < 1e-15
    shared, err = softmax_rows(lg, row_of=[2, 0, 0, 1, 2])
    assert err == 0
    for i, rr in enumerate([2, 0, 0, 1, 2]):
        assert np.array_equal(shared[i], p[rr])


def test_large_logits_do_not_overflow():
    """A planted 'no max subtraction' version overflows here; the oracle does not."""
    row = np.array([[1000.0, 999.0, 0.0]])
    p, _ = softmax_rows(row)
    e1 = np.exp(-1.0)
    assert np.allclose(p[0, :2], [1 / (1 + e1), e1 / (1 + e1)], rtol=1e-15)
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(row) / np.exp(row).sum()
    assert not np.all(np.isfinite(naive))


def test_bad_row_index():
    p, err = softmax_rows(np.zeros((2, 4)), row_of=[0, 2, -1, 1])
    assert err == ERR_ROW
    assert np.all(p[1] == 0) and np.all(p[2] == 0) and np.allclose(p[0], 0.25)


# ---- kept-set rows: page [P525] §2.2.1-2.2.2 (q~ = q 1[x in R] / Z) ----------------
from oracle.acceptance import ratio_accepts, residual_token
from oracle.probs import softmax_rows_kept


def test_kept_all_tokens_is_the_plain_softmax():
    """R = the whole vocabulary (listed shuffled, with padding and repeats)."""
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((3, 257)).astype(np.float32)
    keep = np.full((3, 600), -1, np.int64)
    for r in range(3):
        ids = np.concatenate([rng.permutation(257), rng.integers(0, 257, 200)])
        keep[r, :len(ids)] = ids
    p, err = softmax_rows_kept(lg, keep, inv_temperature=0.7)
    want, _ = softmax_rows(lg, inv_temperature=0.7)
    assert err == 0
    np.testing.assert_allclose(p, want, rtol=1e-12, atol=0)


def test_kept_row_is_the_renormalised_restriction():
    """q~ = q * 1[R] / Z from the library softmax of the whole row (page §2.2.1), and
    the page's logits edit of §2.2.2 (log(1/Z) added on R, -inf elsewhere) gives the
    same row."""
    rng = np.random.default_rng(4)
    lg = (rng.standard_normal((4, 1000)) * 3).astype(np.float32)
    keep = np.full((4, 40), -1, np.int64)
    for r in range(4):
        k = rng.integers(1, 40)
        keep[r, :k] = rng.choice(1000, k, replace=False)
    p, err = softmax_rows_kept(lg, keep)
    assert err == 0
    q = scipy_softmax(lg.astype(np.float64), axis=1)
    for r in range(4):
        ids = keep[r][keep[r] >= 0]
        mask = np.zeros(1000, bool)
        mask[ids] = True
        z = q[r, mask].sum()
        want = np.where(mask, q[r] / z, 0.0)
        np.testing.assert_allclose(p[r], want, rtol=1e-11, atol=1e-300)
        edited = np.where(mask, lg[r].astype(np.float64) + np.log(1.0 / z), -np.inf)
        np.testing.assert_allclose(p[r], scipy_softmax(edited), rtol=1e-11, atol=1e-300)
        assert p[r, ~mask].max(initial=0.0) == 0.0


def test_kept_rows_shared_contexts_and_errors():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((3, 50))
    keep = np.array([[3, 3, 7, -1], [-1, -1, -1, -1], [1, 50, 2, -1]])
    p, err = softmax_rows_kept(lg, keep, row_of=[0, 0, 1, 2, 3])
    assert err == ERR_ROW | oracle.ERR_ZERO_MASS | oracle.ERR_TOKEN
    e = np.exp(lg[0, [3, 7]] - lg[0, [3, 7]].max())
    np.testing.assert_allclose(p[0, [3, 7]], e / e.sum(), rtol=1e-15)   # the repeat counts once
    assert np.array_equal(p[0], p[1])
    assert not p[2:].any()      # empty set, an id past the vocabulary, a bad row index
    bad, err = softmax_rows_kept(lg, np.array([[0, -2, 1, -1]] * 3))
    assert err == oracle.ERR_TOKEN and not bad.any()


def test_kept_rows_make_one_speculative_step_exact():
    """Tokens drawn from the pruned draft are judged against the kept-set row: the
    first emitted token (accepted draft, else a residual draw) then follows the target
    row exactly.  Dividing by the unpruned q instead (the shift page §2.2.1 warns of)
    does not.  Acceptance and residual draws go through the acceptance oracle, over a
    grid of uniforms."""
    rng = np.random.default_rng(6)
    v, grid = 6, 2048
    dl = rng.standard_normal((1, v))
    tl = rng.standard_normal((1, v))
    keep = np.array([[4, 1, 2, -1, 5]])
    qk, err = softmax_rows_kept(dl, keep)
    assert err == 0
    pt = softmax_rows(tl)[0][0].astype(np.float32)
    us = ((np.arange(grid) + 0.5) / grid).astype(np.float32)

    def first_token_dist(pd_row):
        pd_row = pd_row.astype(np.float32)
        res = np.zeros(v)
        for u in us:
            tok, e = residual_token(pt, pd_row, float(u))
            assert e == 0
            res[tok] += 1.0 / grid
        dist = np.zeros(v)
        for x in range(v):
            if qk[0, x] == 0:
                continue
            acc = np.mean([ratio_accepts(float(u), pd_row[x], pt[x]) for u in us])
            dist[x] += qk[0, x] * acc
            dist += qk[0, x] * (1.0 - acc) * res
        return dist

    assert np.abs(first_token_dist(qk[0]) - pt).max() < 4.0 / grid
    q = softmax_rows(dl)[0][0]
    unpruned = np.where(qk[0] > 0, q, 0.0)
    assert np.abs(first_token_dist(unpruned) - pt).max() > 0.02


def test_kept_rows_large_logits():
    """The maximum over the kept set is subtracted first: logits near 1000 stay finite."""
    p, err = softmax_rows_kept(np.array([[1000.0, 999.0, 5000.0]]), np.array([[0, 1, -1]]))
    e1 = np.exp(-1.0)
    assert err == 0
    np.testing.assert_allclose(p[0], [1 / (1 + e1), e1 / (1 + e1), 0.0], rtol=1e-15)
