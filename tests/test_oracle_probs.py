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
