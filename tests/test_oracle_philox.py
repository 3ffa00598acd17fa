"""Pins of the counter-based generator oracle (page [P537] §8.2; Philox4x64-10 of
Salmon et al., SC'11) against numpy's independent Philox4x64-10 bit generator,
exact 24-bit mapping, and the counter layout's properties."""
import numpy as np
import pytest
from scipy import stats

from oracle import philox as P

MASK256 = (1 << 256) - 1


def _words(x: int, n: int):
    return [(x >> (64 * i)) & P.MASK64 for i in range(n)]


def _int(words) -> int:
    return sum(int(w) << (64 * i) for i, w in enumerate(words))


def _numpy_blocks(counter, key, blocks: int):
    """numpy's Philox output for `blocks` consecutive counters starting at `counter`.
    numpy increments its 256-bit counter before each block, so it starts one below."""
    start = (_int(counter) - 1) & MASK256
    bg = np.random.Philox(counter=np.array(_words(start, 4), dtype=np.uint64),
                          key=np.array([int(k) for k in key], dtype=np.uint64))
    raw = [int(x) for x in bg.random_raw(4 * blocks)]
    return [tuple(raw[4 * i:4 * i + 4]) for i in range(blocks)]


def _cases():
    rng = np.random.default_rng(20260501)
    out = [((0, 0, 0, 0), (0, 0)),
           ((P.MASK64,) * 4, (P.MASK64, P.MASK64)),
           ((1, 0, 0, 0), (0, 1)),
           ((5, 7, 11, 13), (0x1234, 0x5678))]
    for _ in range(40):
        c = tuple(int(x) for x in rng.integers(0, 2**64, size=4, dtype=np.uint64))
        k = tuple(int(x) for x in rng.integers(0, 2**64, size=2, dtype=np.uint64))
        out.append((c, k))
    return out


@pytest.mark.parametrize("counter,key", _cases())
def test_cipher_matches_numpy_philox(counter, key):
    assert P.philox4x64(counter, key) == _numpy_blocks(counter, key, 1)[0]


def test_consecutive_counters_with_carry_match_numpy():
    # word 0 wraps after two blocks: the carry runs into word 1 (numpy's increment)
    counter, key = (P.MASK64 - 1, 3, 0, 9), (0xdeadbeef, 42)
    got = []
    c = _int(counter)
    for _ in range(5):
        got.append(P.philox4x64(_words(c, 4), key))
        c = (c + 1) & MASK256
    assert got == _numpy_blocks(counter, key, 5)


def test_planted_round_mistakes_fail_the_numpy_pin(monkeypatch):
    counter, key = (5, 7, 11, 13), (0x1234, 0x5678)
    ref = _numpy_blocks(counter, key, 1)[0]
    assert P.philox4x64(counter, key, rounds=9) != ref
    monkeypatch.setattr(P, "PHILOX_W1", P.PHILOX_W0)
    assert P.philox4x64(counter, key) != ref
    monkeypatch.undo()
    monkeypatch.setattr(P, "PHILOX_M1", P.PHILOX_M0)
    assert P.philox4x64(counter, key) != ref


def test_uniform24_is_exact_in_fp32():
    assert P.uniform24(0) == 0.0
    assert P.uniform24(1 << 40) == 2.0**-24
    assert P.uniform24(P.MASK64) == 1.0 - 2.0**-24
    rng = np.random.default_rng(7)
    for w in rng.integers(0, 2**64, size=1000, dtype=np.uint64):
        u = P.uniform24(int(w))
        assert float(np.float32(u)) == u
        assert u * 2**24 == (int(w) >> 40)
        assert 0.0 <= u < 1.0


def test_node_counter_layout():
    # (local node, 32-bit depth, step, 64-bit request id)
    assert P.node_counter(3, 2, 9, 17) == (3, 2, 9, 17)
    assert P.node_counter(0, -1, 0, -1) == (0, P.MASK32, 0, P.MASK64)


def _trees():
    cu = [0, 5, 5, 12]
    depth = [1, 2, 2, 3, 1, 1, 2, 3, 4, 2, 3, 1]
    return cu, depth


def test_node_uniforms_per_sequence_independent_of_batch_layout():
    cu, depth = _trees()
    req = [101, 202, 303]
    ua, ur = P.node_uniforms(9, 0, 4, req, depth, cu)
    # the same sequences alone, or in another order, draw the same numbers
    for b, (lo, hi) in enumerate(zip(cu[:-1], cu[1:])):
        a1, r1 = P.node_uniforms(9, 0, 4, [req[b]], depth[lo:hi], [0, hi - lo])
        assert np.array_equal(a1, ua[lo:hi]) and np.array_equal(r1, ur[lo:hi])
    assert len(ua) == 12 and ua.dtype == np.float32


def test_node_uniforms_change_with_each_counter_and_key_word():
    cu, depth = _trees()
    req = [101, 202, 303]
    base = P.node_uniforms(9, 0, 4, req, depth, cu)
    variants = [P.node_uniforms(10, 0, 4, req, depth, cu),                 # seed
                P.node_uniforms(9, 1, 4, req, depth, cu),                  # purpose
                P.node_uniforms(9, 0, 5, req, depth, cu),                  # step
                P.node_uniforms(9, 0, 4, [102, 202, 304], depth, cu),      # request
                P.node_uniforms(9, 0, 4, req, [d + 1 for d in depth], cu)]  # tree level
    for ua, ur in variants:
        assert np.mean(ua != base[0]) > 0.9
    # acceptance and resample words differ
    assert np.mean(base[0] != base[1]) > 0.9


def test_node_uniforms_are_uniform():
    n = 20000
    cu = [0, n]
    ua, ur = P.node_uniforms(123, 0, 1, [7], np.arange(n) % 13 + 1, cu)
    assert stats.kstest(ua.astype(np.float64), "uniform").pvalue > 1e-3
    assert stats.kstest(ur.astype(np.float64), "uniform").pvalue > 1e-3
    # independent words: correlation near zero
    assert abs(np.corrcoef(ua, ur)[0, 1]) < 0.03
