"""Pins of the FP8 matrix-core attention oracle (page [P537] §9.2: Q, K, V in E4M3
with one scale per 128 elements; power-of-two E8M0 scales): E4M3 rounding against
torch's float8_e4m3fn cast, the scale rule's closed forms and defining property,
the round-trip error bound, and reduction to the already pinned FP8 and plain
attention oracles on exactly representable inputs."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_mma as M
from oracle.fp8 import e4m3_table


def torch_e4m3(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_rounding_matches_torch_on_random_values():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000),
                        rng.normal(0, 1e-2, 5000), rng.uniform(-2**-6, 2**-6, 5000)]).astype(np.float32)
    np.testing.assert_array_equal(M.e4m3_round(x), torch_e4m3(x))


def test_rounding_matches_torch_on_every_tie_and_value():
    vals = e4m3_table()[:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)       # exact ties (fp32-representable)
    assert np.all(mids.astype(np.float64) == (vals[:-1] + vals[1:]) / 2)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    x = np.concatenate([vals.astype(np.float32), mids, near])
    x = np.concatenate([x, -x]).astype(np.float32)
    np.testing.assert_array_equal(M.e4m3_round(x), torch_e4m3(x))
    # every code decodes back to itself
    np.testing.assert_array_equal(M.e4m3_round(vals.astype(np.float32)), np.arange(0x7F, dtype=np.uint8))


def test_planted_round_half_up_fails_the_tie_pin():
    vals = e4m3_table()[:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    lo = np.searchsorted(vals, mids) - 1
    half_up = (lo + 1).astype(np.uint8)              # the mistake: ties always round up
    assert np.any(half_up != torch_e4m3(mids))


def test_scale_rule_closed_forms():
    assert M.scale_shift(448.0) == 0
    assert M.scale_shift(np.float32(448.0) * np.float32(1 + 2**-23)) == 1
    assert M.scale_shift(224.0) == -1
    assert M.scale_shift(1.0) == -8          # 1 <= 448 * 2^-8 = 1.75, 1 > 448 * 2^-9
    assert M.scale_shift(1.75) == -8
    assert M.scale_shift(1.7500001) == -7
    assert M.scale_shift(0.0) == 0
    assert M.scale_shift(3.0e38) == 120
    assert M.scale_shift(np.float32(2.0**-140)) == -127  # clamped (2^-140 <= 448 * 2^-148)


def test_scale_rule_defining_property():
    rng = np.random.default_rng(11)
    amax = np.exp(rng.uniform(np.log(1e-30), np.log(1e30), 100000)).astype(np.float32)
    s = M.scale_shift(amax)
    r = amax.astype(np.float64) * np.exp2(-s.astype(np.float64))
    # the smallest power of two: amax fits, half of it would not
    assert np.all(r <= 448.0) and np.all(r > 224.0)


def test_quantize_round_trip_error_bound():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 1, (2000, 128)).astype(np.float32) * np.exp(rng.normal(0, 3, (2000, 1))).astype(np.float32)
    codes, exps = M.quantize_rows(x)
    y = M.dequantize_rows(codes, exps)
    s = np.exp2(exps.astype(np.float64) - 127)[:, None]
    err = np.abs(y - x)
    # normal range: half a step = 2^-4 relative; subnormal range: half of 2^-9 * scale
    bound = np.maximum(np.abs(x) * 2.0**-4, 2.0**-10 * s)
    assert np.all(err <= bound * (1 + 1e-12))
    # the row maximum maps into (224, 448] exactly scaled
    assert np.all(np.max(np.abs(y), axis=1) / s[:, 0] <= 448)


def test_power_of_two_rescaling_moves_only_the_exponent():
    rng = np.random.default_rng(8)
    x = rng.normal(0, 1, (50, 128)).astype(np.float32)
    c0, e0 = M.quantize_rows(x)
    c1, e1 = M.quantize_rows(x * np.float32(2.0**5))
    np.testing.assert_array_equal(c0, c1)
    np.testing.assert_array_equal(e1.astype(int), e0.astype(int) + 5)


def _exact_case(seed=2):
    """Rows built as code values times a power of two, each with a +-448 element, so
    that quantization is exact; returns fp32 arrays and their codes/exponents."""
    rng = np.random.default_rng(seed)
    table = e4m3_table()

    def rows(shape):
        codes = rng.integers(0, 0x7F, size=shape + (128,)).astype(np.uint8)
        codes |= (rng.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
        codes[..., 0] = 0x7E                           # 448: the row's maximum
        exps = rng.integers(120, 128, size=shape).astype(np.uint8)
        vals = (table[codes] * np.exp2(exps.astype(np.float64) - 127)[..., None]).astype(np.float32)
        return vals, codes, exps
    return rows


def test_exact_inputs_reduce_to_the_fp32_scale_oracle_and_plain_attention():
    rows = _exact_case()
    hq, hkv, nb = 4, 2, 3
    parent = np.array([-1, 0, 0, 1, -1], np.int32)
    cu = np.array([0, 5], np.int32)
    q, _, _ = rows((5, hq))
    kt, kt8, kte = rows((5, hkv))
    vt, vt8, vte = rows((5, hkv))
    _, k8, ke = rows((nb, hkv, 64))
    _, v8, ve = rows((nb, hkv, 64))
    bt = np.array([[2, 0, 1]], np.int32)
    plen = np.array([150], np.int32)
    scale = 1.0 / np.sqrt(128.0)
    got = M.tree_attention_fp8mma(q, k8, v8, ke, ve, bt, plen, kt8, vt8, kte, vte, cu, parent, hq, hkv,
                                  scale)
    ks = np.exp2(ke.astype(np.float64) - 127)
    vs = np.exp2(ve.astype(np.float64) - 127)
    want = oracle.tree_attention_fp8(q.astype(np.float64), k8, v8, ks, vs, bt, plen, kt.astype(np.float64),
                                     vt.astype(np.float64), cu, parent, hq, hkv, scale)
    np.testing.assert_allclose(got[0], want[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[1], want[1], rtol=0, atol=1e-12)
    # and the round trip of exact rows is the identity
    np.testing.assert_array_equal(M.round_trip(q), q.astype(np.float64))


def test_quantization_error_is_what_separates_it_from_plain_attention():
    """On N(0,1) inputs the FP8 result differs from the fp64 result of the unquantized
    values by the quantization only: replacing q, tree K/V by their round trips in
    plain attention gives the same numbers."""
    rng = np.random.default_rng(4)
    hq, hkv = 2, 1
    parent = np.array([-1, 0, 1], np.int32)
    cu = np.array([0, 3], np.int32)
    q = rng.normal(0, 1, (3, hq, 128)).astype(np.float32)
    kt = rng.normal(0, 1, (3, hkv, 128)).astype(np.float32)
    vt = rng.normal(0, 1, (3, hkv, 128)).astype(np.float32)
    k8, ke = M.quantize_rows(rng.normal(0, 1, (2, hkv, 64, 128)).astype(np.float32))
    v8, ve = M.quantize_rows(rng.normal(0, 1, (2, hkv, 64, 128)).astype(np.float32))
    bt = np.array([[1, 0]], np.int32)
    plen = np.array([100], np.int32)
    kt8, kte = M.quantize_rows(kt)
    vt8, vte = M.quantize_rows(vt)
    got = M.tree_attention_fp8mma(q, k8, v8, ke, ve, bt, plen, kt8, vt8, kte, vte, cu, parent, hq, hkv,
                                  0.1)
    want = oracle.tree_attention(M.round_trip(q), M.dequantize_rows(k8, ke), M.dequantize_rows(v8, ve),
                                 bt, plen, M.round_trip(kt), M.round_trip(vt), cu, parent, hq, hkv, 0.1)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])
    plain = oracle.tree_attention(q.astype(np.float64), M.dequantize_rows(k8, ke), M.dequantize_rows(v8, ve),
                                  bt, plen, kt.astype(np.float64), vt.astype(np.float64), cu, parent, hq, hkv, 0.1)
    d = np.abs(got[0] - plain[0]).max()
    assert 0 < d < 0.05
