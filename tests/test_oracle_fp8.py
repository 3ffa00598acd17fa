"""Pins of the FP8 (E4M3) cache oracle (CPU only): the byte table against a
library decoder and the format's closed forms, dequantization identities, and the
composition with attention checked through invariances."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import tree_attention
from oracle.fp8 import dequantize, e4m3_table, e4m3_value, tree_attention_fp8


def torch_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_table_matches_library_decoder():
    ours, lib = e4m3_table(), torch_table()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan) and list(np.flatnonzero(nan)) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan], lib[~nan])


def test_closed_forms():
    assert e4m3_value(0x7E) == 448.0 and e4m3_value(0xFE) == -448.0      # largest finite
    assert e4m3_value(0x01) == 2.0 ** -9                                   # smallest subnormal
    assert e4m3_value(0x07) == 7 * 2.0 ** -9                               # largest subnormal
    assert e4m3_value(0x08) == 2.0 ** -6                                   # smallest normal
    assert e4m3_value(0x38) == 1.0 and e4m3_value(0xB8) == -1.0
    assert e4m3_value(0x00) == 0.0 and np.signbit(e4m3_value(0x80))
    # values increase with the code over the positive half (the format is monotone)
    pos = e4m3_table()[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_planted_bias_error_is_caught():
    """A decoder with exponent bias 8 (the other FP8 E4M3 convention) fails the pin."""
    def wrong(code):
        e, m = (code >> 3) & 0xF, code & 7
        return (m / 8.0) * 2.0 ** -7 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 8)
    lib = torch_table()
    assert any(wrong(c) != lib[c] for c in range(0x7F))


def test_dequantize_is_byte_value_times_row_scale():
    rng = np.random.default_rng(3)
    codes = W.fp8_random_codes(rng, (3, 2, 64, 8))
    scale = rng.uniform(0.01, 2.0, (3, 2, 64)).astype(np.float32)
    deq = dequantize(codes, scale)
    lib = torch_table()[codes]
    assert np.array_equal(deq / scale.astype(np.float64)[..., None], lib)


def test_generator_round_trip_error_bound():
    """The input generator's codes decode to within half a step of the original:
    2^-4 relative for normal codes, 2^-10 * scale absolute in the subnormal range."""
    case = W.make_case("q", [W.tree_heap(3)], [200], 4, 2, 128, W.DT_BF16, 10, 5, with_probs=False)
    x = W.to_f64(case.k_cache, case.dtype)
    codes, scale = W.fp8_cache(case.k_cache, case.dtype)
    deq = dequantize(codes, scale)
    s = scale.astype(np.float64)[..., None]
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(deq - x) <= bound)
    assert np.all(np.abs(deq) <= 448.0 * s * (1 + 1e-7))
    assert np.isfinite(deq).all()


def _fp8_case(seed):
    case = W.make_case("f", [W.tree_random(np.random.default_rng(seed), 20, 5)], [150], 4, 2, 128,
                       W.DT_BF16, 10, seed, with_probs=False)
    rng = np.random.default_rng(seed + 100)
    k8, v8 = (W.fp8_random_codes(rng, case.k_cache.shape) for _ in range(2))
    ks, vs = (rng.uniform(1e-3, 4e-3, case.k_cache.shape[:3]).astype(np.float32) for _ in range(2))
    f = lambda a: W.to_f64(a, case.dtype)
    return case, k8, v8, ks, vs, f


def test_value_scale_scales_the_output():
    """Doubling every V scale doubles the output exactly: the softmax weights do
    not change.  The single tree node's own V is zero, so every value that
    carries weight comes from the prefix."""
    case = W.make_case("p", [W.tree_chain(1)], [130], 2, 1, 128, W.DT_BF16, 10, 7, with_probs=False)
    rng = np.random.default_rng(8)
    k8, v8 = (W.fp8_random_codes(rng, case.k_cache.shape) for _ in range(2))
    ks, vs = (rng.uniform(1e-3, 4e-3, case.k_cache.shape[:3]).astype(np.float32) for _ in range(2))
    f = lambda a: W.to_f64(a, case.dtype)
    vt0 = np.zeros_like(f(case.v_tree))
    args = (case.block_table, case.prefix_len, f(case.k_tree), vt0, case.cu_nodes, case.parent,
            case.hq, case.hkv, case.scale)
    o1, l1 = tree_attention_fp8(f(case.q), k8, v8, ks, vs, *args)
    o2, l2 = tree_attention_fp8(f(case.q), k8, v8, ks, 2 * vs, *args)
    assert np.array_equal(o2, 2 * o1) and np.array_equal(l1, l2)


def test_key_scale_acts_as_softmax_scale():
    """Multiplying every K scale (and the tree K) by c equals multiplying the
    softmax scale by c."""
    case, k8, v8, ks, vs, f = _fp8_case(11)
    c = 1.75
    common = (case.block_table, case.prefix_len)
    ks_c = ks.astype(np.float64) * c  # exact in fp64
    o1, l1 = tree_attention_fp8(f(case.q), k8, v8, ks_c, vs, *common, f(case.k_tree) * c,
                                f(case.v_tree), case.cu_nodes, case.parent, case.hq, case.hkv,
                                case.scale)
    o2, l2 = tree_attention_fp8(f(case.q), k8, v8, ks, vs, *common, f(case.k_tree), f(case.v_tree),
                                case.cu_nodes, case.parent, case.hq, case.hkv, case.scale * c)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12


def test_unit_scales_reduce_to_the_plain_cache():
    """With scale 1 the FP8 oracle is attention over the decoded bytes, computed
    here from torch's decoder rather than the oracle's own table."""
    case, k8, v8, _, _, f = _fp8_case(12)
    ones = np.ones(case.k_cache.shape[:3], np.float32)
    lib = torch_table()
    o1, l1 = tree_attention_fp8(f(case.q), k8, v8, ones, ones, case.block_table, case.prefix_len,
                                f(case.k_tree), f(case.v_tree), case.cu_nodes, case.parent, case.hq,
                                case.hkv, case.scale)
    o2, l2 = tree_attention(f(case.q), lib[k8], lib[v8], case.block_table, case.prefix_len,
                            f(case.k_tree), f(case.v_tree), case.cu_nodes, case.parent, case.hq,
                            case.hkv, case.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
