"""GPU parity of the FP8 matrix-core path against its oracle (page [P537] §9.2: Q, K,
V in E4M3 with one power-of-two scale per 128 elements): the row quantizer bit for
bit, then tree_verify_attention_fp8 element by element."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_mma as M

pytestmark = pytest.mark.gpu


def quant_rows_case(rng, rows: int) -> np.ndarray:
    """fp32 rows spanning the awkward cases of the scale rule and the rounding."""
    x = rng.normal(0, 1, (rows, 128)).astype(np.float32)
    x *= np.exp(rng.normal(0, 4, (rows, 1))).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2] = 0.0
    x[2, 7] = -3.5
    x[3] = 448.0 * 2.0 ** np.arange(-64, 64).astype(np.float32)[:128]
    x[4] = 1e-39                          # fp32 subnormal row
    x[4, ::3] = -1e-40
    x[5] = np.float32(448.0) * np.float32(1 + 2**-23)
    vals = oracle.e4m3_table()[:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x[6] = np.concatenate([mids, [448.0, 1.0]]).astype(np.float32)  # every tie, row max 448
    x[7] = -x[6]
    return x


@pytest.mark.parametrize("rows", [1, 13, 1000, 4097])
def test_quantize_rows_fp32_bitexact(gpu_lib, rows):
    rng = np.random.default_rng(rows)
    x = quant_rows_case(rng, max(rows, 8))[:rows] if rows < 8 else quant_rows_case(rng, rows)
    codes, exps = gpu_lib.tree_quantize_rows_e4m3(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    want_c, want_e = M.quantize_rows(x)
    np.testing.assert_array_equal(exps.cpu().numpy(), want_e)
    np.testing.assert_array_equal(codes.cpu().numpy(), want_c)


@pytest.mark.parametrize("rows", [7, 2048])
def test_quantize_rows_bf16_bitexact(gpu_lib, rows):
    rng = np.random.default_rng(100 + rows)
    x = quant_rows_case(rng, max(rows, 8))[:rows]
    xb = torch.from_numpy(x).to(torch.bfloat16)
    codes, exps = gpu_lib.tree_quantize_rows_e4m3(xb.cuda())
    torch.cuda.synchronize()
    want_c, want_e = M.quantize_rows(xb.float().numpy())
    np.testing.assert_array_equal(exps.cpu().numpy(), want_e)
    np.testing.assert_array_equal(codes.cpu().numpy(), want_c)


def test_quantize_rows_shapes(gpu_lib):
    x = torch.randn(3, 5, 128, device="cuda", dtype=torch.bfloat16)
    codes, exps = gpu_lib.tree_quantize_rows_e4m3(x)
    assert codes.shape == (3, 5, 128) and exps.shape == (3, 5)
    empty_c, empty_e = gpu_lib.tree_quantize_rows_e4m3(torch.empty(0, 128, device="cuda"))
    assert empty_c.numel() == 0 and empty_e.numel() == 0


# ---- tree_verify_attention_fp8 against oracle.tree_attention_fp8mma ----------------
import workloads as W
from tests._helpers import gpu_index, rows_of, sample_nodes, to_f64

TOL = 2e-2  # as for bf16: P and V reach the P.V product in bf16; Q and K as the oracle has them


def mma8_inputs(case, mode, seed):
    """(k8, v8, k_exp, v_exp): 'codes' = uniform finite bytes with exponents 113..120
    (values up to 448 * 2^-7 = 3.5, so that the bf16 output bar of 2e-2 still applies);
    'quant' = the case's own K/V rows quantized by the oracle's rule."""
    if mode == "codes":
        rng = np.random.default_rng(seed)
        k8, v8 = (W.fp8_random_codes(rng, case.k_cache.shape) for _ in range(2))
        ke, ve = (rng.integers(113, 121, case.k_cache.shape[:3]).astype(np.uint8) for _ in range(2))
        return k8, v8, ke, ve
    k8, ke = M.quantize_rows(W.to_f64(case.k_cache, case.dtype).astype(np.float32))
    v8, ve = M.quantize_rows(W.to_f64(case.v_cache, case.dtype).astype(np.float32))
    return k8, v8, ke, ve


def tree_codes(case):
    """The tree's K/V in the FP8 cache format, by the oracle's rule on the CPU."""
    f = lambda a: W.to_f64(a, case.dtype).astype(np.float32)
    kt8, kte = M.quantize_rows(f(case.k_tree))
    vt8, vte = M.quantize_rows(f(case.v_tree))
    return kt8, vt8, kte, vte


def run_mma8(tv, case, k8, v8, ke, ve):
    dev = W.case_to_device(case, probs=False)
    mn = max(1, case.max_nodes)
    anc, _, _, err = gpu_index(tv, case, dev, mn)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    kt8, vt8, kte, vte = tree_codes(case)
    out, lse, err = tv.tree_verify_attention_fp8(
        dev["q"], t(k8), t(v8), t(ke), t(ve), dev["block_table"], dev["prefix_len"],
        t(kt8), t(vt8), t(kte), t(vte), dev["cu_nodes"], anc, mn, case.max_prefix, err=err)
    torch.cuda.synchronize()
    return out, lse, int(err.item())


def check_mma8(tv, case, mode, seed, nodes=None):
    k8, v8, ke, ve = mma8_inputs(case, mode, seed)
    print(f"fp8-mma case {case.name} mode {mode} B{case.batch} P{list(case.prefix_len)[:4]} "
          f"N{case.total_nodes}", flush=True)
    out, lse, err = run_mma8(tv, case, k8, v8, ke, ve)
    assert err == 0
    kt8, vt8, kte, vte = tree_codes(case)
    f = lambda a: W.to_f64(a, case.dtype).astype(np.float32)
    want, want_lse = M.tree_attention_fp8mma(f(case.q), k8, v8, ke, ve, case.block_table,
                                             case.prefix_len, kt8, vt8, kte, vte, case.cu_nodes,
                                             case.parent, case.hq, case.hkv, case.scale, nodes=nodes)
    got, got_lse = to_f64(out), lse.cpu().numpy().astype(np.float64)
    if nodes is not None:
        rows = rows_of(case, nodes)
        got, want, got_lse, want_lse = got[rows], want[rows], got_lse[rows], want_lse[rows]
    assert np.isfinite(got).all()
    e_out = np.abs(got - want).max() if got.size else 0.0
    e_lse = np.abs(got_lse - want_lse).max() if got.size else 0.0
    print(f"  max |out - oracle| {e_out:.3e}, max |lse - oracle| {e_lse:.3e}", flush=True)
    assert e_out <= TOL, e_out
    assert e_lse <= TOL, e_lse


SMALL = {
    # name: (parents, prefix_lens, hq, hkv)
    "ragged_gqa": ([W.tree_chain(1), W.tree_random(np.random.default_rng(5), 37, 6),
                    W.tree_random(np.random.default_rng(6), 130, 8)], [0, 70, 200], 8, 2),
    "short_prefix": ([W.tree_heap(7), W.tree_heap(7)], [128, 64], 8, 1),
    "split_prefix": ([W.tree_heap(31)], [1000], 4, 4),
    "long_gqa": ([W.tree_random(np.random.default_rng(9), 200, 8)], [5000], 8, 2),
    "no_prefix": ([W.tree_star(100)], [0], 4, 2),
    "ragged_batch": ([W.tree_random(np.random.default_rng(10), 60, 5), W.tree_chain(5),
                      W.tree_random(np.random.default_rng(11), 300, 12)], [1000, 37, 513], 4, 4),
    "many_pairs": ([W.tree_heap(5)] * 64, [64 + 7 * b for b in range(64)], 32, 8),
}


@pytest.mark.parametrize("mode", ["codes", "quant"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_fp8_mma_attention_small(gpu_lib, name, mode):
    parents, plens, hq, hkv = SMALL[name]
    case = W.make_case(name, parents, plens, hq, hkv, 128, W.DT_BF16, 10, 23, with_probs=False)
    check_mma8(gpu_lib, case, mode, seed=31)


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_fp8_mma_attention_full_configs(gpu_lib, index):
    """The four bf16 workloads with quantized caches in the benchmark's launch
    configuration: every node of the LLaVA-like tree, sampled nodes of every
    sequence of the others."""
    case = W.make_config(index, with_probs=False)
    nodes = None if index == 1 else sample_nodes(case, 12 if case.batch <= 8 else 2, seed=index)
    check_mma8(gpu_lib, case, "quant", seed=index, nodes=nodes)


FP8_TAIL = ([W.tree_kary_levels(8, 3)] * 5 + [W.tree_random(np.random.default_rng(12), 300, 8),
             W.tree_chain(1), np.zeros(0, np.int32)], [300, 0, 4096, 64, 65, 1000, 130, 5], 32, 8)


@pytest.mark.parametrize("mode", ["codes", "quant"])
def test_fp8_mma_attention_tail_pieces(gpu_lib, mode):
    parents, plens, hq, hkv = FP8_TAIL
    case = W.make_case("fp8tail", parents, plens, hq, hkv, 128, W.DT_BF16, 10, 27, with_probs=False)
    check_mma8(gpu_lib, case, mode, seed=8, nodes=sample_nodes(case, 8, seed=2))


def test_fp8_mma_attention_repeatable(gpu_lib):
    case = W.make_config(3, with_probs=False)
    k8, v8, ke, ve = mma8_inputs(case, "quant", 3)
    first, first_lse, _ = run_mma8(gpu_lib, case, k8, v8, ke, ve)
    again, again_lse, err = run_mma8(gpu_lib, case, k8, v8, ke, ve)
    assert err == 0 and torch.equal(first, again) and torch.equal(first_lse, again_lse)


def test_fp8_mma_bad_block_sets_error(gpu_lib):
    case = W.make_case("badblk", [W.tree_heap(7)], [300], 4, 2, 128, W.DT_BF16, 10, 3,
                       with_probs=False)
    case.block_table[0, 2] = case.num_blocks  # outside the pool
    k8, v8, ke, ve = mma8_inputs(case, "codes", 4)
    _, _, err = run_mma8(gpu_lib, case, k8, v8, ke, ve)
    assert err & gpu_lib.TV_ERR_BLOCK
