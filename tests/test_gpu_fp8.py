"""GPU parity of tree attention over an FP8 (E4M3) prefix cache.

The HIP path (tree_verify_attention_fp8kv through the C ABI) against the fp64
oracle evaluated on the dequantized cache (oracle.fp8).  Bar: max-abs 2e-2 on
the bf16 output and the log-sum-exp, as for the bf16 cache: each dequantized
element is rounded to bf16 once (relative 2^-9), the same error a bf16 cache
carries.  Caches are either uniform over every finite E4M3 byte (every code
decoded at least once) or N(0,1) K/V quantized with per-row scales.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle.fp8 import tree_attention_fp8
from _helpers import gpu_index, rows_of, sample_nodes, to_f64

pytestmark = pytest.mark.gpu

TOL = 2e-2


def fp8_inputs(case, mode, seed):
    """(k8, v8, k_scale, v_scale) for a case: 'codes' = uniform finite bytes with
    scales in [1/448, 4/448]; 'quant' = the case's own K/V quantized per row."""
    if mode == "codes":
        rng = np.random.default_rng(seed)
        k8, v8 = (W.fp8_random_codes(rng, case.k_cache.shape) for _ in range(2))
        ks, vs = (rng.uniform(1.0 / 448, 4.0 / 448, case.k_cache.shape[:3]).astype(np.float32)
                  for _ in range(2))
        return k8, v8, ks, vs
    k8, ks = W.fp8_cache(case.k_cache, case.dtype)
    v8, vs = W.fp8_cache(case.v_cache, case.dtype)
    return k8, v8, ks, vs


def run_fp8(tv, case, k8, v8, ks, vs):
    dev = W.case_to_device(case, probs=False)
    mn = max(1, case.max_nodes)
    anc, _, _, err = gpu_index(tv, case, dev, mn)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    out, lse, err = tv.tree_verify_attention_fp8kv(
        dev["q"], t(k8), t(v8), t(ks), t(vs), dev["block_table"],
        dev["prefix_len"], dev["k_tree"], dev["v_tree"], dev["cu_nodes"], anc, mn, case.max_prefix,
        err=err)
    torch.cuda.synchronize()
    return out, lse, int(err.item())


def check_fp8(tv, case, mode, seed, nodes=None):
    k8, v8, ks, vs = fp8_inputs(case, mode, seed)
    print(f"fp8 case {case.name} mode {mode} B{case.batch} P{list(case.prefix_len)[:4]} "
          f"N{case.total_nodes}", flush=True)
    out, lse, err = run_fp8(tv, case, k8, v8, ks, vs)
    assert err == 0
    f = lambda a: W.to_f64(a, case.dtype)
    want, want_lse = tree_attention_fp8(f(case.q), k8, v8, ks, vs, case.block_table,
                                        case.prefix_len, f(case.k_tree), f(case.v_tree),
                                        case.cu_nodes, case.parent, case.hq, case.hkv, case.scale,
                                        nodes=nodes)
    got, got_lse = to_f64(out), lse.cpu().numpy().astype(np.float64)
    if nodes is not None:
        rows = rows_of(case, nodes)
        got, want, got_lse, want_lse = got[rows], want[rows], got_lse[rows], want_lse[rows]
    assert np.isfinite(got).all()
    e_out = np.abs(got - want).max() if got.size else 0.0
    e_lse = np.abs(got_lse - want_lse).max() if got.size else 0.0
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
    # 512 (sequence, KV head) pairs: 64 work items per die, run by the persistent launch
    "many_pairs": ([W.tree_heap(5)] * 64, [64 + 7 * b for b in range(64)], 32, 8),
}


@pytest.mark.parametrize("mode", ["codes", "quant"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_fp8_attention_small(gpu_lib, name, mode):
    parents, plens, hq, hkv = SMALL[name]
    case = W.make_case(name, parents, plens, hq, hkv, 128, W.DT_BF16, 10, 23, with_probs=False)
    check_fp8(gpu_lib, case, mode, seed=31)


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_fp8_attention_full_configs(gpu_lib, index):
    """The four bf16 workloads with quantized caches, in the benchmark's launch
    configuration: first, last and random nodes of every sequence."""
    case = W.make_config(index, with_probs=False)
    check_fp8(gpu_lib, case, "quant", seed=index,
              nodes=sample_nodes(case, 12 if case.batch <= 8 else 2, seed=index))


# Long work items of the pipelined kernel's FP8 register path: cut tail items merged
# by tickets (64 pairs x 10 row tiles), sequences without prefix or with a single
# node, prefixes that end inside a block; tree tiles staged through the same registers.
FP8_TAIL = ([W.tree_kary_levels(8, 3)] * 5 + [W.tree_random(np.random.default_rng(12), 300, 8),
             W.tree_chain(1), np.zeros(0, np.int32)], [300, 0, 4096, 64, 65, 1000, 130, 5], 32, 8)


@pytest.mark.parametrize("mode", ["codes", "quant"])
def test_fp8_attention_tail_pieces(gpu_lib, mode):
    parents, plens, hq, hkv = FP8_TAIL
    case = W.make_case("fp8tail", parents, plens, hq, hkv, 128, W.DT_BF16, 10, 27, with_probs=False)
    check_fp8(gpu_lib, case, mode, seed=8, nodes=sample_nodes(case, 8, seed=2))


def test_fp8_attention_repeatable(gpu_lib):
    """Persistent FP8 launches give the same bits call after call."""
    case = W.make_config(3, with_probs=False)
    k8, v8, ks, vs = fp8_inputs(case, "quant", 3)
    first, first_lse, _ = run_fp8(gpu_lib, case, k8, v8, ks, vs)
    again, again_lse, err = run_fp8(gpu_lib, case, k8, v8, ks, vs)
    assert err == 0 and torch.equal(first, again) and torch.equal(first_lse, again_lse)


def test_fp8_bad_block_sets_error(gpu_lib):
    case = W.make_case("badblk", [W.tree_heap(7)], [300], 4, 2, 128, W.DT_BF16, 10, 3,
                       with_probs=False)
    case.block_table[0, 2] = case.num_blocks  # outside the pool
    k8, v8, ks, vs = fp8_inputs(case, "codes", 4)
    _, _, err = run_fp8(gpu_lib, case, k8, v8, ks, vs)
    assert err & gpu_lib.TV_ERR_BLOCK
