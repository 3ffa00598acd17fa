"""GPU parity of the accepted-path KV commit against the oracle (bit-exact copy)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._helpers import gpu_accept, oracle_accept

pytestmark = pytest.mark.gpu


def run_commit(tv, case, dev, acc, path):
    """One commit on the GPU; returns (k_cache, v_cache, prefix_len, err) on the host."""
    acc_t = torch.from_numpy(np.ascontiguousarray(acc, dtype=np.int32)).cuda()
    path_t = torch.from_numpy(np.ascontiguousarray(path, dtype=np.int32)).cuda()
    err = tv.tree_commit_kv(dev["k_tree"], dev["v_tree"], dev["cu_nodes"], acc_t, path_t,
                            dev["k_cache"], dev["v_cache"], dev["block_table"], dev["prefix_len"])
    torch.cuda.synchronize()
    host = lambda t: (t.view(torch.int16).cpu().numpy().view(np.uint16) if t.dtype == torch.bfloat16
                      else t.cpu().numpy())
    return host(dev["k_cache"]), host(dev["v_cache"]), dev["prefix_len"].cpu().numpy(), int(err.item())


def assert_commit_equal(got, want):
    kc, vc, pl, err = got
    wk, wv, wpl, werr = want
    assert err == werr
    np.testing.assert_array_equal(pl, wpl)
    assert np.array_equal(kc, wk) and np.array_equal(vc, wv)


def chain_case(plens, lengths, hq, hkv, d, dtype, seed):
    parents = [np.asarray(list(range(-1, n - 1)) + [max(-1, n - 2)] * 3, dtype=np.int32)
               for n in lengths]
    return W.make_case("commit", parents, plens, hq, hkv, d, dtype, 10, seed, with_probs=False,
                       reserve_tokens=max(lengths) + 70)


CASES = {
    "fp32_d64_boundary": ([62, 64, 0], [5, 3, 4], 4, 2, 64, W.DT_F32),
    "bf16_d128_gqa": ([100, 7, 128, 1000], [6, 0, 1, 9], 32, 8, 128, W.DT_BF16),
    "bf16_d64_mha": ([63], [2], 4, 4, 64, W.DT_BF16),
    "fp32_d128_long_path": ([130], [20], 8, 2, 128, W.DT_F32),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_commit_chains(gpu_lib, name):
    plens, lengths, hq, hkv, d, dt = CASES[name]
    case = chain_case(plens, lengths, hq, hkv, d, dt, seed=5)
    max_path = max(lengths) + 2
    acc = np.asarray(lengths, dtype=np.int32)
    path = np.full((case.batch, max_path), -1, dtype=np.int32)
    for b, n in enumerate(lengths):
        path[b, :n] = np.arange(n)
    dev = W.case_to_device(case, probs=False)
    got = run_commit(gpu_lib, case, dev, acc, path)
    want = oracle.commit_kv(case.k_cache, case.v_cache, case.block_table, case.prefix_len,
                            case.num_blocks, case.k_tree, case.v_tree, case.cu_nodes, acc, path,
                            max_path)
    assert_commit_equal(got, want)
    # a second round on top of the first (prefix_len already advanced on both sides)
    case2 = W.Case(**{**case.__dict__})
    case2.k_cache, case2.v_cache, case2.prefix_len = want[0], want[1], want[2].astype(np.int32)
    acc2 = np.minimum(acc, 2).astype(np.int32)
    got2 = run_commit(gpu_lib, case2, dev, acc2, path)
    want2 = oracle.commit_kv(case2.k_cache, case2.v_cache, case2.block_table, case2.prefix_len,
                             case2.num_blocks, case2.k_tree, case2.v_tree, case2.cu_nodes, acc2, path,
                             max_path)
    assert_commit_equal(got2, want2)


@pytest.mark.parametrize("index", [0, 1, 3])
def test_commit_after_accept(gpu_lib, index):
    """accept -> commit on the GPU equals oracle accept -> oracle commit, on the verify
    workloads (with room reserved past each prefix)."""
    parents, plens, hq, hkv, d, dt, vocab, _ = W.config_trees(index, 1234)
    case = W.make_case(W.CONFIG_NAMES[index], parents, plens, hq, hkv, d, dt, vocab, 1234,
                       reserve_tokens=16)
    rng = np.random.default_rng(index)
    same = rng.random(case.total_nodes) < 0.8     # long accepted paths
    case.p_target[same] = case.p_draft[same]
    dev = W.case_to_device(case)
    max_path = 16
    acc_gpu = gpu_accept(gpu_lib, case, dev, max_path)
    acc_ref = oracle_accept(case, max_path)
    assert np.array_equal(acc_gpu["path"], acc_ref["path"])
    assert acc_ref["accept_len"].max() >= 2
    got = run_commit(gpu_lib, case, dev, acc_gpu["accept_len"], acc_gpu["path"])
    want = oracle.commit_kv(case.k_cache, case.v_cache, case.block_table, case.prefix_len,
                            case.num_blocks, case.k_tree, case.v_tree, case.cu_nodes,
                            acc_ref["accept_len"], acc_ref["path"], max_path)
    assert_commit_equal(got, want)


def test_commit_errors(gpu_lib):
    case = chain_case([10, 20, 30, 40], [3, 3, 3, 3], 4, 2, 64, W.DT_F32, seed=9)
    max_path = 4
    acc = np.array([3, 3, 5, 3], dtype=np.int32)   # sequence 2: longer than max_path
    path = np.tile(np.arange(max_path, dtype=np.int32), (case.batch, 1))
    path[3, 1] = 99                                # sequence 3: node outside its tree
    case.block_table = case.block_table.copy()
    case.block_table[1, 0] = case.num_blocks       # sequence 1: block outside the pool
    dev = W.case_to_device(case, probs=False)
    got = run_commit(gpu_lib, case, dev, acc, path)
    want = oracle.commit_kv(case.k_cache, case.v_cache, case.block_table, case.prefix_len,
                            case.num_blocks, case.k_tree, case.v_tree, case.cu_nodes, acc, path,
                            max_path)
    assert want[3] == oracle.ERR_BLOCK | oracle.ERR_PATH
    assert_commit_equal(got, want)


@pytest.mark.parametrize("plen, shared", [(100, 2), (128, 2)])
def test_commit_shared_prefix_blocks(gpu_lib, plen, shared):
    """Sequences 0 and 1 share their first blocks.  A 100-token shared prefix ends
    inside a shared block: neither sequence may append there (block bit, both left
    untouched, the private third one committed).  A 128-token one ends on a block
    boundary: every sequence appends into a private block."""
    case = chain_case([plen, plen, 40], [3, 3, 3], 8, 2, 128, W.DT_BF16, seed=13)
    case.block_table = case.block_table.copy()
    case.block_table[1, :shared] = case.block_table[0, :shared]
    max_path = 4
    acc = np.array([3, 3, 3], dtype=np.int32)
    path = np.tile(np.arange(max_path, dtype=np.int32), (case.batch, 1))
    dev = W.case_to_device(case, probs=False)
    got = run_commit(gpu_lib, case, dev, acc, path)
    want = oracle.commit_kv(case.k_cache, case.v_cache, case.block_table, case.prefix_len,
                            case.num_blocks, case.k_tree, case.v_tree, case.cu_nodes, acc, path,
                            max_path)
    assert want[3] == (oracle.ERR_BLOCK if plen % 64 else 0)
    assert_commit_equal(got, want)
