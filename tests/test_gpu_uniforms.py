"""GPU parity of the counter-based node uniforms (tree_uniforms) against the oracle's
Philox4x64-10 (page [P537] §8.2): bit-exact, on the trees of every workload, with
extreme key and counter words, empty sequences, one output omitted, and feeding
the acceptance step."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._helpers import assert_accept_equal

pytestmark = pytest.mark.gpu


def flat_trees(parents):
    cu = np.concatenate([[0], np.cumsum([len(p) for p in parents])]).astype(np.int32)
    parent = (np.concatenate(parents) if parents else np.zeros(0)).astype(np.int32)
    return parent, cu


def oracle_depths(parents):
    return (np.concatenate([oracle.depths(np.asarray(p, np.int32)) for p in parents])
            if parents else np.zeros(0, np.int32))


def gpu_uniforms(tv, parents, req, seed, purpose, step):
    parent, cu = flat_trees(parents)
    p_t, cu_t = torch.from_numpy(parent).cuda(), torch.from_numpy(cu).cuda()
    mn = max(1, int(np.diff(cu).max()) if len(cu) > 1 else 1)
    _, depth, _, err = tv.tree_build_index(p_t, cu_t, mn)
    ua, ur = tv.tree_uniforms(torch.from_numpy(np.asarray(req, np.int64)).cuda(), depth, cu_t,
                              seed=seed, step=step, purpose=purpose)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return ua.cpu().numpy(), ur.cpu().numpy()


KEYS = [(0, 0, 0), (2**64 - 1, 1, 2**63 + 5), (0x1234ABCD9876, 7, 99)]


@pytest.mark.parametrize("index", range(5))
@pytest.mark.parametrize("seed,purpose,step", KEYS)
def test_uniforms_bitexact_on_workload_trees(gpu_lib, index, seed, purpose, step):
    parents = W.config_trees(index, 1234)[0]
    rng = np.random.default_rng(100 + index)
    req = rng.integers(-2**63, 2**63 - 1, size=len(parents), dtype=np.int64)
    _, cu = flat_trees(parents)
    want = oracle.node_uniforms(seed, purpose, step, req, oracle_depths(parents), cu)
    got = gpu_uniforms(gpu_lib, parents, req, seed, purpose, step)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])


def test_uniforms_with_empty_sequences(gpu_lib):
    parents = [np.array([-1, 0, 0], np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32),
               np.array([-1, -1, 1, 2], np.int32), np.zeros(0, np.int32)]
    req = [5, 6, 7, 8, 9]
    _, cu = flat_trees(parents)
    want = oracle.node_uniforms(3, 0, 11, req, oracle_depths(parents), cu)
    got = gpu_uniforms(gpu_lib, parents, req, 3, 0, 11)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])


def test_uniforms_no_nodes(gpu_lib):
    ua, ur = gpu_lib.tree_uniforms(torch.zeros(2, dtype=torch.int64, device="cuda"),
                                   torch.zeros(0, dtype=torch.int32, device="cuda"),
                                   torch.zeros(3, dtype=torch.int32, device="cuda"), seed=1, step=2)
    assert ua.numel() == 0 and ur.numel() == 0


def test_uniforms_one_output_omitted(gpu_lib):
    tv = gpu_lib
    parents = W.config_trees(1, 1234)[0]
    parent, cu = flat_trees(parents)
    req = np.array([42], np.int64)
    want = oracle.node_uniforms(77, 2, 5, req, oracle_depths(parents), cu)
    depth = torch.from_numpy(oracle_depths(parents)).cuda()
    req_t, cu_t = torch.from_numpy(req).cuda(), torch.from_numpy(cu).cuda()
    total = len(parent)
    for which in (0, 1):
        out = torch.full((total,), -1.0, dtype=torch.float32, device="cuda")
        ptrs = [None, None]
        ptrs[which] = ctypes.c_void_p(out.data_ptr())
        st = tv.load().tree_uniforms(77, 2, 5, ctypes.c_void_p(req_t.data_ptr()),
                                     ctypes.c_void_p(depth.data_ptr()), ctypes.c_void_p(cu_t.data_ptr()),
                                     1, total, ptrs[0], ptrs[1],
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert st == tv.TV_OK
        np.testing.assert_array_equal(out.cpu().numpy(), want[which])


@pytest.mark.parametrize("index", [0, 1])
def test_uniforms_feed_acceptance(gpu_lib, index):
    """Generated uniforms drive tree_accept to the oracle's decisions made with the
    oracle's own uniforms."""
    tv = gpu_lib
    case = W.make_config(index, 1234)
    dev = W.case_to_device(case, "cuda:0")
    req = np.arange(case.batch, dtype=np.int64) + 1000
    depth_o = np.concatenate([oracle.depths(case.parent[case.cu_nodes[b]:case.cu_nodes[b + 1]])
                              for b in range(case.batch)])
    ua_o, ur_o = oracle.node_uniforms(2026, 0, 3, req, depth_o, case.cu_nodes)
    mn = max(1, case.max_nodes)
    _, depth, _, err = tv.tree_build_index(dev["parent"], dev["cu_nodes"], mn)
    ua, ur = tv.tree_uniforms(torch.from_numpy(req).cuda(), depth, dev["cu_nodes"], seed=2026, step=3)
    o = tv.tree_accept(dev["p_target"], dev["p_draft"], dev["token"], ua, ur, dev["parent"],
                       dev["cu_nodes"], mn, 16)
    torch.cuda.synchronize()
    got = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in o.items()}
    want = oracle.accept(case.p_target, case.p_draft, case.token, ua_o, ur_o, case.parent,
                         case.cu_nodes, case.vocab, 16)
    assert_accept_equal(got, want)
