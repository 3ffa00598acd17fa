"""tree_accept_noalloc (the library's fixed per-GPU scratch, nothing allocated per
call) against tree_accept with a workspace of its own: bit-exact outputs and error
words on two calls in a row, the second with a smaller input, both on the chunked
launch that uses the scratch."""
import numpy as np
import pytest
import torch

import workloads as W
from _helpers import assert_accept_equal, gpu_accept

pytestmark = pytest.mark.gpu


def case_with_bonus(parents, vocab, seed):
    case = W.make_case("noalloc", parents, [0] * len(parents), 1, 1, 64, W.DT_F32, vocab, seed)
    rng = np.random.default_rng(seed)
    same = rng.random(case.total_nodes) < 0.7
    case.p_target[same] = case.p_draft[same]
    own_row = np.where(rng.random(case.total_nodes) < 0.8, np.arange(case.total_nodes), -1)
    return case, (W.prob_rows(seed, 5, case.total_nodes, vocab), own_row.astype(np.int32))


def noalloc(tv, case, dev, own, max_path):
    n = case.batch
    outputs = dict(accept_len=torch.full((n,), -7, dtype=torch.int32, device="cuda"),
                   path=torch.full((n, max_path), -7, dtype=torch.int32, device="cuda"),
                   resample_node=torch.full((n,), -7, dtype=torch.int32, device="cuda"),
                   resample_token=torch.full((n,), -7, dtype=torch.int32, device="cuda"),
                   node_ok=torch.full((case.total_nodes,), 7, dtype=torch.uint8, device="cuda"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    tv.tree_accept_noalloc(dev["p_target"], dev["p_draft"], dev["token"], dev["u_accept"],
                           dev["u_resample"], dev["parent"], dev["cu_nodes"],
                           max(1, case.max_nodes), max_path,
                           p_own=torch.from_numpy(own[0]).cuda(),
                           own_row=torch.from_numpy(own[1]).cuda(), outputs=outputs, err=err)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in outputs.items()}
    got["err"] = err.cpu().numpy()
    return got


def test_noalloc_matches_tree_accept_twice(gpu_lib):
    big = [W.tree_random(np.random.default_rng(70 + b), 20 + 7 * b, 6) for b in range(9)]
    small = [W.tree_chain(4), W.tree_random(np.random.default_rng(90), 11, 4)]
    for parents, vocab, seed in ((big, 152064, 3), (small, 70002, 4)):
        case, own = case_with_bonus(parents, vocab, seed)
        dev = W.case_to_device(case)
        want = gpu_accept(gpu_lib, case, dev, 8, own=own)
        got = noalloc(gpu_lib, case, dev, own, 8)
        assert_accept_equal(got, want)
        assert (want["resample_token"] >= 0).any()


def test_noalloc_refuses_more_than_its_scratch(gpu_lib):
    n = 1025
    case = W.make_case("wide", [W.tree_chain(1)] * n, [0] * n, 1, 1, 64, W.DT_F32, 65537, 5,
                       with_probs=False)
    z = torch.zeros((n, 65537), dtype=torch.float32, device="cuda")
    i32 = torch.zeros(n, dtype=torch.int32, device="cuda")
    u = torch.zeros(n, dtype=torch.float32, device="cuda")
    cu = torch.from_numpy(case.cu_nodes).cuda()
    outputs = dict(accept_len=i32.clone(), path=torch.zeros((n, 1), dtype=torch.int32, device="cuda"),
                   resample_node=i32.clone(), resample_token=i32.clone(), node_ok=None)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(gpu_lib.TreeVerifyError, match="scratch"):
        gpu_lib.tree_accept_noalloc(z, z, i32, u, u, i32, cu, 1, 1, outputs=outputs, err=err)
