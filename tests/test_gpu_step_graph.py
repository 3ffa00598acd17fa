"""The step as one call (tree_verify_step) and as a replayed HIP graph
(tree_verify_graph_*, page [ViSpec] §3.2): bit-identical to the three separate
calls, on every replay, with eager work and synchronisations between replays, and
after inputs are refreshed in place."""
import numpy as np
import pytest
import torch

import workloads as W
from tests._helpers import gpu_accept, gpu_attention, gpu_index

pytestmark = pytest.mark.gpu

MAX_PATH = 16


def make_step(tv, case, dev):
    return tv.VerifyStep(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                         dev["prefix_len"], dev["k_tree"], dev["v_tree"], dev["parent"],
                         dev["cu_nodes"], dev["p_target"], dev["p_draft"], dev["token"],
                         dev["u_accept"], dev["u_resample"], max_nodes=max(1, case.max_nodes),
                         max_prefix=case.max_prefix, max_path=MAX_PATH, want_lse=True)


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    elif t.dtype == torch.float32:
        t = t.view(torch.int32)
    return t.cpu().numpy().copy()


def snapshot(step) -> dict:
    torch.cuda.synchronize()
    s = dict(anc=bits(step.anc), depth=bits(step.depth), out=bits(step.out), lse=bits(step.lse),
             err=bits(step.err))
    for k, v in step.accept.items():
        if k != "err":
            s[k] = bits(v)
    return s


def assert_same(got: dict, want: dict):
    assert got.keys() == want.keys()
    for k in want:
        np.testing.assert_array_equal(got[k], want[k], err_msg=k)


@pytest.mark.parametrize("index", [0, 1, 3])
def test_step_equals_the_three_calls(gpu_lib, index):
    tv = gpu_lib
    case = W.make_config(index, 1234)
    dev = W.case_to_device(case, "cuda:0")
    anc, depth, _, err_i = gpu_index(tv, case, dev)
    out, lse, err_a = gpu_attention(tv, case, dev, anc)
    acc = gpu_accept(tv, case, dev, MAX_PATH)
    step = make_step(tv, case, dev)
    step.run()
    got = snapshot(step)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got["anc"], bits(anc)[:, :got["anc"].shape[1]])
    np.testing.assert_array_equal(got["depth"], bits(depth))
    np.testing.assert_array_equal(got["out"], bits(out))
    np.testing.assert_array_equal(got["lse"], bits(lse))
    for k in ("accept_len", "path", "resample_node", "resample_token", "node_ok"):
        np.testing.assert_array_equal(got[k].astype(np.int64), np.asarray(acc[k]).astype(np.int64),
                                      err_msg=k)
    assert int(got["err"][0]) == 0 and int(err_i.item()) == 0 and int(err_a.item()) == 0


@pytest.mark.parametrize("index", [1, 3])
def test_graph_replays_equal_the_eager_step(gpu_lib, index):
    tv = gpu_lib
    case = W.make_config(index, 1234)
    dev = W.case_to_device(case, "cuda:0")
    step = make_step(tv, case, dev)
    step.run()
    want = snapshot(step)
    graph = step.capture()
    try:
        for rep in range(4):
            # the program's own eager work between replays: poison the outputs,
            # unrelated kernels, a synchronisation
            step.out.fill_(float("nan"))
            step.lse.fill_(-1.0)
            step.anc.zero_()
            step.depth.fill_(-5)
            for k in ("accept_len", "path", "resample_node", "resample_token"):
                step.accept[k].fill_(-9)
            step.accept["node_ok"].fill_(7)
            x = torch.randn(1 << 20, device="cuda")
            _ = (x * 2.0 + 1.0).sum().item()
            torch.cuda.synchronize()
            graph.launch()
            assert_same(snapshot(step), want)
        # inputs refreshed in place: the replay reads the new values
        gen = torch.Generator(device="cpu").manual_seed(99 + index)
        new_u = torch.rand(dev["u_accept"].shape, generator=gen).to(dev["u_accept"].device)
        dev["u_accept"].copy_(new_u)
        dev["u_resample"].copy_(torch.rand(dev["u_resample"].shape, generator=gen).cuda())
        torch.cuda.synchronize()
        graph.launch()
        got = snapshot(step)
        step.run()
        assert_same(got, snapshot(step))
        assert int(got["err"][0]) == 0
    finally:
        graph.close()
