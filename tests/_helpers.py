"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as W


def max_nodes_of(case: W.Case) -> int:
    return max(1, case.max_nodes)


def gpu_index(tv, case: W.Case, dev, max_nodes=None):
    mn = max_nodes or max_nodes_of(case)
    anc, depth, pos, err = tv.tree_build_index(dev["parent"], dev["cu_nodes"], mn, dev["prefix_len"])
    return anc, depth, pos, err


def gpu_attention(tv, case: W.Case, dev, anc, max_nodes=None):
    mn = max_nodes or max_nodes_of(case)
    out, lse, err = tv.tree_verify_attention(
        dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"], dev["prefix_len"],
        dev["k_tree"], dev["v_tree"], dev["cu_nodes"], anc, mn, case.max_prefix)
    return out, lse, err


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_attention(case: W.Case, nodes=None):
    f = lambda a: W.to_f64(a, case.dtype)
    return oracle.tree_attention(f(case.q), f(case.k_cache), f(case.v_cache), case.block_table,
                                 case.prefix_len, f(case.k_tree), f(case.v_tree), case.cu_nodes,
                                 case.parent, case.hq, case.hkv, case.scale, nodes=nodes)


def sample_nodes(case: W.Case, per_seq: int, seed: int = 0, seqs=None):
    """A few local nodes per sequence: the first, the last, and random ones."""
    rng = np.random.default_rng(seed)
    sel = []
    for b in range(case.batch):
        n = int(case.cu_nodes[b + 1] - case.cu_nodes[b])
        if n == 0 or (seqs is not None and b not in seqs):
            sel.append(np.zeros(0, np.int64))
            continue
        pick = {0, n - 1} | set(int(x) for x in rng.integers(0, n, size=per_seq))
        sel.append(np.array(sorted(pick), np.int64))
    return sel


def rows_of(case: W.Case, nodes):
    return np.concatenate([case.cu_nodes[b] + np.asarray(nodes[b], np.int64)
                           for b in range(case.batch)]).astype(np.int64)


def gpu_accept(tv, case: W.Case, dev, max_path: int, max_nodes=None, own=None, workspace=None):
    """tree_accept on the device; own = (p_own, own_row) numpy arrays for bonus tokens."""
    mn = max_nodes or max_nodes_of(case)
    kw = {}
    if own is not None:
        kw = dict(p_own=torch.from_numpy(np.ascontiguousarray(own[0])).cuda(),
                  own_row=torch.from_numpy(np.ascontiguousarray(own[1], dtype=np.int32)).cuda())
    o = tv.tree_accept(dev["p_target"], dev["p_draft"], dev["token"], dev["u_accept"],
                       dev["u_resample"], dev["parent"], dev["cu_nodes"], mn, max_path,
                       workspace=workspace, **kw)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in o.items()}


def oracle_accept(case: W.Case, max_path: int, own=None):
    p_own, own_row = own if own is not None else (None, None)
    return oracle.accept(case.p_target, case.p_draft, case.token, case.u_accept, case.u_resample,
                         case.parent, case.cu_nodes, case.vocab, max_path, p_own, own_row)


def assert_accept_equal(got: dict, want: dict):
    for k in ("accept_len", "path", "resample_node", "resample_token", "node_ok"):
        np.testing.assert_array_equal(np.asarray(got[k]).astype(np.int64),
                                      np.asarray(want[k]).astype(np.int64), err_msg=k)
    got_err = int(np.asarray(got["err"]).reshape(-1)[0])
    want_err = int(np.asarray(want["err"]).reshape(-1)[0])
    assert got_err == want_err, (got_err, want_err)
