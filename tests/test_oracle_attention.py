"""Pins for the tree-attention oracle.

Each test checks the oracle against something other than itself: a
hand-worked fixture, torch's own scaled-dot-product attention on cases where
tree attention reduces to it (a chain is causal attention; a single node is
decode attention), an explicit per-node loop over the node's own path, a
closed form (q = 0 gives the mean of the visible values) and invariants
(relabelling, paging, GQA expansion).  A few planted mistakes show the pins
catch a dropped term, a wrong head map and swapped operands.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as OA
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_oracle(case: W.Case, nodes=None, scale=None):
    f = lambda a: W.to_f64(a, case.dtype)
    return oracle.tree_attention(f(case.q), f(case.k_cache), f(case.v_cache), case.block_table,
                                 case.prefix_len, f(case.k_tree), f(case.v_tree), case.cu_nodes,
                                 case.parent, case.hq, case.hkv,
                                 case.scale if scale is None else scale, nodes=nodes)


def small_case(parents, plens, hq=4, hkv=2, d=16, dtype=W.DT_F32, seed=3, **kw):
    return W.make_case("t", parents, plens, hq, hkv, d, dtype, 50, seed, with_probs=False, **kw)


def prefix_rows(case, b, cache):
    c = W.to_f64(cache, case.dtype)
    t = np.arange(case.prefix_len[b])
    return c[case.block_table[b, t // 64], :, t % 64, :]


def parse(v):
    if isinstance(v, str):
        return math.log(float(v[2:]))
    return float(v)


def test_golden_hand_worked():
    with open(os.path.join(GOLDEN, "attention_tiny.json")) as f:
        g = json.load(f)
    arr = lambda x: np.array([[parse(v) for v in row] for row in x], dtype=np.float64)
    q = arr(g["q"])[:, None, :]
    kc = np.zeros((1, 1, 64, 2))
    vc = np.zeros((1, 1, 64, 2))
    kc[0, 0, 0] = arr(g["prefix_k"])[0]
    vc[0, 0, 0] = arr(g["prefix_v"])[0]
    kt = arr(g["tree_k"])[:, None, :]
    vt = arr(g["tree_v"])[:, None, :]
    out, lse = oracle.tree_attention(q, kc, vc, np.array([[0]]), np.array([1]), kt, vt,
                                     np.array([0, 3]), np.array(g["parent"]), 1, 1, 1.0)
    np.testing.assert_allclose(out[:, 0, :], np.array(g["out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, 0], [parse(v) for v in g["lse"]], rtol=0, atol=1e-12)


def sdpa_ref(q, k, v, mask, scale):
    """torch's SDPA on the CPU in fp64 (q [r,d], k/v [s,d], mask [r,s] bool)."""
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], attn_mask=torch.from_numpy(mask)[None, None], scale=scale)
    return o[0, 0].numpy()


@pytest.mark.parametrize("plen,n", [(0, 5), (70, 1), (130, 70), (64, 33)])
def test_chain_equals_causal_attention(plen, n):
    case = small_case([W.tree_chain(n)], [plen], hq=4, hkv=2, d=16)
    out, _ = run_oracle(case)
    for h in range(case.hq):
        g = OA.kv_head(h, case.hq, case.hkv)
        kp, vp = prefix_rows(case, 0, case.k_cache)[:, g], prefix_rows(case, 0, case.v_cache)[:, g]
        k = np.concatenate([kp, case.k_tree[:, g].astype(np.float64)])
        v = np.concatenate([vp, case.v_tree[:, g].astype(np.float64)])
        # query i sits at position plen + i and sees keys 0 .. plen + i
        mask = np.arange(plen + n)[None, :] <= (plen + np.arange(n))[:, None]
        ref = sdpa_ref(case.q[:, h].astype(np.float64), k, v, mask, case.scale)
        np.testing.assert_allclose(out[:, h], ref, rtol=0, atol=1e-12)


def test_single_node_is_decode_attention():
    case = small_case([np.array([-1], np.int32)], [200], hq=2, hkv=1, d=32)
    out, _ = run_oracle(case)
    kp, vp = prefix_rows(case, 0, case.k_cache)[:, 0], prefix_rows(case, 0, case.v_cache)[:, 0]
    k = np.concatenate([kp, case.k_tree[:, 0].astype(np.float64)])
    v = np.concatenate([vp, case.v_tree[:, 0].astype(np.float64)])
    for h in range(2):
        ref = sdpa_ref(case.q[:, h].astype(np.float64), k, v, np.ones((1, 201), bool), case.scale)
        np.testing.assert_allclose(out[:, h], ref, rtol=0, atol=1e-12)


def brute_force_node(case, b, n, h):
    """Attention of one node over prefix + its own root path, with explicit loops."""
    par = case.local_parent(b)
    path = []
    i = n
    while i >= 0:
        path.append(i)
        i = int(par[i])
    n0 = int(case.cu_nodes[b])
    g = h // (case.hq // case.hkv)
    kc, vc = W.to_f64(case.k_cache, case.dtype), W.to_f64(case.v_cache, case.dtype)
    kt, vt = W.to_f64(case.k_tree, case.dtype), W.to_f64(case.v_tree, case.dtype)
    qv = W.to_f64(case.q, case.dtype)[n0 + n, h]
    keys, vals = [], []
    for t in range(int(case.prefix_len[b])):
        blk = int(case.block_table[b, t // 64])
        keys.append(kc[blk, g, t % 64])
        vals.append(vc[blk, g, t % 64])
    for j in path:
        keys.append(kt[n0 + j, g])
        vals.append(vt[n0 + j, g])
    scores = [case.scale * sum(float(a) * float(c) for a, c in zip(qv, k)) for k in keys]
    mx = max(scores)
    ws = [math.exp(s - mx) for s in scores]
    tot = sum(ws)
    return np.array([sum(w * float(v[d]) for w, v in zip(ws, vals)) / tot for d in range(case.d)])


def test_every_node_equals_its_own_path_brute_force():
    rng = np.random.default_rng(9)
    parents = [W.tree_random(rng, 24, 5), W.tree_heap(7), W.tree_star(3)]
    case = small_case(parents, [40, 3, 0], hq=4, hkv=2, d=8, seed=12)
    out, _ = run_oracle(case)
    for b in range(case.batch):
        for n in range(int(case.cu_nodes[b + 1] - case.cu_nodes[b])):
            for h in range(case.hq):
                ref = brute_force_node(case, b, n, h)
                np.testing.assert_allclose(out[case.cu_nodes[b] + n, h], ref, rtol=0, atol=1e-12)


def test_bf16_brute_force_and_node_subset():
    case = small_case([W.tree_kary_levels(3, 3)], [100], hq=4, hkv=1, d=8, dtype=W.DT_BF16, seed=2)
    sel = [np.array([0, 5, 38])]
    out, _ = run_oracle(case, nodes=sel)
    for n in sel[0]:
        for h in range(4):
            np.testing.assert_allclose(out[n, h], brute_force_node(case, 0, int(n), h), atol=1e-12)
    mask = np.ones(case.total_nodes, bool)
    mask[sel[0]] = False
    assert np.isnan(out[mask]).all()


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(4)
    case = small_case([W.tree_random(rng, 30, 6)], [77], hq=2, hkv=2, d=8)
    case.q[:] = 0
    out, lse = run_oracle(case)
    par = case.parent
    vp = prefix_rows(case, 0, case.v_cache)
    for n in range(30):
        anc = oracle.ancestors_or_self(par, n)
        for h in range(2):
            rows = np.concatenate([vp[:, h], case.v_tree[anc, h].astype(np.float64)])
            np.testing.assert_allclose(out[n, h], rows.mean(axis=0), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[n, h], math.log(77 + len(anc)), atol=1e-12)


def test_relabelling_permutes_outputs():
    rng = np.random.default_rng(7)
    par = W.tree_random(rng, 40, 6)
    case = small_case([par], [65], hq=2, hkv=1, d=8)
    out, _ = run_oracle(case)
    # a random topological order: repeatedly pick any node whose parent is placed
    placed, order = set(), []
    remaining = list(range(40))
    while remaining:
        ready = [i for i in remaining if par[i] < 0 or par[i] in placed]
        pick = ready[int(rng.integers(0, len(ready)))]
        order.append(pick)
        placed.add(pick)
        remaining.remove(pick)
    new_of = {o: n for n, o in enumerate(order)}
    par2 = np.array([-1 if par[o] < 0 else new_of[int(par[o])] for o in order], np.int32)
    case2 = small_case([par2], [65], hq=2, hkv=1, d=8)
    case2.q[:] = case.q[order]
    case2.k_tree[:] = case.k_tree[order]
    case2.v_tree[:] = case.v_tree[order]
    case2.k_cache[:], case2.v_cache[:], case2.block_table[:] = case.k_cache, case.v_cache, case.block_table
    out2, _ = run_oracle(case2)
    np.testing.assert_allclose(out2, out[order], rtol=0, atol=1e-12)


def test_gqa_equals_expanded_mha():
    case = small_case([W.tree_heap(15)], [90], hq=6, hkv=2, d=8)
    out, _ = run_oracle(case)
    rep = lambda a, ax: np.repeat(a, 3, axis=ax)
    mha = W.Case(**{**case.__dict__, "hkv": 6, "k_cache": rep(case.k_cache, 1),
                    "v_cache": rep(case.v_cache, 1), "k_tree": rep(case.k_tree, 1),
                    "v_tree": rep(case.v_tree, 1)})
    out2, _ = run_oracle(mha)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-13)


def test_paging_and_aliasing_invariance():
    parents = [W.tree_heap(7), W.tree_heap(7)]
    a = small_case(parents, [150, 150], seed=5, alias_prefix=True, spare_blocks=3)
    out, _ = run_oracle(a)
    # both sequences read the same physical prefix; equal queries -> equal outputs
    b = small_case(parents, [150, 150], seed=5, alias_prefix=True, spare_blocks=3)
    b.q[7:] = b.q[:7]
    b.k_tree[7:] = b.k_tree[:7]
    b.v_tree[7:] = b.v_tree[:7]
    o2, _ = run_oracle(b)
    np.testing.assert_allclose(o2[7:], o2[:7], rtol=0, atol=0)
    # moving blocks around in the pool (and the table with them) changes nothing
    perm = np.random.default_rng(1).permutation(a.num_blocks)
    inv = np.argsort(perm)
    c = W.Case(**{**a.__dict__, "k_cache": a.k_cache[perm], "v_cache": a.v_cache[perm],
                  "block_table": np.where(a.block_table >= 0, inv[np.maximum(a.block_table, 0)], -1)})
    o3, _ = run_oracle(c)
    np.testing.assert_allclose(o3, out, rtol=0, atol=0)


def test_empty_sequence_and_empty_prefix():
    case = small_case([np.zeros(0, np.int32), W.tree_chain(3), W.tree_star(2)], [64, 0, 0])
    out, _ = run_oracle(case)
    assert out.shape == (5, 4, 16)
    # a node under the prefix with an empty prefix sees only itself: out = its own v
    for h in range(4):
        g = OA.kv_head(h, 4, 2)
        np.testing.assert_allclose(out[0, h], case.v_tree[0, g], atol=1e-15)
        np.testing.assert_allclose(out[3, h], case.v_tree[3, g], atol=1e-15)
        np.testing.assert_allclose(out[4, h], case.v_tree[4, g], atol=1e-15)


def test_paging_errors():
    bt = np.array([[0, 1], [2, -1]], np.int32)
    assert OA.check_paging(bt, np.array([128, 64]), 3) == 0
    assert OA.check_paging(bt, np.array([129, 64]), 3) & oracle.ERR_BLOCK
    assert OA.check_paging(bt, np.array([128, 65]), 3) & oracle.ERR_BLOCK
    assert OA.check_paging(bt, np.array([128, 64]), 2) & oracle.ERR_BLOCK


def test_bf16_tolerance_budget():
    """fp32 scores with probabilities rounded to bf16 before P.V, output rounded
    to bf16: the error against the fp64 definition sits well inside 2e-2."""
    case = small_case([W.tree_kary_levels(4, 3)], [1000], hq=4, hkv=1, d=128, dtype=W.DT_BF16, seed=8)
    out, _ = run_oracle(case)
    f32 = lambda a: W.bf16_bits_to_f32(a)
    kp = torch.from_numpy(prefix_rows(case, 0, case.k_cache)[:, 0].astype(np.float32))
    vp = torch.from_numpy(prefix_rows(case, 0, case.v_cache)[:, 0].astype(np.float32))
    kt, vt = torch.from_numpy(f32(case.k_tree)[:, 0]), torch.from_numpy(f32(case.v_tree)[:, 0])
    worst = 0.0
    for n in range(case.total_nodes):
        anc = oracle.ancestors_or_self(case.parent, n)
        k = torch.cat([kp, kt[anc]])
        v = torch.cat([vp, vt[anc]])
        for h in range(4):
            q = torch.from_numpy(f32(case.q)[n, h])
            s = (k @ q) * np.float32(case.scale)
            p = torch.exp(s - s.max())
            o = (p.to(torch.bfloat16).float() @ v) / p.sum()
            o = o.to(torch.bfloat16).double().numpy()
            worst = max(worst, float(np.abs(o - out[n, h]).max()))
    assert worst < 1e-2, worst


def test_planted_mistakes_are_caught(monkeypatch):
    # (1) the node itself dropped from its visible set -> the chain pin breaks
    case = small_case([W.tree_chain(6)], [10], hq=2, hkv=1, d=8)
    good, _ = run_oracle(case)
    monkeypatch.setattr(OA, "ancestors_or_self",
                        lambda par, n: oracle.ancestors_or_self(par, n)[1:] or [])
    with np.errstate(all="ignore"):
        bad, _ = run_oracle(case)
    assert not np.allclose(bad, good)
    monkeypatch.undo()
    # (2) head map h % hkv instead of h // G -> the GQA pin breaks
    case = small_case([W.tree_heap(7)], [30], hq=4, hkv=2, d=8)
    good, _ = run_oracle(case)
    monkeypatch.setattr(OA, "kv_head", lambda h, hq, hkv: h % hkv)
    bad, _ = run_oracle(case)
    assert not np.allclose(bad, good)
    monkeypatch.undo()
    # (3) keys and values swapped -> the hand-worked fixture breaks
    with open(os.path.join(GOLDEN, "attention_tiny.json")) as f:
        g = json.load(f)
    arr = lambda x: np.array([[parse(v) for v in row] for row in x], dtype=np.float64)
    kc = np.zeros((1, 1, 64, 2))
    vc = np.zeros((1, 1, 64, 2))
    kc[0, 0, 0], vc[0, 0, 0] = arr(g["prefix_k"])[0], arr(g["prefix_v"])[0]
    out, _ = oracle.tree_attention(arr(g["q"])[:, None], vc, kc, np.array([[0]]), np.array([1]),
                                   arr(g["tree_v"])[:, None], arr(g["tree_k"])[:, None],
                                   np.array([0, 3]), np.array(g["parent"]), 1, 1, 1.0)
    assert not np.allclose(out[:, 0], np.array(g["out"]), atol=1e-6)
