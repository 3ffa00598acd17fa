"""GPU parity of draft-tree construction (tree_draft_build through the C ABI)
against the oracle.

Integer outputs (parent, slot, count, error word) and q_draft must match bit for
bit.  The one legitimate difference: the device sums a draw's weights in
wavefront chunks while the oracle sums them left to right, so a draw whose
threshold u * total lies within rounding (relative 1e-12) of a running-sum
boundary may resolve to either neighbour; such a sequence is compared up to that
draw and the oracle's margin there is checked.  The built trees then go through
tree_build_index, bit-exact against the oracle's index.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.draft_tree import build_tree

pytestmark = pytest.mark.gpu

AMBIGUOUS = 1e-12

CASES = {
    # name: (batch, rows, k, n_max, max_depth, beta, prune_ratio)
    "llava_like": (1, 65, 8, 64, 6, 0.7, 0.1),
    "batch_no_truncation": (8, 65, 8, 64, 6, 0.7, 0.0),
    "long_chains": (2, 257, 4, 256, 10, 0.5, 0.05),
    "wide_shallow": (3, 129, 16, 128, 3, 1.0, 0.3),
    "uniform_weights": (4, 33, 6, 32, 4, 0.0, 0.2),
    "one_candidate": (2, 40, 1, 40, 40, 0.7, 0.1),
    "few_rows": (2, 10, 8, 64, 6, 0.7, 0.1),
    # every limit at once: 256 draws, 16 slots a row, no truncation, no depth cap
    # (up to 16 * 257 candidates, all 33 chunks of the candidate store in use)
    "max_size": (2, 257, 16, 256, 256, 0.7, 0.0),
}


def inputs(name, seed=3):
    batch, rows, k, n_max, depth, beta, ratio = CASES[name]
    rng = np.random.default_rng(seed)
    probs = W.draft_rows(rng, batch, rows, k, vocab=4096)
    u = np.stack([W.grid_uniforms(rng, n_max) for _ in range(batch)]).astype(np.float32)
    return probs, u, n_max, depth, beta, ratio


def run_gpu(tv, probs, u, depth, beta, ratio):
    p = torch.from_numpy(probs).cuda()
    uu = torch.from_numpy(u).cuda()
    parent, slot, qd, count, err = tv.tree_draft_build(p, uu, depth, beta, ratio)
    torch.cuda.synchronize()
    return (parent.cpu().numpy(), slot.cpu().numpy(), qd.cpu().numpy(), count.cpu().numpy(),
            int(err.item()))


@pytest.mark.parametrize("name", sorted(CASES))
def test_draft_tree_matches_oracle(gpu_lib, name):
    probs, u, n_max, depth, beta, ratio = inputs(name)
    print(f"draft case {name} shape {probs.shape} n_max {n_max}", flush=True)
    g_par, g_slot, g_q, g_cnt, g_err = run_gpu(gpu_lib, probs, u, depth, beta, ratio)
    assert g_err == 0
    exact = 0
    for b in range(probs.shape[0]):
        par, sl, _, q, margins = build_tree(probs[b], u[b], n_max, depth, beta, ratio)
        n = len(par)
        same = (g_cnt[b] == n and np.array_equal(g_par[b, :n], par) and
                np.array_equal(g_slot[b, :n], sl) and np.array_equal(g_q[b, :n], q))
        if same:
            exact += 1
            assert np.all(g_par[b, n:] == -2) and np.all(g_slot[b, n:] == -2)
            assert np.all(g_q[b, n:] == 0)
            continue
        m = min(n, int(g_cnt[b]))
        d = np.flatnonzero((g_par[b, :m] != par[:m]) | (g_slot[b, :m] != sl[:m]))
        assert d.size, f"sequence {b}: same nodes, different count or q_draft"
        i = int(d[0])
        assert np.array_equal(g_q[b, :i], q[:i])
        assert margins[i] < AMBIGUOUS, (b, i, margins[i])
    assert exact >= 1


def test_built_trees_feed_the_index(gpu_lib):
    probs, u, n_max, depth, beta, ratio = inputs("batch_no_truncation", seed=5)
    g_par, _, _, g_cnt, _ = run_gpu(gpu_lib, probs, u, depth, beta, ratio)
    cu = np.concatenate([[0], np.cumsum(g_cnt)]).astype(np.int32)
    flat = np.concatenate([g_par[b, :g_cnt[b]] for b in range(len(g_cnt))]).astype(np.int32)
    mn = int(g_cnt.max())
    anc, dep, _, err = gpu_lib.tree_build_index(torch.from_numpy(flat).cuda(),
                                                torch.from_numpy(cu).cuda(), mn)
    torch.cuda.synchronize()
    want_anc, want_dep, _, want_err = oracle.build_index(flat, cu, mn)
    assert int(err.item()) == want_err == 0
    np.testing.assert_array_equal(anc.cpu().numpy().view(np.uint64), want_anc)
    np.testing.assert_array_equal(dep.cpu().numpy(), want_dep)


def test_draft_tree_errors(gpu_lib):
    probs, u, n_max, depth, beta, ratio = inputs("uniform_weights", seed=6)
    probs[1, 3, 2] = np.float32(np.nan)
    u[2, 5] = 1.0
    g_par, _, g_q, g_cnt, g_err = run_gpu(gpu_lib, probs, u, depth, beta, ratio)
    _, _, _, _, want_cnt, want_err = oracle.build_trees(probs, u, n_max, depth, beta, ratio)
    assert g_err == want_err == (gpu_lib.TV_ERR_DRAFT | gpu_lib.TV_ERR_UNIFORM)
    assert list(g_cnt[1:3]) == [0, 0] == list(want_cnt[1:3])
    assert np.all(g_par[1:3] == -2) and np.all(g_q[1:3] == 0)
