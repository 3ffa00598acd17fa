"""GPU parity of the probability rows (fp32) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._helpers import gpu_accept, oracle_accept

pytestmark = pytest.mark.gpu

REL = 5e-6  # fp32 exp (~1 ulp), fp32 sums of <= 32 terms per thread then a tree, one division


def logits_rows(rows, vocab, seed, sigma2=2.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, vocab)) * np.sqrt(sigma2)).astype(np.float32)


def context_rows(parents):
    """row_of for a tree: node i is judged at its parent's context; contexts are
    the prefix end (row 0) and every node that has a child (rows 1..)."""
    ctx = {-1: 0}
    for p in parents:
        if p >= 0 and p not in ctx:
            ctx[p] = len(ctx)
    return np.array([ctx[p] for p in parents], dtype=np.int32), len(ctx)


def check(got, want):
    got = got.astype(np.float64)
    assert np.all(np.abs(got - want) <= REL * want + 1e-30), np.max(np.abs(got - want) / np.maximum(want, 1e-300))


@pytest.mark.parametrize("rows,vocab,t", [(15, 1000, 1.0), (64, 32000, 1.0), (8, 152064, 0.7),
                                          (5, 50257, 1.3), (3, 7, 1.0)])
def test_softmax_rows_own_rows(gpu_lib, rows, vocab, t):
    lg = logits_rows(rows, vocab, seed=rows + vocab)
    got, err = gpu_lib.tree_softmax_rows(torch.from_numpy(lg).cuda(), inv_temperature=t)
    torch.cuda.synchronize()
    want, werr = oracle.softmax_rows(lg, inv_temperature=t)
    assert int(err.item()) == werr == 0
    check(got.cpu().numpy(), want)


def test_softmax_rows_shared_contexts(gpu_lib):
    parents = W.tree_kary_levels(8, 3)      # 584 nodes, 73 contexts
    row_of, ctx = context_rows(parents)
    vocab = 32000
    lg = logits_rows(ctx, vocab, seed=4)
    got, err = gpu_lib.tree_softmax_rows(torch.from_numpy(lg).cuda(),
                                         torch.from_numpy(row_of).cuda())
    torch.cuda.synchronize()
    want, werr = oracle.softmax_rows(lg, row_of=row_of)
    assert int(err.item()) == werr == 0
    check(got.cpu().numpy(), want)


def test_softmax_rows_bad_index_and_large_logits(gpu_lib):
    lg = np.zeros((3, 1000), np.float32)
    lg[1, :2] = [1000.0, 999.0]
    row_of = np.array([1, 3, 0, -2, 2], dtype=np.int32)
    got, err = gpu_lib.tree_softmax_rows(torch.from_numpy(lg).cuda(), torch.from_numpy(row_of).cuda())
    torch.cuda.synchronize()
    want, werr = oracle.softmax_rows(lg, row_of=row_of)
    assert werr == oracle.probs.ERR_ROW and int(err.item()) == werr
    g = got.cpu().numpy()
    assert np.all(g[1] == 0) and np.all(g[3] == 0)
    check(g[[0, 2, 4]], want[[0, 2, 4]])


def test_softmax_rows_feed_acceptance(gpu_lib):
    """Rows produced on the GPU drive the acceptance exactly as the oracle's
    acceptance run on the same rows."""
    case = W.make_config(0)
    row_of, ctx = context_rows(case.parent)
    lt = logits_rows(ctx, case.vocab, seed=11)
    ld = logits_rows(ctx, case.vocab, seed=12)
    pt, _ = gpu_lib.tree_softmax_rows(torch.from_numpy(lt).cuda(), torch.from_numpy(row_of).cuda())
    pd, _ = gpu_lib.tree_softmax_rows(torch.from_numpy(ld).cuda(), torch.from_numpy(row_of).cuda())
    torch.cuda.synchronize()
    case.p_target, case.p_draft = pt.cpu().numpy(), pd.cpu().numpy()
    dev = W.case_to_device(case)
    got = gpu_accept(gpu_lib, case, dev, 8)
    want = oracle_accept(case, 8)
    for k in ("accept_len", "path", "resample_node", "resample_token"):
        np.testing.assert_array_equal(np.asarray(got[k]), np.asarray(want[k]), err_msg=k)
