"""GPU parity of the probability rows (fp32) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._helpers import assert_accept_equal, gpu_accept, oracle_accept

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


# The one-pass kernel (a context row held on one compute unit) runs for at least
# 256 output rows with a vocabulary in [90112, 130560] (88 floats a thread in
# registers, the rest in LDS) or [114688, 155136] (112 a thread): its edges (no LDS
# part; the largest LDS part of each instance), both instances, groups of one and
# of two output rows, shared contexts and bad context indices.
@pytest.mark.parametrize("vocab,levels", [(90112, (4, 4)), (128256, (8, 3)), (130560, (4, 4)),
                                          (131072, (4, 4)), (152064, (8, 3)), (155136, (4, 4))])
def test_softmax_rows_one_pass(gpu_lib, vocab, levels):
    parents = W.tree_kary_levels(*levels)   # 340 nodes / 85 contexts, 584 / 73
    row_of, ctx = context_rows(parents)
    row_of[5] = -1
    row_of[-1] = ctx
    lg = logits_rows(ctx, vocab, seed=vocab + ctx)
    lg[1, 17] = np.float32(-np.inf)          # a masked entry keeps probability 0
    print(f"one-pass rows: vocab {vocab} rows {len(row_of)} contexts {ctx}", flush=True)
    got, err = gpu_lib.tree_softmax_rows(torch.from_numpy(lg).cuda(), torch.from_numpy(row_of).cuda(),
                                         inv_temperature=0.8)
    torch.cuda.synchronize()
    assert int(err.item()) == oracle.probs.ERR_ROW
    g = got.cpu().numpy()
    want, werr = oracle.softmax_rows(lg, inv_temperature=0.8)  # one row per context
    assert werr == 0
    ok = (row_of >= 0) & (row_of < ctx)
    assert np.all(g[~ok] == 0)
    check(g[ok], want[row_of[ok]])
    assert np.all(g[row_of == 1][:, 17] == 0)


def test_softmax_rows_one_pass_own_rows(gpu_lib):
    """The one-pass kernel without row_of (output row i from context row i), groups
    of one row, the smaller instance with an LDS part."""
    lg = logits_rows(300, 100000, seed=12)
    got, err = gpu_lib.tree_softmax_rows(torch.from_numpy(lg).cuda(), inv_temperature=1.2)
    torch.cuda.synchronize()
    want, werr = oracle.softmax_rows(lg, inv_temperature=1.2)
    assert int(err.item()) == werr == 0
    check(got.cpu().numpy(), want)


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


# ---- kept-set rows (the pruned draft distribution) --------------------------------

def kept_sets(rng, ctx_rows, vocab, keep_max, pad=True):
    """Per context row: a random number of distinct ids, some repeated, padded with -1."""
    keep = np.full((ctx_rows, keep_max), -1, np.int32)
    for r in range(ctx_rows):
        k = int(rng.integers(1, keep_max + 1)) if pad else keep_max
        ids = rng.choice(vocab, size=min(k, vocab), replace=False)
        if k > 2 and pad:
            ids[-1] = ids[0]            # a repeat counts once
        keep[r, :len(ids)] = rng.permutation(ids)
    return keep


@pytest.mark.parametrize("ctx_rows,vocab,keep_max,t", [(7, 1000, 16, 1.0), (5, 3001, 64, 0.8),
                                                       (3, 152064, 256, 1.0), (4, 32000, 1, 1.3),
                                                       (2, 7, 8, 1.0)])
def test_softmax_rows_kept_parity(gpu_lib, ctx_rows, vocab, keep_max, t):
    rng = np.random.default_rng(vocab + keep_max)
    lg = logits_rows(ctx_rows, vocab, seed=ctx_rows + vocab)
    keep = kept_sets(rng, ctx_rows, vocab, keep_max)
    row_of = rng.integers(0, ctx_rows, 2 * ctx_rows + 1).astype(np.int32)
    got, err = gpu_lib.tree_softmax_rows_kept(torch.from_numpy(lg).cuda(), torch.from_numpy(keep).cuda(),
                                              torch.from_numpy(row_of).cuda(), inv_temperature=t)
    torch.cuda.synchronize()
    want, werr = oracle.softmax_rows_kept(lg, keep, row_of=row_of, inv_temperature=t)
    assert int(err.item()) == werr == 0
    check(got.cpu().numpy(), want)
    own, err2 = gpu_lib.tree_softmax_rows_kept(torch.from_numpy(lg).cuda(), torch.from_numpy(keep).cuda(),
                                               inv_temperature=t)
    torch.cuda.synchronize()
    assert int(err2.item()) == 0
    check(own.cpu().numpy(), oracle.softmax_rows_kept(lg, keep, inv_temperature=t)[0])


def test_softmax_rows_kept_errors_leave_zero_rows(gpu_lib):
    lg = logits_rows(3, 1001, seed=9)
    keep = np.array([[5, 5, 900, -1], [-1, -1, -1, -1], [3, 1001, -1, -1]], np.int32)
    row_of = np.array([0, 1, 2, 3, -1, 0], np.int32)
    probs = torch.full((6, 1001), 7.0, device="cuda")        # every row must be overwritten
    got, err = gpu_lib.tree_softmax_rows_kept(torch.from_numpy(lg).cuda(), torch.from_numpy(keep).cuda(),
                                              torch.from_numpy(row_of).cuda(), probs=probs)
    torch.cuda.synchronize()
    want, werr = oracle.softmax_rows_kept(lg, keep, row_of=row_of)
    assert werr == oracle.ERR_ZERO_MASS | oracle.ERR_TOKEN | oracle.probs.ERR_ROW
    assert int(err.item()) == werr
    check(got.cpu().numpy(), want)
    assert not got[1:5].any()


def test_kept_draft_rows_feed_acceptance(gpu_lib):
    """Draft rows restricted to their kept sets are the p_draft of tree_accept: the
    acceptance outputs match the oracle's on the same rows, bit for bit."""
    rng = np.random.default_rng(11)
    parents = W.tree_kary_levels(4, 3)          # 84 nodes, 21 contexts
    row_of, ctx = context_rows(parents)
    vocab = 5000
    dl = logits_rows(ctx, vocab, seed=12)
    tl = logits_rows(ctx, vocab, seed=13)
    keep = kept_sets(rng, ctx, vocab, 32, pad=False)
    n = len(parents)
    token = np.array([keep[row_of[i], rng.integers(0, 32)] for i in range(n)], np.int32)
    pd, e1 = gpu_lib.tree_softmax_rows_kept(torch.from_numpy(dl).cuda(), torch.from_numpy(keep).cuda(),
                                            torch.from_numpy(row_of).cuda())
    pt, e2 = gpu_lib.tree_softmax_rows(torch.from_numpy(tl).cuda(), torch.from_numpy(row_of).cuda())
    torch.cuda.synchronize()
    assert int(e1.item()) == int(e2.item()) == 0
    case = W.make_case("kept", [parents], [100], 1, 1, 64, W.DT_F32, vocab, 14, with_probs=True)
    case.p_target = pt.cpu().numpy()
    case.p_draft = pd.cpu().numpy()
    case.token = token
    dev = W.case_to_device(case, probs=True)
    got = gpu_accept(gpu_lib, case, dev, max_path=8)
    assert_accept_equal(got, oracle_accept(case, max_path=8))


def test_kept_rows_agree_with_the_draft_tree(gpu_lib):
    """The draft tree builder judges a drafted token by its top-K probability over its
    context's kept mass (q_draft); the kept-set row of the same context's draft
    logits, with the kept slots' tokens as the set, gives the same number at that
    token (two routes to q~ of page [P525] §2.2.1)."""
    from oracle.draft_tree import kept_count
    rng = np.random.default_rng(21)
    n_max, vocab, k, ratio = 48, 4096, 8, 0.1
    ctx = n_max + 1
    lg = (rng.standard_normal((ctx, vocab)) * 3.0).astype(np.float32)   # peaked: truncation bites
    lg_t = torch.from_numpy(lg).cuda()
    full = torch.softmax(lg_t.double(), dim=1)
    p_top, tok_top = torch.topk(full, k, dim=1)                        # non-increasing slots
    probs = p_top.float().contiguous()[None]
    u = torch.from_numpy(W.grid_uniforms(rng, n_max).astype(np.float32)[None]).cuda()
    parent, slot, qd, count, err = gpu_lib.tree_draft_build(probs, u, 5, 0.7, ratio)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    n = int(count[0].item())
    assert n > 1
    p_np, tok_np = probs[0].cpu().numpy(), tok_top.cpu().numpy()
    keep = np.full((ctx, k), -1, np.int32)
    for r in range(ctx):
        m, _ = kept_count(p_np[r], ratio)
        keep[r, :m] = tok_np[r, :m]
    par, sl = parent[0, :n].cpu().numpy(), slot[0, :n].cpu().numpy()
    row_of = (par + 1).astype(np.int32)                                 # context after the parent
    pd, err2 = gpu_lib.tree_softmax_rows_kept(lg_t, torch.from_numpy(keep).cuda(),
                                              torch.from_numpy(row_of).cuda())
    torch.cuda.synchronize()
    assert int(err2.item()) == 0
    tokens = tok_np[row_of, sl]
    got = pd.cpu().numpy()[np.arange(n), tokens].astype(np.float64)
    want = qd[0, :n].cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=2e-5, atol=0)
