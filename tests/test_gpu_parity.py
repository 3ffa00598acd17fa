"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer outputs (bitsets, depths, positions, accepted paths, resampled tokens,
error words) must match bit for bit.  Attention outputs must be within
max-abs 1e-5 (fp32 inputs) or 2e-2 (bf16 inputs, bf16 output) of the fp64
oracle evaluated on the same input bits.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _helpers import (assert_accept_equal, gpu_accept, gpu_attention, gpu_index, oracle_accept,
                      oracle_attention, rows_of, sample_nodes, to_f64)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def check_index(tv, case, max_nodes=None):
    dev = W.case_to_device(case, probs=False)
    mn = max_nodes or max(1, case.max_nodes)
    anc, depth, pos, err = gpu_index(tv, case, dev, mn)
    torch.cuda.synchronize()
    want_anc, want_depth, want_pos, want_err = oracle.build_index(case.parent, case.cu_nodes, mn,
                                                                  case.prefix_len)
    assert int(err.item()) == want_err
    np.testing.assert_array_equal(anc.cpu().numpy().view(np.uint64), want_anc)
    np.testing.assert_array_equal(depth.cpu().numpy(), want_depth)
    np.testing.assert_array_equal(pos.cpu().numpy(), want_pos)
    return dev, anc


TREE_CASES = {
    "heap15": ([W.tree_heap(15)], [128]),
    "kary584": ([W.tree_kary_levels(8, 3)] * 2, [10, 70]),
    "long256": ([W.tree_branch_then_chains(4, 3, 10, 256)], [0]),
    "random_batch": ([W.tree_random(np.random.default_rng(s), n, 8) for s, n in
                      [(1, 16), (2, 96), (3, 50), (4, 1)]], [512, 700, 4096, 3]),
    "empty_seq": ([np.zeros(0, np.int32), W.tree_star(5), np.zeros(0, np.int32)], [64, 0, 9]),
    "chain2048": ([W.tree_chain(2048)], [0]),
    "star2048": ([W.tree_star(2048)], [100]),
}


@pytest.mark.parametrize("name", sorted(TREE_CASES))
def test_build_index_bitexact(gpu_lib, name):
    parents, plens = TREE_CASES[name]
    case = W.make_case(name, parents, plens, 1, 1, 64, W.DT_F32, 10, 1, with_probs=False)
    check_index(gpu_lib, case)


def test_build_index_error_bits(gpu_lib):
    bad = np.array([-1, 0, 3, 1], np.int32)   # node 2 points forward
    case = W.make_case("bad", [bad, W.tree_heap(7)], [5, 5], 1, 1, 64, W.DT_F32, 10, 1,
                       with_probs=False)
    dev = W.case_to_device(case, probs=False)
    _, _, _, err = gpu_index(gpu_lib, case, dev)
    assert int(err.item()) == oracle.ERR_BAD_PARENT
    # a sequence longer than max_nodes
    case = W.make_case("big", [W.tree_chain(70)], [5], 1, 1, 64, W.DT_F32, 10, 1, with_probs=False)
    dev = W.case_to_device(case, probs=False)
    _, _, _, err = gpu_index(gpu_lib, case, dev, max_nodes=64)
    assert int(err.item()) == oracle.ERR_TOO_MANY_NODES


@pytest.mark.parametrize("mn", [64, 300])
def test_build_index_errors_leave_other_sequences(gpu_lib, mn):
    """A sequence with a bad link or too many nodes (here also past the nodes the
    launch covers for max_nodes = 300) flags its bit; the other sequences' rows are
    still exact."""
    rng = np.random.default_rng(mn)
    good = [W.tree_random(rng, 40, 5), W.tree_heap(mn), W.tree_chain(mn)]
    bad = np.array([-1, 0, 3, 1], np.int32)
    parents = [good[0], W.tree_chain(2 * mn + 7), good[1], bad, good[2]]
    case = W.make_case("mixed_err", parents, [5, 6, 7, 8, 9], 1, 1, 64, W.DT_F32, 10, 1,
                       with_probs=False)
    dev = W.case_to_device(case, probs=False)
    anc, depth, pos, err = gpu_index(gpu_lib, case, dev, max_nodes=mn)
    torch.cuda.synchronize()
    assert int(err.item()) == oracle.ERR_TOO_MANY_NODES | oracle.ERR_BAD_PARENT
    anc = anc.cpu().numpy().view(np.uint64)
    depth, pos = depth.cpu().numpy(), pos.cpu().numpy()
    cu = case.cu_nodes
    for b in (0, 2, 4):
        n0, n1 = int(cu[b]), int(cu[b + 1])
        want_anc, want_depth, want_pos, want_err = oracle.build_index(
            case.parent[n0:n1], np.array([0, n1 - n0]), mn, case.prefix_len[b:b + 1])
        assert want_err == 0
        np.testing.assert_array_equal(anc[n0:n1], want_anc)
        np.testing.assert_array_equal(depth[n0:n1], want_depth)
        np.testing.assert_array_equal(pos[n0:n1], want_pos)


# ------------------------------------------------------------------ attention

def check_attention(tv, case, tol, nodes=None):
    dev, anc = check_index(tv, case)
    out, lse, err = gpu_attention(tv, case, dev, anc)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    want, want_lse = oracle_attention(case, nodes)
    got = to_f64(out)
    got_lse = lse.cpu().numpy().astype(np.float64)
    if nodes is not None:
        rows = rows_of(case, nodes)
        got, want, got_lse, want_lse = got[rows], want[rows], got_lse[rows], want_lse[rows]
    assert np.isfinite(got).all()
    err_out = np.abs(got - want).max() if got.size else 0.0
    err_lse = np.abs(got_lse - want_lse).max() if got.size else 0.0
    assert err_out <= tol, err_out
    assert err_lse <= tol, err_lse
    return out


def test_attention_tiny_fp32_config(gpu_lib):
    check_attention(gpu_lib, W.make_config(0, with_probs=False), TOL_F32)


SMALL = {
    # name: (parents, prefix_lens, hq, hkv, d, dtype)
    "ragged_bf16_gqa": ([W.tree_chain(1), W.tree_random(np.random.default_rng(5), 37, 6),
                         W.tree_random(np.random.default_rng(6), 130, 8)], [0, 70, 200], 8, 2, 128,
                        W.DT_BF16),
    "wide_rows_bf16": ([W.tree_kary_levels(5, 3)], [333], 16, 4, 128, W.DT_BF16),
    "split_prefix_mha": ([W.tree_heap(31)], [1000], 4, 4, 128, W.DT_BF16),
    "prefix_multiple_of_64": ([W.tree_heap(7), W.tree_heap(7)], [128, 64], 8, 1, 128, W.DT_BF16),
    "star_no_prefix": ([W.tree_star(100)], [0], 4, 2, 128, W.DT_BF16),
    "chain_deep": ([W.tree_chain(300)], [65], 2, 1, 128, W.DT_BF16),
    "fp32_d128": ([W.tree_random(np.random.default_rng(7), 70, 6)], [150], 4, 2, 128, W.DT_F32),
    "bf16_d64": ([W.tree_random(np.random.default_rng(8), 70, 6)], [150], 4, 2, 64, W.DT_BF16),
    "fp32_d64_batch": ([W.tree_heap(15), W.tree_star(3), np.zeros(0, np.int32)], [1, 64, 5], 6, 3,
                       64, W.DT_F32),
    # long work items (64-rows-per-wavefront kernel): many prefix blocks per split,
    # a last row tile holding a single 32-row group, sequences with no prefix tile in
    # most splits
    "long_split_gqa": ([W.tree_random(np.random.default_rng(9), 200, 8)], [8000], 8, 2, 128,
                       W.DT_BF16),
    "long_ragged_mha": ([W.tree_random(np.random.default_rng(10), 130, 5), W.tree_chain(5),
                         W.tree_random(np.random.default_rng(11), 600, 12)], [1000, 37, 513], 4, 4,
                        128, W.DT_BF16),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_attention_small(gpu_lib, name):
    parents, plens, hq, hkv, d, dt = SMALL[name]
    case = W.make_case(name, parents, plens, hq, hkv, d, dt, 10, 17, with_probs=False)
    check_attention(gpu_lib, case, TOL_F32 if dt == W.DT_F32 else TOL_BF16)


TAIL_CASES = {
    # 64 (sequence, KV head) pairs x 10 row tiles: 16 items per die are cut in 2
    # prefix pieces; sequences with no prefix, a single node, no nodes
    "pieces2": ([W.tree_kary_levels(8, 3)] * 5 + [W.tree_random(np.random.default_rng(12), 300, 8),
                 W.tree_chain(1), np.zeros(0, np.int32)], [300, 0, 4096, 64, 65, 1000, 130, 5],
                32, 8),
    # 8 pairs x 33 row tiles: one item per die, cut in 7 pieces, most of them with no
    # prefix tile (2 blocks); the last piece holds only tree tiles
    "pieces7_short": ([W.tree_random(np.random.default_rng(13), 1025, 12)], [100], 64, 8),
    "pieces7_long": ([W.tree_random(np.random.default_rng(14), 1025, 12)], [2000], 64, 8),
    # 2056 pairs (more than the ordering kernel ranks) x 1 row tile: the last item of
    # each die (sequence 256) cut in 7 pieces, its tickets cleared by a kernel of their own
    "pieces7_unordered": ([W.tree_heap(63)] * 257, [200 + 3 * (b % 50) for b in range(257)], 32,
                          8),
}
TAIL_SEQS = {"pieces7_unordered": {0, 100, 255, 256}}


@pytest.mark.parametrize("name", sorted(TAIL_CASES))
def test_attention_tail_pieces(gpu_lib, name):
    """Work items of the last round cut into prefix pieces and merged by the piece that
    finishes last; a second call (tickets cleared again) gives the same bits."""
    parents, plens, hq, hkv = TAIL_CASES[name]
    case = W.make_case(name, parents, plens, hq, hkv, 128, W.DT_BF16, 10, 21, with_probs=False)
    nodes = sample_nodes(case, 10, seed=5, seqs=TAIL_SEQS.get(name))
    out = check_attention(gpu_lib, case, TOL_BF16, nodes=nodes)
    dev = W.case_to_device(case, probs=False)
    anc, _, _, _ = gpu_index(gpu_lib, case, dev)
    again, _, _ = gpu_attention(gpu_lib, case, dev, anc)
    torch.cuda.synchronize()
    assert torch.equal(out, again)


COUNTER_CASES = {
    # 16 prefix splits merged by the split-merge kernel
    "splits16": ([W.tree_random(np.random.default_rng(9), 200, 8)], [8000], 8, 2),
    # persistent launch with tail pieces (queue heads, exit count, tickets)
    "persistent_tail": TAIL_CASES["pieces2"][:4],
    # persistent launch, every die's last round full (queue heads only)
    "persistent": ([W.tree_random(np.random.default_rng(30 + b), 90, 8) for b in range(64)],
                   [512 + 57 * b for b in range(64)], 32, 8),
}


@pytest.mark.parametrize("name", sorted(COUNTER_CASES))
def test_attention_workspace_counters_left_zero(gpu_lib, name):
    """The workspace's counter words are zero after every call, so one zero-filled
    workspace serves any number of calls; the outputs of repeated calls are identical."""
    parents, plens, hq, hkv = COUNTER_CASES[name]
    case = W.make_case(name, parents, plens, hq, hkv, 128, W.DT_BF16, 10, 23, with_probs=False)
    dev = W.case_to_device(case, probs=False)
    mn = max(1, case.max_nodes)
    anc, _, _, _ = gpu_index(gpu_lib, case, dev)
    need = gpu_lib.tree_verify_attention_workspace_size(case.batch, case.total_nodes, mn,
                                                        case.max_prefix, hq, hkv, 128,
                                                        gpu_lib.TV_DTYPE_BF16)
    assert need > 2048
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        out, lse, err = gpu_lib.tree_verify_attention(
            dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"], dev["prefix_len"],
            dev["k_tree"], dev["v_tree"], dev["cu_nodes"], anc, mn, case.max_prefix, workspace=ws)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert int(ws[:2048].count_nonzero().item()) == 0
        outs.append((out.clone(), lse.clone()))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    nodes = sample_nodes(case, 6, seed=3)
    want, want_lse = oracle_attention(case, nodes)
    rows = rows_of(case, nodes)
    assert np.abs(to_f64(outs[0][0])[rows] - want[rows]).max() <= TOL_BF16


def test_attention_workspace_shared_across_plans(gpu_lib):
    """One zero-filled workspace serves calls of different launch plans in turn
    (persistent with cut items, prefix splits, persistent, one plain round): each
    output equals the output with a workspace of its own, bit for bit."""
    names = ["persistent_tail", "splits16", "persistent", "one_round"]
    # one_round: 32 pairs x 8 row tiles = 32 items per die, no split: a plain launch
    specs = dict(COUNTER_CASES,
                 one_round=([W.tree_random(np.random.default_rng(50), 512, 8)] * 4,
                            [300, 200, 100, 64], 32, 8))
    runs = []
    for name in names:
        parents, plens, hq, hkv = specs[name]
        case = W.make_case(name, parents, plens, hq, hkv, 128, W.DT_BF16, 10, 29, with_probs=False)
        dev = W.case_to_device(case, probs=False)
        anc, _, _, _ = gpu_index(gpu_lib, case, dev)
        runs.append((case, dev, anc))
    sizes = [gpu_lib.tree_verify_attention_workspace_size(c.batch, c.total_nodes, max(1, c.max_nodes),
                                                          c.max_prefix, c.hq, c.hkv, 128,
                                                          gpu_lib.TV_DTYPE_BF16) for c, _, _ in runs]
    shared = torch.zeros(max(sizes), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        for (case, dev, anc), need in zip(runs, sizes):
            args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"], dev["prefix_len"],
                    dev["k_tree"], dev["v_tree"], dev["cu_nodes"], anc, max(1, case.max_nodes),
                    case.max_prefix)
            out, lse, err = gpu_lib.tree_verify_attention(*args, workspace=shared)
            own, own_lse, _ = gpu_lib.tree_verify_attention(
                *args, workspace=torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda"))
            torch.cuda.synchronize()
            assert int(err.item()) == 0
            assert torch.equal(out, own) and torch.equal(lse, own_lse), case.name
            assert int(shared[:2048].count_nonzero().item()) == 0


def test_attention_persistent_bad_block_and_prefix(gpu_lib):
    """A persistent launch (512 pairs) with one sequence's block id out of range and
    another's prefix longer than max_prefix: the block error bit is set, nothing
    faults, and every other sequence's output still matches the oracle."""
    parents = [W.tree_random(np.random.default_rng(60 + b), 40 + b % 50, 8) for b in range(64)]
    plens = [300 + 41 * b for b in range(64)]
    case = W.make_case("badpers", parents, plens, 32, 8, 128, W.DT_BF16, 10, 37, with_probs=False)
    dev = W.case_to_device(case, probs=False)
    mn = max(1, case.max_nodes)
    anc, _, _, _ = gpu_index(gpu_lib, case, dev)
    dev["block_table"][5, 1] = case.k_cache.shape[0] + 7   # sequence 5: a block id past the pool
    dev["prefix_len"][9] = case.max_prefix + 1             # sequence 9: longer than max_prefix
    out, lse, err = gpu_lib.tree_verify_attention(
        dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"], dev["prefix_len"],
        dev["k_tree"], dev["v_tree"], dev["cu_nodes"], anc, mn, case.max_prefix)
    torch.cuda.synchronize()
    assert int(err.item()) & oracle.ERR_BLOCK
    nodes = sample_nodes(case, 4, seed=6, seqs={0, 4, 6, 8, 10, 63})
    want, _ = oracle_attention(case, nodes)
    rows = rows_of(case, nodes)
    assert np.isfinite(to_f64(out)[rows]).all()
    assert np.abs(to_f64(out)[rows] - want[rows]).max() <= TOL_BF16


def test_attention_aliased_block_tables(gpu_lib):
    parents = [W.tree_kary_levels(3, 3)] * 4
    case = W.make_case("alias", parents, [700] * 4, 8, 2, 128, W.DT_BF16, 10, 3, alias_prefix=True,
                       spare_blocks=5, with_probs=False)
    check_attention(gpu_lib, case, TOL_BF16)


def test_attention_max_node_cap(gpu_lib):
    case = W.make_case("cap", [W.tree_random(np.random.default_rng(2), 2048, 64)], [64], 2, 1, 128,
                       W.DT_BF16, 10, 4, with_probs=False)
    check_attention(gpu_lib, case, TOL_BF16, nodes=sample_nodes(case, 40))


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_attention_full_configs(gpu_lib, index):
    """The four bf16 verify workloads at full size, in the launch configuration the
    benchmark times: every node of the LLaVA-like tree; first, last and random nodes
    (all heads) of every sequence of the others."""
    case = W.make_config(index, with_probs=False)
    if index == 1:
        nodes = None
    else:
        nodes = sample_nodes(case, 12 if case.batch <= 8 else 2, seed=index)
    check_attention(gpu_lib, case, TOL_BF16, nodes=nodes)


def test_attention_repeatable(gpu_lib):
    case = W.make_config(1, with_probs=False)
    dev, anc = check_index(gpu_lib, case)
    a, la, _ = gpu_attention(gpu_lib, case, dev, anc)
    for _ in range(5):
        b, lb, _ = gpu_attention(gpu_lib, case, dev, anc)
        assert torch.equal(a, b) and torch.equal(la, lb)


# ------------------------------------------------------------------ acceptance

@pytest.mark.parametrize("index", [0, 1, 2, 3, 4])
def test_accept_configs_bitexact(gpu_lib, index):
    case = W.make_config(index)
    dev = W.case_to_device(case)
    got = gpu_accept(gpu_lib, case, dev, 16)
    assert_accept_equal(got, oracle_accept(case, 16))


@pytest.mark.parametrize("index", [0, 1, 3])
def test_accept_mostly_equal_rows(gpu_lib, index):
    """p_target = p_draft on ~80% of nodes: long accepted paths, residuals deep in the
    tree, and the target fallback when the rejection row has no residual mass."""
    case = W.make_config(index)
    rng = np.random.default_rng(index)
    same = rng.random(case.total_nodes) < 0.8
    case.p_target[same] = case.p_draft[same]
    dev = W.case_to_device(case)
    got = gpu_accept(gpu_lib, case, dev, 16)
    want = oracle_accept(case, 16)
    assert want["accept_len"].max() >= 2
    assert_accept_equal(got, want)


def test_accept_exhaustive_patterns_batched(gpu_lib):
    """Every accept pattern of a 9-node tree, one sequence per pattern, in one call."""
    par = W.tree_random(np.random.default_rng(3), 9, 4)
    n, vocab = 9, 4
    pats = 1 << n
    parents = [par] * pats
    case = W.make_case("pat", parents, [0] * pats, 1, 1, 64, W.DT_F32, vocab, 2, with_probs=False)
    pt = np.full((n * pats, vocab), 0.25, np.float32)
    for m in range(pats):
        for i in range(n):
            if not (m >> i) & 1:
                pt[m * n + i] = [0.0, 0.5, 0.25, 0.25]
    case.p_target, case.p_draft = pt, np.full_like(pt, 0.25)
    case.token = np.zeros(n * pats, np.int32)
    case.u_accept = np.full(n * pats, 0.5, np.float32)
    case.u_resample = W.grid_uniforms(np.random.default_rng(1), n * pats)
    dev = W.case_to_device(case)
    assert_accept_equal(gpu_accept(gpu_lib, case, dev, n), oracle_accept(case, n))


@pytest.mark.parametrize("vocab", [65537, 70002, 131072])
def test_accept_large_vocab_bitexact(gpu_lib, vocab):
    """Vocabularies past the one-kernel limit: residual sums per 4096-entry chunk (whole
    chunks by 16-byte loads when rows are 16-byte aligned, else element by element),
    then the chunk and the element; rows with mostly equal probabilities put the
    rejection point deep in the trees."""
    parents = [W.tree_random(np.random.default_rng(40 + b), n, 5) for b, n in enumerate([9, 1, 30])]
    case = W.make_case("bigv", parents, [0, 0, 0], 1, 1, 64, W.DT_F32, vocab, 31)
    rng = np.random.default_rng(vocab)
    same = rng.random(case.total_nodes) < 0.6
    case.p_target[same] = case.p_draft[same]
    dev = W.case_to_device(case)
    assert_accept_equal(gpu_accept(gpu_lib, case, dev, 8), oracle_accept(case, 8))


def own_rows_for(case, seed: int, frac: float = 0.8):
    """Own-context rows for bonus tokens: node i reads row i of a fresh set of
    probability rows with probability frac, else -1 (no row)."""
    rng = np.random.default_rng(seed)
    own_row = np.where(rng.random(case.total_nodes) < frac, np.arange(case.total_nodes), -1)
    return W.prob_rows(seed, 7, case.total_nodes, case.vocab), own_row.astype(np.int32)


@pytest.mark.parametrize("index", [0, 1, 2, 3, 4])
def test_accept_bonus_configs_bitexact(gpu_lib, index):
    """Bonus tokens on the five workloads: p_target = p_draft on ~90% of nodes, so
    many accepted paths end at leaves and draw from their own-context rows (80% of
    nodes have one); single-kernel and chunked vocabularies."""
    case = W.make_config(index)
    rng = np.random.default_rng(50 + index)
    same = rng.random(case.total_nodes) < 0.9
    case.p_target[same] = case.p_draft[same]
    own = own_rows_for(case, 60 + index)
    dev = W.case_to_device(case)
    want = oracle_accept(case, 16, own)
    got = gpu_accept(gpu_lib, case, dev, 16, own=own)
    assert_accept_equal(got, want)
    bonus = [b for b in range(case.batch)
             if want["accept_len"][b] > 0 and want["resample_node"][b] == want["path"][b][want["accept_len"][b] - 1]]
    assert bonus or case.batch == 1


def test_accept_bonus_exhaustive_patterns_batched(gpu_lib):
    """Every accept pattern of a 9-node tree with a point-mass own row per node: the
    bonus is drawn exactly when the winner is a leaf (its token names the node)."""
    par = W.tree_random(np.random.default_rng(3), 9, 4)
    n, vocab = 9, 16
    pats = 1 << n
    case = W.make_case("patb", [par] * pats, [0] * pats, 1, 1, 64, W.DT_F32, vocab, 2,
                       with_probs=False)
    pt = np.full((n * pats, vocab), 1.0 / vocab, np.float32)
    for m in range(pats):
        for i in range(n):
            if not (m >> i) & 1:
                pt[m * n + i, 0] = 0.0       # the drafted token 0 has no target mass
    case.p_target, case.p_draft = pt, np.full_like(pt, 1.0 / vocab)
    case.token = np.zeros(n * pats, np.int32)
    case.u_accept = np.full(n * pats, 0.5, np.float32)
    case.u_resample = W.grid_uniforms(np.random.default_rng(1), n * pats)
    own = np.zeros((n, vocab), np.float32)
    own[np.arange(n), np.arange(n) + 1] = 1.0
    own_row = np.tile(np.arange(n, dtype=np.int32), pats)
    dev = W.case_to_device(case)
    want = oracle_accept(case, n, (own, own_row))
    assert_accept_equal(gpu_accept(gpu_lib, case, dev, n, own=(own, own_row)), want)
    leaf_wins = sum(1 for m in range(pats) if want["resample_token"][m] == want["resample_node"][m] + 1)
    assert leaf_wins > 0


@pytest.mark.parametrize("vocab", [1000, 65537, 131072])
def test_accept_bonus_errors(gpu_lib, vocab):
    """Bonus rows outside [-1, own_rows), a bad uniform at the leaf and an all-zero own
    row: the same error bits and outputs as the oracle, in both launch shapes."""
    parents = [W.tree_chain(3)] * 5
    case = W.make_case("bonerr", parents, [0] * 5, 1, 1, 64, W.DT_F32, vocab, 12)
    case.p_target[:] = case.p_draft          # every chain accepted to its leaf
    own_rows = 4
    p_own = W.prob_rows(3, 9, own_rows, vocab)
    p_own[3] = 0.0
    own_row = np.full(case.total_nodes, -1, np.int32)
    leaf = [3 * b + 2 for b in range(5)]
    own_row[leaf] = [1, own_rows, 3, 2, -2]  # ok, past the rows, zero row, ok (bad u), negative
    case.u_resample[leaf[3]] = 1.0
    dev = W.case_to_device(case)
    ws = torch.zeros(max(1, gpu_lib.tree_accept_workspace_size(5, vocab)), dtype=torch.uint8,
                     device="cuda")
    want = oracle_accept(case, 4, (p_own, own_row))
    assert want["err"] == oracle.ERR_ZERO_MASS | oracle.ERR_UNIFORM | 128
    for _ in range(2):
        assert_accept_equal(gpu_accept(gpu_lib, case, dev, 4, own=(p_own, own_row), workspace=ws),
                            want)
        assert int(ws[:256].count_nonzero().item()) == 0   # ticket words left zero


def test_accept_error_words(gpu_lib):
    case = W.make_case("err", [W.tree_chain(3), W.tree_heap(7), W.tree_chain(4)], [0, 0, 0], 1, 1,
                       64, W.DT_F32, 50, 9)
    case.token[1] = 50                     # outside the vocabulary
    case.u_accept[4] = 1.0                 # uniform outside [0, 1)
    case.p_target[10:14] = case.p_draft[10:14]   # chain of 4 accepted, longer than max_path 3
    dev = W.case_to_device(case)
    got = gpu_accept(gpu_lib, case, dev, 3)
    want = oracle_accept(case, 3)
    assert want["err"] & oracle.ERR_TOKEN and want["err"] & oracle.ERR_UNIFORM
    assert want["err"] & oracle.ERR_PATH
    assert_accept_equal(got, want)


def test_accept_zero_mass(gpu_lib):
    case = W.make_case("zero", [W.tree_chain(2)], [0], 1, 1, 64, W.DT_F32, 8, 9)
    case.p_target[:] = 0.0
    dev = W.case_to_device(case)
    got = gpu_accept(gpu_lib, case, dev, 2)
    want = oracle_accept(case, 2)
    assert want["err"] == oracle.ERR_ZERO_MASS
    assert_accept_equal(got, want)


def test_accept_bad_parent_and_cap(gpu_lib):
    case = W.make_case("badp", [np.array([-1, 2, 0], np.int32), W.tree_heap(3)], [0, 0], 1, 1, 64,
                       W.DT_F32, 8, 9)
    dev = W.case_to_device(case)
    got = gpu_accept(gpu_lib, case, dev, 4)
    want = oracle_accept(case, 4)
    assert want["err"] == oracle.ERR_BAD_PARENT
    assert_accept_equal(got, want)


def test_accept_repeatable(gpu_lib):
    case = W.make_config(3)
    dev = W.case_to_device(case)
    first = gpu_accept(gpu_lib, case, dev, 16)
    for _ in range(20):
        again = gpu_accept(gpu_lib, case, dev, 16)
        for k in ("accept_len", "path", "resample_node", "resample_token", "node_ok"):
            np.testing.assert_array_equal(first[k], again[k])
