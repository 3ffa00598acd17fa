"""Pins of the accepted-path KV commit oracle (CPU only).

The commit is a copy, so it is pinned by what the copy must achieve, checked
with code of the oracle it does not use:
  * reading the new prefix through the block table (the attention oracle's
    gather) gives the old prefix followed by the path's rows, and nothing else
    in the pool changes;
  * attention is unchanged by the commit: the last accepted node attends to the
    same keys whether its ancestors are tree nodes or committed prefix
    positions (the tree-attention oracle evaluated both ways);
  * invalid inputs leave the sequence untouched and set the documented bit.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle.attention import gather_prefix


def f64(case, a):
    return W.to_f64(a, case.dtype)


def chain_case(plens, lengths, seed=3, hq=4, hkv=2, d=64, dtype=W.DT_F32, extra_nodes=3):
    """Sequences whose trees are a chain (the accepted path) plus a few side nodes."""
    parents = []
    for n in lengths:
        p = list(range(-1, n - 1)) + [max(-1, n - 2)] * extra_nodes  # side nodes off the chain
        parents.append(np.asarray(p, dtype=np.int32))
    return W.make_case("commit", parents, plens, hq, hkv, d, dtype, 10, seed, with_probs=False,
                       reserve_tokens=max(lengths) + 1)


def paths_of(case, lengths, max_path):
    path = np.full((case.batch, max_path), -1, dtype=np.int32)
    for b, n in enumerate(lengths):
        path[b, :n] = np.arange(n)
    return np.asarray(lengths, dtype=np.int32), path


@pytest.mark.parametrize("plens,lengths", [([62], [5]), ([64], [3]), ([0], [4]),
                                           ([100, 7, 128], [6, 0, 1])])
def test_commit_appends_path_rows(plens, lengths):
    case = chain_case(plens, lengths)
    acc, path = paths_of(case, lengths, 8)
    kc, vc, pl, err = oracle.commit_kv(case.k_cache, case.v_cache, case.block_table, case.prefix_len,
                                       case.num_blocks, case.k_tree, case.v_tree, case.cu_nodes,
                                       acc, path, 8)
    assert err == 0
    touched = np.zeros(case.k_cache.shape[:1] + case.k_cache.shape[2:3], dtype=bool)  # [blk, t]
    for b in range(case.batch):
        n0, p0, n = case.cu_nodes[b], case.prefix_len[b], lengths[b]
        assert pl[b] == p0 + n
        for cache, new, tree in ((case.k_cache, kc, case.k_tree), (case.v_cache, vc, case.v_tree)):
            want = np.concatenate([gather_prefix(cache, case.block_table[b], p0),
                                   tree[n0 + path[b, :n]]], axis=0)
            assert np.array_equal(gather_prefix(new, case.block_table[b], p0 + n), want)
        for t in range(p0, p0 + n):
            touched[case.block_table[b, t // 64], t % 64] = True
    # every other slot of the pool is unchanged
    for cache, new in ((case.k_cache, kc), (case.v_cache, vc)):
        keep = ~touched
        assert np.array_equal(np.moveaxis(new, 2, 1)[keep], np.moveaxis(cache, 2, 1)[keep])


def test_commit_keeps_attention_of_the_last_node():
    """Committing the ancestors of w and then attending with w alone gives the
    same output as attending with w inside the tree (same visible keys)."""
    lengths, plens = [6], [70]
    case = chain_case(plens, lengths, dtype=W.DT_F32, d=64)
    w = lengths[0] - 1
    scale = 1.0 / np.sqrt(case.d)
    before, lse_b = oracle.tree_attention(
        f64(case, case.q), f64(case, case.k_cache), f64(case, case.v_cache), case.block_table,
        case.prefix_len, f64(case, case.k_tree), f64(case, case.v_tree), case.cu_nodes, case.parent,
        case.hq, case.hkv, scale, nodes=[[w]])
    acc, path = paths_of(case, [w], 8)  # commit the ancestors of w only
    kc, vc, pl, err = oracle.commit_kv(case.k_cache, case.v_cache, case.block_table, case.prefix_len,
                                       case.num_blocks, case.k_tree, case.v_tree, case.cu_nodes,
                                       acc, path, 8)
    assert err == 0 and pl[0] == plens[0] + w
    one = np.array([0, 1], dtype=np.int32)
    after, lse_a = oracle.tree_attention(
        f64(case, case.q[w:w + 1]), f64(case, kc), f64(case, vc), case.block_table, pl,
        f64(case, case.k_tree[w:w + 1]), f64(case, case.v_tree[w:w + 1]), one,
        np.array([-1], dtype=np.int32), case.hq, case.hkv, scale)
    assert np.abs(after[0] - before[w]).max() < 1e-12
    assert np.abs(lse_a[0] - lse_b[w]).max() < 1e-12


def test_commit_errors_leave_sequences_untouched():
    case = chain_case([10, 20, 30], [3, 3, 3])
    acc, path = paths_of(case, [3, 3, 3], 4)
    bt = case.block_table.copy()
    bt[1, 0] = case.num_blocks        # sequence 1: its block is outside the pool
    acc[2] = 5                        # sequence 2: longer than max_path
    kc, vc, pl, err = oracle.commit_kv(case.k_cache, case.v_cache, bt, case.prefix_len,
                                       case.num_blocks, case.k_tree, case.v_tree, case.cu_nodes,
                                       acc, path, 4)
    assert err == oracle.ERR_BLOCK | oracle.ERR_PATH
    assert list(pl) == [13, 20, 30]
    # sequence 0 was committed: its positions 10..12 changed, the others did not
    k_changed = np.argwhere(np.any(kc != case.k_cache, axis=(1, 3)))
    assert all(bt[0, t // 64] == blk and 10 <= t < 13 for blk, t in
               [(int(x), int(y)) for x, y in k_changed]) and len(k_changed) == 3
    # a path entry outside the sequence's nodes
    acc2, path2 = paths_of(case, [3, 3, 3], 4)
    path2[0, 1] = 99
    _, _, pl2, err2 = oracle.commit_kv(case.k_cache, case.v_cache, case.block_table, case.prefix_len,
                                       case.num_blocks, case.k_tree, case.v_tree, case.cu_nodes,
                                       acc2, path2, 4)
    assert err2 == oracle.ERR_PATH and list(pl2) == [10, 23, 33]


def test_planted_off_by_one_is_caught():
    """A commit that writes each row one position late fails the gather pin."""
    case = chain_case([62], [5])
    acc, path = paths_of(case, [5], 8)
    kc = case.k_cache.copy()
    for j in range(5):
        t = 62 + j + 1
        kc[case.block_table[0, t // 64], :, t % 64, :] = case.k_tree[path[0, j]]
    want = np.concatenate([gather_prefix(case.k_cache, case.block_table[0], 62),
                           case.k_tree[path[0, :5]]], axis=0)
    assert not np.array_equal(gather_prefix(kc, case.block_table[0], 67), want)


def shared_prefix_tables(case, shared_blocks: int):
    """Sequence 1's first `shared_blocks` logical blocks mapped to sequence 0's blocks."""
    bt = case.block_table.copy()
    bt[1, :shared_blocks] = bt[0, :shared_blocks]
    return bt


def test_commit_into_a_shared_block_is_refused():
    """Two sequences share a 100-token prefix (its second block is partly filled):
    both would append into that block, so neither is written and the block bit is
    set; a third, private sequence is committed."""
    case = chain_case([100, 100, 40], [3, 3, 3])
    bt = shared_prefix_tables(case, 2)
    acc, path = paths_of(case, [3, 3, 3], 4)
    kc, vc, pl, err = oracle.commit_kv(case.k_cache, case.v_cache, bt, case.prefix_len,
                                       case.num_blocks, case.k_tree, case.v_tree, case.cu_nodes,
                                       acc, path, 4)
    assert err == oracle.ERR_BLOCK
    assert list(pl) == [100, 100, 43]
    changed = {int(x) for x in np.argwhere(np.any(kc != case.k_cache, axis=(1, 2, 3)))[:, 0]}
    assert changed == {int(bt[2, 0])}
    # the shared prefix reads back unchanged through both tables
    for b in (0, 1):
        np.testing.assert_array_equal(gather_prefix(kc, bt[b], 100),
                                      gather_prefix(case.k_cache, bt[0], 100))


def test_commit_after_a_shared_whole_block_prefix():
    """A shared prefix of whole blocks (128 tokens) is only read: each sequence
    appends into a private block, no error, and the gather pin holds for both."""
    case = chain_case([128, 128], [4, 2])
    bt = shared_prefix_tables(case, 2)
    acc, path = paths_of(case, [4, 2], 4)
    kc, vc, pl, err = oracle.commit_kv(case.k_cache, case.v_cache, bt, case.prefix_len,
                                       case.num_blocks, case.k_tree, case.v_tree, case.cu_nodes,
                                       acc, path, 4)
    assert err == 0 and list(pl) == [132, 130]
    for b, n in enumerate([4, 2]):
        n0 = int(case.cu_nodes[b])
        want = np.concatenate([gather_prefix(case.k_cache, bt[b], 128),
                               case.k_tree[n0 + path[b, :n]]], axis=0)
        np.testing.assert_array_equal(gather_prefix(kc, bt[b], 128 + n), want)
