"""The C-ABI library: it loads, exports every entry point its header declares,
and rejects bad arguments on the host (no GPU work is enqueued for these)."""
import ctypes
import os
import re

import pytest

import tree_attention_verification_04_amd as tv
import oracle.probs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "treeverify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(tree_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tv.LIB_PATH):
        pytest.fail("libtreeverify.so is not built (run python -m tree_attention_verification_04_amd.build)")
    return tv.load()


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("tree_build_index", "tree_verify_attention", "tree_accept", "tree_last_error",
              "tree_verify_attention_workspace_size", "tree_accept_workspace_size"):
        assert n in names
    assert set(names) == set(tv.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(tv.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_last_error_starts_empty(lib):
    assert lib.tree_last_error() in (b"",) or isinstance(lib.tree_last_error(), bytes)


def test_build_index_host_checks(lib):
    one = ctypes.c_void_p(16)  # never dereferenced: the checks fail first
    assert lib.tree_build_index(one, one, 1, 4, 0, None, one, 1, one, None, one, None) == tv.TV_EUNSUPPORTED
    assert b"max_nodes" in lib.tree_last_error()
    assert lib.tree_build_index(one, one, 1, 4, 3000, None, one, 47, one, None, one, None) == tv.TV_EUNSUPPORTED
    assert lib.tree_build_index(one, one, 1, 4, 65, None, one, 1, one, None, one, None) == tv.TV_EINVAL
    assert lib.tree_build_index(one, None, 1, 4, 64, None, one, 1, one, None, one, None) == tv.TV_EINVAL
    assert lib.tree_build_index(one, one, -1, 4, 64, None, one, 1, one, None, one, None) == tv.TV_EINVAL
    assert lib.tree_build_index(one, one, 1, 4, 64, None, one, 1, one, one, one, None) == tv.TV_EINVAL
    # empty input: nothing to do, nothing launched
    assert lib.tree_build_index(None, one, 0, 0, 64, None, None, 1, None, None, one, None) == tv.TV_OK


def attn_call(lib, **kw):
    one = ctypes.c_void_p(16)
    args = dict(q=one, kc=one, vc=one, nblocks=4, bt=one, max_blocks=2, plen=one, kt=one, vt=one,
                cu=one, anc=one, words=1, batch=1, total=3, max_nodes=3, max_prefix=100, hq=4,
                hkv=2, d=128, dtype=tv.TV_DTYPE_BF16, scale=0.088, out=one, lse=None, ws=None,
                ws_bytes=0, err=one, stream=None)
    args.update(kw)
    return lib.tree_verify_attention(*args.values())


def test_attention_host_checks(lib):
    assert attn_call(lib, d=96) == tv.TV_EUNSUPPORTED
    assert attn_call(lib, dtype=7) == tv.TV_EUNSUPPORTED
    assert attn_call(lib, hq=3) == tv.TV_EINVAL
    assert attn_call(lib, words=0) == tv.TV_EINVAL
    assert attn_call(lib, scale=0.0) == tv.TV_EINVAL
    assert attn_call(lib, max_prefix=200) == tv.TV_EINVAL      # > max_blocks * 64
    assert attn_call(lib, q=None) == tv.TV_EINVAL
    assert attn_call(lib, err=None) == tv.TV_EINVAL
    assert attn_call(lib, max_nodes=4096, words=64) == tv.TV_EUNSUPPORTED
    # a short single verify splits its prefix: the workspace must be provided
    need = lib.tree_verify_attention_workspace_size(1, 64, 64, 1088, 32, 32, 128, tv.TV_DTYPE_BF16)
    assert need > 0
    assert attn_call(lib, total=64, max_nodes=64, max_prefix=1088, max_blocks=17, hq=32, hkv=32,
                     ws_bytes=need - 1, ws=ctypes.c_void_p(16)) == tv.TV_EWORKSPACE
    assert b"workspace" in lib.tree_last_error()
    # the fp32 path needs no workspace; one long work item per (sequence, KV head) and
    # compute unit needs none either
    assert lib.tree_verify_attention_workspace_size(1, 15, 15, 128, 4, 4, 64, tv.TV_DTYPE_F32) == 0
    assert lib.tree_verify_attention_workspace_size(4, 1024, 256, 32768, 64, 8, 128, tv.TV_DTYPE_BF16) == 0
    # every workspace starts with 2048 bytes of counter words (zero between calls)
    counters = 2048
    # more long items than compute units run persistently (queue heads in the counter
    # words), then the pair order; 512 pairs x 2 row tiles fill every die's last round,
    # so nothing is cut
    assert lib.tree_verify_attention_workspace_size(64, 5000, 96, 4096, 32, 8, 128,
                                                    tv.TV_DTYPE_BF16) == counters + 512 * 4
    # 64 pairs x 10 row tiles = 80 items per die of 32 compute units: the 16 items of the
    # last round are cut in 2 pieces, each with a 256-row partial (128 fp32 outputs, then
    # 1 log-sum-exp per row); then the pair order
    rows = 8 * 16 * 2 * 256
    lse_off = counters + rows * 128 * 4
    assert lse_off % 256 == 0 and (lse_off + rows * 4) % 256 == 0
    assert lib.tree_verify_attention_workspace_size(8, 4672, 584, 4096, 32, 8, 128,
                                                    tv.TV_DTYPE_BF16) == lse_off + rows * 4 + 64 * 4
    # one die's worth of items past full rounds decides the cut: 8 pairs x 41 row tiles
    # leave 9 items per die in the last round, cut in 3 pieces (3 rounds of a third of an
    # item, ceil(27/32) = 1, beat 2 pieces: ceil(18/32) / 2 + 0.02); 8 pairs x 33 row
    # tiles leave 1, cut in 7
    for max_nodes, plen, tail, pieces in ((1312, 512, 9, 3), (1025, 100, 1, 7)):
        rows = 8 * tail * pieces * 256
        lse_off = counters + rows * 128 * 4
        order_off = (lse_off + rows * 4 + 255) // 256 * 256
        assert lib.tree_verify_attention_workspace_size(1, max_nodes, max_nodes, plen, 64, 8, 128,
                                                        tv.TV_DTYPE_BF16) == order_off + 8 * 4
    # a single short verify: 32 pairs x 5 prefix splits of 64 rows
    rows = 5 * 64 * 32
    assert need == counters + rows * 128 * 4 + rows * 4


def fp8_call(lib, **kw):
    one = ctypes.c_void_p(16)
    args = dict(q=one, kc=one, vc=one, ks=one, vs=one, nblocks=4, bt=one, max_blocks=2, plen=one,
                kt=one, vt=one, cu=one, anc=one, words=1, batch=1, total=3, max_nodes=3,
                max_prefix=100, hq=4, hkv=2, scale=0.088, out=one, lse=None, ws=None, ws_bytes=0,
                err=one, stream=None)
    args.update(kw)
    return lib.tree_verify_attention_fp8kv(*args.values())


def test_fp8_attention_host_checks(lib):
    assert fp8_call(lib, ks=None) == tv.TV_EINVAL               # a prefix needs its scales
    assert fp8_call(lib, vs=None) == tv.TV_EINVAL
    assert b"scales" in lib.tree_last_error()
    assert fp8_call(lib, hq=3) == tv.TV_EINVAL
    assert fp8_call(lib, max_prefix=200) == tv.TV_EINVAL
    assert b"tree_verify_attention_fp8kv" in lib.tree_last_error()
    assert fp8_call(lib, batch=0) == tv.TV_OK                  # nothing to do
    # the FP8 cache is laid out like the bf16 one (its long items run the pipelined
    # kernel's register path): split partials of a short verify
    rows = 64 * 32
    need = lib.tree_verify_attention_fp8kv_workspace_size(1, 64, 64, 1088, 32, 32)
    # 2048 bytes of counter words first (every attention workspace keeps them), then
    # 5 splits of 4 blocks
    assert need == 2048 + 5 * rows * 128 * 4 + 5 * rows * 4
    # the same plans as bf16: persistent with cut tail items (wide tree), one round
    # (long context: no workspace)
    for shape in ((8, 4672, 584, 4096, 32, 8), (4, 1024, 256, 32768, 64, 8), (1, 64, 64, 1088, 32, 32)):
        assert lib.tree_verify_attention_fp8kv_workspace_size(*shape) == \
            lib.tree_verify_attention_workspace_size(*shape, 128, tv.TV_DTYPE_BF16)
    assert lib.tree_verify_attention_fp8kv_workspace_size(4, 1024, 256, 32768, 64, 8) == 0
    assert fp8_call(lib, total=64, max_nodes=64, max_prefix=1088, max_blocks=17, hq=32, hkv=32,
                    ws_bytes=need - 1, ws=ctypes.c_void_p(16)) == tv.TV_EWORKSPACE


def test_draft_build_host_checks(lib):
    one = ctypes.c_void_p(16)

    def call(**kw):
        args = dict(probs=one, u=one, batch=2, rows=65, k=8, n_max=64, depth=6, beta=0.7,
                    ratio=0.1, parent=one, slot=one, q=one, count=one, err=one, stream=None)
        args.update(kw)
        return lib.tree_draft_build(*args.values())

    assert call(k=17) == tv.TV_EUNSUPPORTED
    assert call(n_max=257) == tv.TV_EUNSUPPORTED
    assert call(k=0) == tv.TV_EINVAL
    assert call(depth=0) == tv.TV_EINVAL
    assert call(beta=-0.5) == tv.TV_EINVAL
    assert call(beta=float("inf")) == tv.TV_EINVAL
    assert call(ratio=1.5) == tv.TV_EINVAL
    assert call(err=None) == tv.TV_EINVAL
    assert call(probs=None) == tv.TV_EINVAL
    assert b"tree_draft_build" in lib.tree_last_error()
    assert call(batch=0) == tv.TV_OK


def test_accept_host_checks(lib):
    one = ctypes.c_void_p(16)
    need = lib.tree_accept_workspace_size(2, 100000)
    assert need >= 256 + 2 * 25 * 16          # tickets, then 25 chunks of 4096 entries

    def call(**kw):
        a = dict(pt=one, pd=one, tok=one, ua=one, ur=one, par=one, cu=one, own=None, own_row=None,
                 own_rows=0, batch=2, total=5, max_nodes=4, vocab=100000, max_path=4, alen=one,
                 path=one, rn=one, rt=one, ok=None, ws=one, ws_bytes=need, err=one, stream=None)
        a.update(kw)
        return lib.tree_accept(*a.values())

    assert call(vocab=0) == tv.TV_EUNSUPPORTED
    assert call(vocab=1 << 19) == tv.TV_EUNSUPPORTED
    assert call(max_nodes=5000) == tv.TV_EUNSUPPORTED
    assert call(ws_bytes=need - 1) == tv.TV_EWORKSPACE
    assert call(ws=None) == tv.TV_EWORKSPACE
    assert call(own_row=one, own_rows=3) == tv.TV_EINVAL      # own rows without p_own
    assert call(own_rows=-1) == tv.TV_EINVAL
    assert b"tree_accept" in lib.tree_last_error()
    assert call(pt=None) == tv.TV_EINVAL
    assert call(path=None) == tv.TV_EINVAL
    assert call(batch=0) == tv.TV_OK


def test_binding_refuses_cpu_tensors(lib):
    import torch
    par = torch.tensor([-1, 0], dtype=torch.int32)
    cu = torch.tensor([0, 2], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        tv.tree_build_index(par, cu, 2)


def commit_call(lib, **kw):
    one = ctypes.c_void_p(16)
    args = dict(kt=one, vt=one, cu=one, acc=one, path=one, batch=2, total=5, max_path=4, hkv=2,
                d=128, dtype=tv.TV_DTYPE_BF16, kc=one, vc=one, nblocks=4, bt=one, max_blocks=2,
                plen=one, err=one, stream=None)
    args.update(kw)
    return lib.tree_commit_kv(*args.values())


def test_commit_host_checks(lib):
    assert commit_call(lib, d=96) == tv.TV_EUNSUPPORTED
    assert commit_call(lib, dtype=5) == tv.TV_EUNSUPPORTED
    assert commit_call(lib, hkv=0) == tv.TV_EINVAL
    assert commit_call(lib, batch=-1) == tv.TV_EINVAL
    assert commit_call(lib, max_path=-2) == tv.TV_EINVAL
    assert commit_call(lib, err=None) == tv.TV_EINVAL
    assert commit_call(lib, plen=None) == tv.TV_EINVAL
    assert commit_call(lib, path=None) == tv.TV_EINVAL
    assert b"path" in lib.tree_last_error()
    assert commit_call(lib, kt=None) == tv.TV_EINVAL
    # nothing to do: no sequences (returns before any launch)
    assert commit_call(lib, batch=0, kt=None, vt=None, path=None) == tv.TV_OK


def test_softmax_rows_host_checks(lib):
    one = ctypes.c_void_p(16)
    call = lambda **kw: lib.tree_softmax_rows(*{**dict(lg=one, c=4, v=1000, row_of=None, r=4, t=1.0,
                                                       p=one, ws=one, wsb=64, err=one, s=None),
                                               **kw}.values())
    assert lib.tree_softmax_rows_workspace_size(4, 1000) == 4 * 1 * 8
    assert lib.tree_softmax_rows_workspace_size(2, 152064) == 2 * 19 * 8
    assert call(t=0.0) == tv.TV_EINVAL
    assert call(r=5) == tv.TV_EINVAL                 # rows != ctx_rows without row_of
    assert call(c=-1) == tv.TV_EINVAL
    assert call(err=None) == tv.TV_EINVAL
    assert call(wsb=8) == tv.TV_EWORKSPACE
    assert call(r=0, c=0) == tv.TV_OK                # nothing to do
    assert tv.TV_ERR_ROW == oracle.probs.ERR_ROW


def test_softmax_rows_kept_host_checks(lib):
    one = ctypes.c_void_p(16)  # never dereferenced: the checks fail first
    call = lambda **kw: lib.tree_softmax_rows_kept(*{**dict(lg=one, c=4, v=1000, keep=one, km=8,
                                                            row_of=None, r=4, t=1.0, p=one,
                                                            err=one, s=None), **kw}.values())
    assert call(km=0) == tv.TV_EUNSUPPORTED
    assert call(km=257) == tv.TV_EUNSUPPORTED
    assert b"keep_max" in lib.tree_last_error()
    assert call(t=-1.0) == tv.TV_EINVAL
    assert call(r=5) == tv.TV_EINVAL                 # rows != ctx_rows without row_of
    assert call(v=-1) == tv.TV_EINVAL
    assert call(err=None) == tv.TV_EINVAL
    assert call(keep=None) == tv.TV_EINVAL
    assert call(r=0, c=0) == tv.TV_OK                # nothing to do
    assert (tv.TV_ERR_TOKEN, tv.TV_ERR_ZERO_MASS) == (oracle.ERR_TOKEN, oracle.ERR_ZERO_MASS)


def test_uniforms_host_checks(lib):
    one = ctypes.c_void_p(16)  # never dereferenced: the checks fail first
    assert lib.tree_uniforms(1, 0, 0, one, one, one, -1, 4, one, one, None) == tv.TV_EINVAL
    assert lib.tree_uniforms(1, 0, 0, one, one, one, 1, -4, one, one, None) == tv.TV_EINVAL
    assert lib.tree_uniforms(1, 0, 0, one, one, one, 0, 4, one, one, None) == tv.TV_EINVAL
    assert lib.tree_uniforms(1, 0, 0, None, one, one, 1, 4, one, one, None) == tv.TV_EINVAL
    assert b"request_id" in lib.tree_last_error()
    assert lib.tree_uniforms(1, 0, 0, one, None, one, 1, 4, one, one, None) == tv.TV_EINVAL
    # nothing to do: no nodes, or no output asked for
    assert lib.tree_uniforms(1, 0, 0, None, None, None, 0, 0, None, None, None) == tv.TV_OK
    assert lib.tree_uniforms(1, 0, 0, one, one, one, 1, 4, None, None, None) == tv.TV_OK
    # 64-bit key and counter words pass through the ABI unchanged
    assert lib.tree_uniforms(2**64 - 1, 2**63, 2**64 - 1, one, one, one, 1, 0, one, one, None) == tv.TV_OK


def test_step_and_graph_host_checks(lib):
    assert lib.tree_verify_step_args_size() == ctypes.sizeof(tv.StepArgs)
    assert lib.tree_verify_step(None, None) == tv.TV_EINVAL
    h = ctypes.c_void_p()
    assert lib.tree_verify_graph_create(None, None, ctypes.byref(h)) == tv.TV_EINVAL
    assert lib.tree_verify_graph_create(ctypes.byref(tv.StepArgs()), None, None) == tv.TV_EINVAL
    assert lib.tree_verify_graph_launch(None, None) == tv.TV_EINVAL
    assert lib.tree_verify_graph_destroy(None) == tv.TV_OK
    # a step whose first call fails its host checks enqueues nothing
    a = tv.StepArgs()
    a.batch, a.total_nodes, a.max_nodes, a.words = 1, 4, 0, 1
    assert lib.tree_verify_step(ctypes.byref(a), None) == tv.TV_EUNSUPPORTED
    assert b"max_nodes" in lib.tree_last_error()


def mma8_call(lib, **kw):
    one = ctypes.c_void_p(16)  # 16-byte aligned, never dereferenced: the checks fail first
    args = dict(q=one, kc=one, vc=one, ke=one, ve=one, nblocks=4, bt=one, max_blocks=2, plen=one,
                kt=one, vt=one, kte=one, vte=one, cu=one, anc=one, words=1, batch=1, total=3,
                max_nodes=3, max_prefix=100, hq=4, hkv=2, scale=0.088, out=one, lse=None, ws=None,
                ws_bytes=0, err=one, stream=None)
    args.update(kw)
    return lib.tree_verify_attention_fp8(*args.values())


def test_fp8_matrix_core_attention_host_checks(lib):
    assert mma8_call(lib, ke=None) == tv.TV_EINVAL               # a prefix needs its exponents
    assert mma8_call(lib, ve=None) == tv.TV_EINVAL
    assert b"cache exponents" in lib.tree_last_error()
    assert mma8_call(lib, kte=None) == tv.TV_EINVAL              # the tree rows always do
    assert b"tree exponents" in lib.tree_last_error()
    assert mma8_call(lib, kt=ctypes.c_void_p(24)) == tv.TV_EINVAL  # 16-byte row chunks
    assert mma8_call(lib, vc=ctypes.c_void_p(40)) == tv.TV_EINVAL
    assert b"aligned" in lib.tree_last_error()
    assert mma8_call(lib, hq=3) == tv.TV_EINVAL
    assert mma8_call(lib, max_prefix=200) == tv.TV_EINVAL
    assert b"tree_verify_attention_fp8" in lib.tree_last_error()
    assert mma8_call(lib, batch=0) == tv.TV_OK                  # nothing to do
    # its plans are the bf16 ones (every work item runs the pipelined kernel)
    for shape in ((8, 4672, 584, 4096, 32, 8), (4, 1024, 256, 32768, 64, 8), (1, 64, 64, 1088, 32, 32),
                  (64, 3600, 96, 4096, 32, 8)):
        assert lib.tree_verify_attention_fp8_workspace_size(*shape) == \
            lib.tree_verify_attention_workspace_size(*shape, 128, tv.TV_DTYPE_BF16)
    need = lib.tree_verify_attention_fp8_workspace_size(1, 64, 64, 1088, 32, 32)
    assert mma8_call(lib, total=64, max_nodes=64, max_prefix=1088, max_blocks=17, hq=32, hkv=32,
                     ws_bytes=need - 1, ws=ctypes.c_void_p(16)) == tv.TV_EWORKSPACE


def test_quantize_rows_host_checks(lib):
    one = ctypes.c_void_p(16)
    assert lib.tree_quantize_rows_e4m3(one, tv.TV_DTYPE_BF16, -1, one, one, None) == tv.TV_EINVAL
    assert lib.tree_quantize_rows_e4m3(one, 7, 4, one, one, None) == tv.TV_EUNSUPPORTED
    assert lib.tree_quantize_rows_e4m3(None, tv.TV_DTYPE_BF16, 4, one, one, None) == tv.TV_EINVAL
    assert lib.tree_quantize_rows_e4m3(None, tv.TV_DTYPE_F32, 0, None, None, None) == tv.TV_OK
