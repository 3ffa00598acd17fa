"""Python binding of libtreeverify (tree verification for speculative decoding on MI355X).

Argument marshalling only: each function checks tensor devices, dtypes and
shapes, allocates outputs with torch on the current device when the caller
does not pass them, and calls the C entry point of the same name on torch's
current HIP stream.  Every step of the computation runs in the HIP kernels of
libtreeverify.so; there is no other implementation behind these functions,
and they raise if the library is missing.

Device error words: `err` is an int32 tensor of one element that the kernels
OR TV_ERR_* bits into; functions create a zeroed one unless given one.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtreeverify.so")

TV_OK, TV_EINVAL, TV_EUNSUPPORTED, TV_EHIP, TV_EWORKSPACE = 0, 1, 2, 3, 4
TV_ERR_BAD_PARENT = 1
TV_ERR_TOO_MANY_NODES = 2
TV_ERR_TOKEN = 4
TV_ERR_BLOCK = 8
TV_ERR_ZERO_MASS = 16
TV_ERR_PATH = 32
TV_ERR_UNIFORM = 64
TV_ERR_ROW = 128
TV_ERR_DRAFT = 256
TV_DTYPE_F32, TV_DTYPE_BF16 = 0, 1
TV_MAX_NODES = 2048
TV_BLOCK = 64

EXPORTS = (
    "tree_build_index",
    "tree_verify_attention_workspace_size",
    "tree_verify_attention",
    "tree_verify_attention_fp8kv_workspace_size",
    "tree_verify_attention_fp8kv",
    "tree_verify_attention_fp8_workspace_size",
    "tree_verify_attention_fp8",
    "tree_draft_build",
    "tree_accept_workspace_size",
    "tree_accept",
    "tree_accept_noalloc",
    "tree_commit_kv",
    "tree_softmax_rows_workspace_size",
    "tree_softmax_rows",
    "tree_softmax_rows_kept",
    "tree_uniforms",
    "tree_quantize_rows_e4m3",
    "tree_verify_step_args_size",
    "tree_verify_step",
    "tree_verify_graph_create",
    "tree_verify_graph_launch",
    "tree_verify_graph_destroy",
    "tree_last_error",
)

_lib = None


class TreeVerifyError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class StepArgs(ctypes.Structure):
    """tree_verify_step_args of treeverify.h, field for field."""
    _P, _I = ctypes.c_void_p, ctypes.c_int32
    _fields_ = [
        ("parent", _P), ("cu_nodes", _P), ("batch", _I), ("total_nodes", _I), ("max_nodes", _I),
        ("words", _I), ("prefix_len", _P), ("anc_bits", _P), ("depth", _P), ("pos", _P),
        ("q", _P), ("k_cache", _P), ("v_cache", _P), ("block_table", _P), ("num_blocks", _I),
        ("max_blocks", _I), ("max_prefix", _I), ("hq", _I), ("hkv", _I), ("head_dim", _I),
        ("dtype", _I), ("softmax_scale", ctypes.c_float), ("k_tree", _P), ("v_tree", _P),
        ("out", _P), ("lse", _P), ("attn_workspace", _P), ("attn_workspace_bytes", ctypes.c_size_t),
        ("p_target", _P), ("p_draft", _P), ("token", _P), ("u_accept", _P), ("u_resample", _P),
        ("p_own", _P), ("own_row", _P), ("own_rows", _I), ("vocab", _I), ("max_path", _I),
        ("reserved", _I), ("accept_len", _P), ("path", _P), ("resample_node", _P),
        ("resample_token", _P), ("node_ok", _P), ("accept_workspace", _P),
        ("accept_workspace_bytes", ctypes.c_size_t), ("err", _P),
    ]


def _declare(lib: ctypes.CDLL) -> None:
    P, I, Z, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    lib.tree_build_index.argtypes = [P, P, I, I, I, P, P, I, P, P, P, P]
    lib.tree_build_index.restype = ctypes.c_int
    lib.tree_verify_attention_workspace_size.argtypes = [I] * 8
    lib.tree_verify_attention_workspace_size.restype = Z
    lib.tree_verify_attention.argtypes = [P, P, P, I, P, I, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                          I, F, P, P, P, Z, P, P]
    lib.tree_verify_attention.restype = ctypes.c_int
    lib.tree_verify_attention_fp8kv_workspace_size.argtypes = [I] * 6
    lib.tree_verify_attention_fp8kv_workspace_size.restype = Z
    lib.tree_verify_attention_fp8kv.argtypes = [P, P, P, P, P, I, P, I, P, P, P, P, P, I, I, I, I,
                                                I, I, I, F, P, P, P, Z, P, P]
    lib.tree_verify_attention_fp8kv.restype = ctypes.c_int
    lib.tree_verify_attention_fp8_workspace_size.argtypes = [I] * 6
    lib.tree_verify_attention_fp8_workspace_size.restype = Z
    lib.tree_verify_attention_fp8.argtypes = [P, P, P, P, P, I, P, I, P, P, P, P, P, P, P, I, I,
                                              I, I, I, I, I, F, P, P, P, Z, P, P]
    lib.tree_verify_attention_fp8.restype = ctypes.c_int
    lib.tree_draft_build.argtypes = [P, P, I, I, I, I, I, F, F, P, P, P, P, P, P]
    lib.tree_draft_build.restype = ctypes.c_int
    lib.tree_accept_workspace_size.argtypes = [I, I]
    lib.tree_accept_workspace_size.restype = Z
    lib.tree_accept.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, P,
                                Z, P, P]
    lib.tree_accept.restype = ctypes.c_int
    lib.tree_accept_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P,
                                        P, P]
    lib.tree_accept_noalloc.restype = ctypes.c_int
    lib.tree_commit_kv.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, P, I, P, I, P, P, P]
    lib.tree_commit_kv.restype = ctypes.c_int
    lib.tree_softmax_rows_workspace_size.argtypes = [I, I]
    lib.tree_softmax_rows_workspace_size.restype = Z
    lib.tree_softmax_rows.argtypes = [P, I, I, P, I, F, P, P, Z, P, P]
    lib.tree_softmax_rows.restype = ctypes.c_int
    lib.tree_softmax_rows_kept.argtypes = [P, I, I, P, I, P, I, F, P, P, P]
    lib.tree_softmax_rows_kept.restype = ctypes.c_int
    U64 = ctypes.c_uint64
    lib.tree_uniforms.argtypes = [U64, U64, U64, P, P, P, I, I, P, P, P]
    lib.tree_uniforms.restype = ctypes.c_int
    lib.tree_quantize_rows_e4m3.argtypes = [P, I, ctypes.c_int64, P, P, P]
    lib.tree_quantize_rows_e4m3.restype = ctypes.c_int
    lib.tree_verify_step_args_size.argtypes = []
    lib.tree_verify_step_args_size.restype = Z
    lib.tree_verify_step.argtypes = [ctypes.POINTER(StepArgs), P]
    lib.tree_verify_step.restype = ctypes.c_int
    lib.tree_verify_graph_create.argtypes = [ctypes.POINTER(StepArgs), P, ctypes.POINTER(P)]
    lib.tree_verify_graph_create.restype = ctypes.c_int
    lib.tree_verify_graph_launch.argtypes = [P, P]
    lib.tree_verify_graph_launch.restype = ctypes.c_int
    lib.tree_verify_graph_destroy.argtypes = [P]
    lib.tree_verify_graph_destroy.restype = ctypes.c_int
    if lib.tree_verify_step_args_size() != ctypes.sizeof(StepArgs):
        raise RuntimeError("tree_verify_step_args layout differs between the library and the binding")
    lib.tree_last_error.argtypes = []
    lib.tree_last_error.restype = ctypes.c_char_p


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtreeverify.so (built by build.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing: build it with `python -m tree_attention_verification_04_amd.build`")
        lib = ctypes.CDLL(path)
        _declare(lib)
        _lib = lib
    return _lib


def _check(fn: str, status: int) -> None:
    if status != TV_OK:
        raise TreeVerifyError(fn, status, load().tree_last_error().decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype | tuple, dim: int | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise TypeError(f"{name} must have dtype {dts}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions, got {t.dim()}")


def _err_word(err, device) -> torch.Tensor:
    if err is None:
        return torch.zeros(1, dtype=torch.int32, device=device)
    _need(err, "err", torch.int32)
    return err


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return TV_DTYPE_F32
    if dt == torch.bfloat16:
        return TV_DTYPE_BF16
    raise TypeError(f"unsupported dtype {dt}")


def tree_build_index(parent: torch.Tensor, cu_nodes: torch.Tensor, max_nodes: int,
                     prefix_len: torch.Tensor | None = None, *, words: int | None = None,
                     anc: torch.Tensor | None = None, depth: torch.Tensor | None = None,
                     pos: torch.Tensor | None = None, err: torch.Tensor | None = None,
                     stream=None):
    """Depth and ancestor-or-self bitsets of flattened draft trees.

    Returns (anc [total, words] int64 holding the uint64 bit patterns,
    depth [total] int32, pos [total] int32 or None, err [1] int32).
    """
    lib = load()
    _need(parent, "parent", torch.int32, 1)
    _need(cu_nodes, "cu_nodes", torch.int32, 1)
    dev = parent.device
    total = parent.numel()
    batch = cu_nodes.numel() - 1
    words = words if words is not None else max(1, math.ceil(max_nodes / 64))
    if anc is None:
        anc = torch.empty((total, words), dtype=torch.int64, device=dev)
    if depth is None:
        depth = torch.empty(total, dtype=torch.int32, device=dev)
    if prefix_len is not None:
        _need(prefix_len, "prefix_len", torch.int32, 1)
        if pos is None:
            pos = torch.empty(total, dtype=torch.int32, device=dev)
    err = _err_word(err, dev)
    _check("tree_build_index",
           lib.tree_build_index(_ptr(parent), _ptr(cu_nodes), batch, total, max_nodes,
                                _ptr(prefix_len), _ptr(anc), words, _ptr(depth),
                                _ptr(pos) if prefix_len is not None else None, _ptr(err),
                                _stream(stream)))
    return anc, depth, (pos if prefix_len is not None else None), err


def tree_verify_attention_workspace_size(batch, total_nodes, max_nodes, max_prefix, hq, hkv,
                                         head_dim, dtype: int) -> int:
    return int(load().tree_verify_attention_workspace_size(batch, total_nodes, max_nodes,
                                                           max_prefix, hq, hkv, head_dim, dtype))


def tree_verify_attention(q, k_cache, v_cache, block_table, prefix_len, k_tree, v_tree, cu_nodes,
                          anc, max_nodes: int, max_prefix: int, scale: float | None = None, *,
                          out=None, lse=None, want_lse: bool = True, workspace=None, err=None,
                          stream=None):
    """Tree attention over the paged prefix and each node's ancestors.

    q [total, hq, D]; k_cache/v_cache [num_blocks, hkv, 64, D]; block_table
    [batch, max_blocks] int32; prefix_len [batch] int32; k_tree/v_tree
    [total, hkv, D]; anc from tree_build_index.  Returns (out, lse, err).
    workspace: a uint8 device tensor of at least the queried size, zero-filled
    before its first use (every call leaves its counter words zero again); a
    fresh zeroed one is allocated when none is given.
    """
    lib = load()
    fdt = (torch.float32, torch.bfloat16)
    _need(q, "q", fdt, 3)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, name, q.dtype, 4)
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree)):
        _need(t, name, q.dtype, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(prefix_len, "prefix_len", torch.int32, 1)
    _need(cu_nodes, "cu_nodes", torch.int32, 1)
    _need(anc, "anc", torch.int64, 2)
    total, hq, d = q.shape
    num_blocks, hkv, blk, d2 = k_cache.shape
    if blk != TV_BLOCK or d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [num_blocks, hkv, 64, head_dim]")
    if tuple(k_tree.shape) != (total, hkv, d) or tuple(v_tree.shape) != (total, hkv, d):
        raise ValueError("k_tree/v_tree must be [total_nodes, hkv, head_dim]")
    if anc.shape[0] != total:
        raise ValueError("anc must have one row per node")
    batch = cu_nodes.numel() - 1
    if block_table.shape[0] != batch or prefix_len.numel() != batch:
        raise ValueError("block_table / prefix_len must have one row per sequence")
    dt = dtype_code(q.dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((total, hq), dtype=torch.float32, device=q.device)
    need = tree_verify_attention_workspace_size(batch, total, max_nodes, max_prefix, hq, hkv, d, dt)
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)  # zeroed once, kept zero
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    err = _err_word(err, q.device)
    _check("tree_verify_attention",
           lib.tree_verify_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), num_blocks,
                                     _ptr(block_table), block_table.shape[1], _ptr(prefix_len),
                                     _ptr(k_tree), _ptr(v_tree), _ptr(cu_nodes), _ptr(anc),
                                     anc.shape[1], batch, total, max_nodes, max_prefix, hq, hkv,
                                     d, dt, scale, _ptr(out), _ptr(lse), _ptr(workspace),
                                     ws_bytes, _ptr(err), _stream(stream)))
    return out, lse, err


def tree_verify_attention_fp8kv_workspace_size(batch, total_nodes, max_nodes, max_prefix, hq,
                                               hkv) -> int:
    return int(load().tree_verify_attention_fp8kv_workspace_size(batch, total_nodes, max_nodes,
                                                                 max_prefix, hq, hkv))


def tree_verify_attention_fp8kv(q, k_cache, v_cache, k_scale, v_scale, block_table, prefix_len,
                                k_tree, v_tree, cu_nodes, anc, max_nodes: int, max_prefix: int,
                                scale: float | None = None, *, out=None, lse=None,
                                want_lse: bool = True, workspace=None, err=None, stream=None):
    """Tree attention over an FP8 (E4M3) paged prefix cache with per-row scales.

    q [total, hq, 128] bf16; k_cache/v_cache [num_blocks, hkv, 64, 128] uint8;
    k_scale/v_scale [num_blocks, hkv, 64] float32; the rest as for
    tree_verify_attention.  Returns (out, lse, err).
    """
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, name, torch.uint8, 4)
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _need(t, name, torch.float32, 3)
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree)):
        _need(t, name, torch.bfloat16, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(prefix_len, "prefix_len", torch.int32, 1)
    _need(cu_nodes, "cu_nodes", torch.int32, 1)
    _need(anc, "anc", torch.int64, 2)
    total, hq, d = q.shape
    num_blocks, hkv, blk, d2 = k_cache.shape
    if d != 128 or blk != TV_BLOCK or d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [num_blocks, hkv, 64, 128] and head_dim 128")
    if tuple(k_scale.shape) != (num_blocks, hkv, blk) or tuple(v_scale.shape) != tuple(k_scale.shape):
        raise ValueError("k_scale/v_scale must be [num_blocks, hkv, 64]")
    if tuple(k_tree.shape) != (total, hkv, d) or tuple(v_tree.shape) != (total, hkv, d):
        raise ValueError("k_tree/v_tree must be [total_nodes, hkv, head_dim]")
    if anc.shape[0] != total:
        raise ValueError("anc must have one row per node")
    batch = cu_nodes.numel() - 1
    if block_table.shape[0] != batch or prefix_len.numel() != batch:
        raise ValueError("block_table / prefix_len must have one row per sequence")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((total, hq), dtype=torch.float32, device=q.device)
    need = tree_verify_attention_fp8kv_workspace_size(batch, total, max_nodes, max_prefix, hq, hkv)
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    err = _err_word(err, q.device)
    _check("tree_verify_attention_fp8kv",
           lib.tree_verify_attention_fp8kv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                           _ptr(v_scale), num_blocks, _ptr(block_table),
                                           block_table.shape[1], _ptr(prefix_len), _ptr(k_tree),
                                           _ptr(v_tree), _ptr(cu_nodes), _ptr(anc), anc.shape[1],
                                           batch, total, max_nodes, max_prefix, hq, hkv, scale,
                                           _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                           _ptr(err), _stream(stream)))
    return out, lse, err


def tree_draft_build(probs, u, max_depth: int, beta: float, prune_ratio: float, *, parent=None,
                     slot=None, q_draft=None, count=None, err=None, stream=None):
    """Candidate trees from draft top-K rows.  probs [batch, rows, k] float32
    (rows non-increasing), u [batch, n_max] float32 in [0, 1).  Returns
    (parent, slot, q_draft, count, err); see tree_draft_build in treeverify.h."""
    lib = load()
    _need(probs, "probs", torch.float32, 3)
    _need(u, "u", torch.float32, 2)
    batch, rows, k = probs.shape
    if u.shape[0] != batch:
        raise ValueError("u must have one row per sequence")
    n_max = u.shape[1]
    dev = probs.device
    if parent is None:
        parent = torch.empty((batch, n_max), dtype=torch.int32, device=dev)
    if slot is None:
        slot = torch.empty((batch, n_max), dtype=torch.int32, device=dev)
    if q_draft is None:
        q_draft = torch.empty((batch, n_max), dtype=torch.float32, device=dev)
    if count is None:
        count = torch.empty(batch, dtype=torch.int32, device=dev)
    err = _err_word(err, dev)
    _check("tree_draft_build",
           lib.tree_draft_build(_ptr(probs), _ptr(u), batch, rows, k, n_max, max_depth,
                                float(beta), float(prune_ratio), _ptr(parent), _ptr(slot),
                                _ptr(q_draft), _ptr(count), _ptr(err), _stream(stream)))
    return parent, slot, q_draft, count, err


def tree_accept_workspace_size(batch: int, vocab: int) -> int:
    return int(load().tree_accept_workspace_size(batch, vocab))


def tree_accept(p_target, p_draft, token, u_accept, u_resample, parent, cu_nodes, max_nodes: int,
                max_path: int, *, p_own=None, own_row=None, node_ok=True,
                outputs: dict | None = None, workspace=None, err=None, stream=None) -> dict:
    """Ratio test, longest accepted path and residual resample for every sequence.

    p_own [R, vocab] float32 / own_row [total] int32 (optional, together): target
    rows at each node's own context (-1 = none); a path that ends at a leaf then
    draws its bonus token from the leaf's row.
    workspace: a uint8 device tensor of at least tree_accept_workspace_size bytes,
    zero-filled before its first use (every call leaves its ticket words zero); a
    zeroed one is allocated when none is given.
    Returns dict(accept_len [B], path [B, max_path], resample_node [B],
    resample_token [B], node_ok [total] uint8 or None, err [1]).
    """
    lib = load()
    _need(p_target, "p_target", torch.float32, 2)
    _need(p_draft, "p_draft", torch.float32, 2)
    for name, t in (("token", token), ("parent", parent), ("cu_nodes", cu_nodes)):
        _need(t, name, torch.int32, 1)
    for name, t in (("u_accept", u_accept), ("u_resample", u_resample)):
        _need(t, name, torch.float32, 1)
    total, vocab = p_target.shape
    if tuple(p_draft.shape) != (total, vocab):
        raise ValueError("p_draft must match p_target")
    if (p_own is None) != (own_row is None):
        raise ValueError("p_own and own_row go together")
    own_rows = 0
    if p_own is not None:
        _need(p_own, "p_own", torch.float32, 2)
        _need(own_row, "own_row", torch.int32, 1)
        if p_own.shape[1] != vocab or own_row.numel() != total:
            raise ValueError("p_own must be [rows, vocab] and own_row [total_nodes]")
        own_rows = p_own.shape[0]
    batch = cu_nodes.numel() - 1
    dev = p_target.device
    o = outputs if outputs is not None else {}
    if not o:
        o["accept_len"] = torch.empty(batch, dtype=torch.int32, device=dev)
        o["path"] = torch.empty((batch, max_path), dtype=torch.int32, device=dev)
        o["resample_node"] = torch.empty(batch, dtype=torch.int32, device=dev)
        o["resample_token"] = torch.empty(batch, dtype=torch.int32, device=dev)
        o["node_ok"] = torch.empty(total, dtype=torch.uint8, device=dev) if node_ok else None
    need = tree_accept_workspace_size(batch, vocab)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)  # kept zero
    err = _err_word(err, dev)
    o["err"] = err
    _check("tree_accept",
           lib.tree_accept(_ptr(p_target), _ptr(p_draft), _ptr(token), _ptr(u_accept),
                           _ptr(u_resample), _ptr(parent), _ptr(cu_nodes), _ptr(p_own),
                           _ptr(own_row), own_rows, batch, total, max_nodes, vocab, max_path,
                           _ptr(o["accept_len"]), _ptr(o["path"]),
                           _ptr(o["resample_node"]), _ptr(o["resample_token"]),
                           _ptr(o.get("node_ok")), _ptr(workspace),
                           workspace.numel(), _ptr(err), _stream(stream)))
    return o


def tree_accept_noalloc(p_target, p_draft, token, u_accept, u_resample, parent, cu_nodes,
                        max_nodes: int, max_path: int, *, p_own=None, own_row=None, outputs: dict,
                        err: torch.Tensor, stream=None) -> dict:
    """tree_accept without a workspace: the chunked launch uses the library's fixed
    per-GPU scratch (at most 1024 sequences above 65536 vocabulary entries).  The
    caller passes every output (outputs: accept_len, path, resample_node,
    resample_token, node_ok or None) and the error word; nothing is allocated here.
    Calls that overlap on one GPU race on the scratch."""
    lib = load()
    _need(p_target, "p_target", torch.float32, 2)
    _need(p_draft, "p_draft", torch.float32, 2)
    for name, t in (("token", token), ("parent", parent), ("cu_nodes", cu_nodes)):
        _need(t, name, torch.int32, 1)
    for name, t in (("u_accept", u_accept), ("u_resample", u_resample)):
        _need(t, name, torch.float32, 1)
    total, vocab = p_target.shape
    if tuple(p_draft.shape) != (total, vocab):
        raise ValueError("p_draft must match p_target")
    if (p_own is None) != (own_row is None):
        raise ValueError("p_own and own_row go together")
    own_rows = 0
    if p_own is not None:
        _need(p_own, "p_own", torch.float32, 2)
        _need(own_row, "own_row", torch.int32, 1)
        if p_own.shape[1] != vocab or own_row.numel() != total:
            raise ValueError("p_own must be [rows, vocab] and own_row [total_nodes]")
        own_rows = p_own.shape[0]
    batch = cu_nodes.numel() - 1
    _need(err, "err", torch.int32)
    o = outputs
    if tuple(o["path"].shape) != (batch, max_path):
        raise ValueError("outputs['path'] must be [batch, max_path]")
    _check("tree_accept_noalloc",
           lib.tree_accept_noalloc(_ptr(p_target), _ptr(p_draft), _ptr(token), _ptr(u_accept),
                                   _ptr(u_resample), _ptr(parent), _ptr(cu_nodes), _ptr(p_own),
                                   _ptr(own_row), own_rows, batch, total, max_nodes, vocab,
                                   max_path, _ptr(o["accept_len"]), _ptr(o["path"]),
                                   _ptr(o["resample_node"]), _ptr(o["resample_token"]),
                                   _ptr(o.get("node_ok")), _ptr(err), _stream(stream)))
    return o


def tree_commit_kv(k_tree, v_tree, cu_nodes, accept_len, path, k_cache, v_cache, block_table,
                   prefix_len, *, err=None, stream=None) -> torch.Tensor:
    """Append each sequence's accepted path (tree_accept's accept_len / path) to its
    paged prefix: K/V rows copied to positions prefix_len[b] + j, prefix_len
    increased in place.  Returns the error word."""
    lib = load()
    _need(k_tree, "k_tree", (torch.float32, torch.bfloat16), 3)
    _need(v_tree, "v_tree", k_tree.dtype, 3)
    _need(k_cache, "k_cache", k_tree.dtype, 4)
    _need(v_cache, "v_cache", k_tree.dtype, 4)
    for name, t in (("cu_nodes", cu_nodes), ("accept_len", accept_len), ("prefix_len", prefix_len)):
        _need(t, name, torch.int32, 1)
    _need(path, "path", torch.int32, 2)
    _need(block_table, "block_table", torch.int32, 2)
    total, hkv, d = k_tree.shape
    if tuple(v_tree.shape) != (total, hkv, d):
        raise ValueError("v_tree must match k_tree")
    num_blocks = k_cache.shape[0]
    if tuple(k_cache.shape[1:]) != (hkv, TV_BLOCK, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [num_blocks, hkv, 64, head_dim]")
    batch = cu_nodes.numel() - 1
    if accept_len.numel() != batch or path.shape[0] != batch or prefix_len.numel() != batch \
            or block_table.shape[0] != batch:
        raise ValueError("accept_len, path, prefix_len and block_table need one row per sequence")
    err = _err_word(err, k_tree.device)
    _check("tree_commit_kv",
           lib.tree_commit_kv(_ptr(k_tree), _ptr(v_tree), _ptr(cu_nodes), _ptr(accept_len),
                              _ptr(path), batch, total, path.shape[1], hkv, d,
                              dtype_code(k_tree.dtype), _ptr(k_cache), _ptr(v_cache), num_blocks,
                              _ptr(block_table), block_table.shape[1], _ptr(prefix_len), _ptr(err),
                              _stream(stream)))
    return err


def tree_softmax_rows(logits, row_of=None, *, inv_temperature: float = 1.0, probs=None,
                      workspace=None, err=None, stream=None):
    """Probability rows softmax(t * logits[row_of[i]]) (row_of=None: one row per
    logits row).  Returns (probs [rows, vocab] float32, err)."""
    lib = load()
    _need(logits, "logits", torch.float32, 2)
    ctx_rows, vocab = logits.shape
    if row_of is not None:
        _need(row_of, "row_of", torch.int32, 1)
    rows = ctx_rows if row_of is None else row_of.numel()
    if probs is None:
        probs = torch.empty((rows, vocab), dtype=torch.float32, device=logits.device)
    _need(probs, "probs", torch.float32, 2)
    if tuple(probs.shape) != (rows, vocab):
        raise ValueError("probs must be [rows, vocab]")
    need = int(lib.tree_softmax_rows_workspace_size(ctx_rows, vocab))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=logits.device)
    err = _err_word(err, logits.device)
    _check("tree_softmax_rows",
           lib.tree_softmax_rows(_ptr(logits), ctx_rows, vocab, _ptr(row_of), rows,
                                 float(inv_temperature), _ptr(probs), _ptr(workspace),
                                 workspace.numel(), _ptr(err), _stream(stream)))
    return probs, err


def tree_softmax_rows_kept(logits, keep, row_of=None, *, inv_temperature: float = 1.0,
                           probs=None, err=None, stream=None):
    """Probability rows over each context row's kept set (keep [ctx_rows, keep_max]
    int32 token ids, -1 = padding), zero elsewhere: the pruned draft distribution.
    Returns (probs [rows, vocab] float32, err)."""
    lib = load()
    _need(logits, "logits", torch.float32, 2)
    _need(keep, "keep", torch.int32, 2)
    ctx_rows, vocab = logits.shape
    if keep.shape[0] != ctx_rows:
        raise ValueError("keep must have one row per logits row")
    if row_of is not None:
        _need(row_of, "row_of", torch.int32, 1)
    rows = ctx_rows if row_of is None else row_of.numel()
    if probs is None:
        probs = torch.empty((rows, vocab), dtype=torch.float32, device=logits.device)
    _need(probs, "probs", torch.float32, 2)
    if tuple(probs.shape) != (rows, vocab):
        raise ValueError("probs must be [rows, vocab]")
    err = _err_word(err, logits.device)
    _check("tree_softmax_rows_kept",
           lib.tree_softmax_rows_kept(_ptr(logits), ctx_rows, vocab, _ptr(keep), keep.shape[1],
                                      _ptr(row_of), rows, float(inv_temperature), _ptr(probs),
                                      _ptr(err), _stream(stream)))
    return probs, err


def tree_uniforms(request_id, depth, cu_nodes, *, seed: int, step: int, purpose: int = 0,
                  u_accept=None, u_resample=None, stream=None):
    """Acceptance and resample uniforms of every node from the counter-based generator
    (Philox4x64-10 keyed by (seed, purpose), counter = (local node, depth, step,
    request_id[b])).  Returns (u_accept, u_resample), float32 [total_nodes]."""
    lib = load()
    _need(request_id, "request_id", torch.int64, 1)
    _need(depth, "depth", torch.int32, 1)
    _need(cu_nodes, "cu_nodes", torch.int32, 1)
    batch, total = request_id.numel(), depth.numel()
    if cu_nodes.numel() != batch + 1:
        raise ValueError("cu_nodes must hold batch + 1 entries")
    if u_accept is None:
        u_accept = torch.empty(total, dtype=torch.float32, device=depth.device)
    if u_resample is None:
        u_resample = torch.empty(total, dtype=torch.float32, device=depth.device)
    for t, name in ((u_accept, "u_accept"), (u_resample, "u_resample")):
        _need(t, name, torch.float32, 1)
        if t.numel() != total:
            raise ValueError(f"{name} must hold total_nodes entries")
    mask = (1 << 64) - 1
    _check("tree_uniforms",
           lib.tree_uniforms(int(seed) & mask, int(purpose) & mask, int(step) & mask,
                             _ptr(request_id), _ptr(depth), _ptr(cu_nodes), batch, total,
                             _ptr(u_accept), _ptr(u_resample), _stream(stream)))
    return u_accept, u_resample


class VerifyStep:
    """The step's buffers bound once: run() enqueues tree_verify_step (index, attention,
    acceptance); capture() returns a VerifyGraph that replays the same three calls on
    the same buffers (refresh inputs in place between replays).  Outputs: anc, depth,
    out, lse (if want_lse), accept (dict as tree_accept returns), err."""

    def __init__(self, q, k_cache, v_cache, block_table, prefix_len, k_tree, v_tree, parent,
                 cu_nodes, p_target, p_draft, token, u_accept, u_resample, *, max_nodes: int,
                 max_prefix: int, max_path: int, scale: float | None = None, p_own=None,
                 own_row=None, want_lse: bool = False):
        lib = load()
        fdt = (torch.float32, torch.bfloat16)
        _need(q, "q", fdt, 3)
        for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
            _need(t, name, q.dtype, 4)
        for name, t in (("k_tree", k_tree), ("v_tree", v_tree)):
            _need(t, name, q.dtype, 3)
        for name, t in (("block_table", block_table),):
            _need(t, name, torch.int32, 2)
        for name, t in (("prefix_len", prefix_len), ("parent", parent), ("cu_nodes", cu_nodes),
                        ("token", token)):
            _need(t, name, torch.int32, 1)
        for name, t in (("p_target", p_target), ("p_draft", p_draft)):
            _need(t, name, torch.float32, 2)
        for name, t in (("u_accept", u_accept), ("u_resample", u_resample)):
            _need(t, name, torch.float32, 1)
        if (p_own is None) != (own_row is None):
            raise ValueError("p_own and own_row go together")
        total, hq, d = q.shape
        num_blocks, hkv, blk, d2 = k_cache.shape
        if blk != TV_BLOCK or d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
            raise ValueError("k_cache/v_cache must be [num_blocks, hkv, 64, head_dim]")
        if tuple(k_tree.shape) != (total, hkv, d) or tuple(v_tree.shape) != (total, hkv, d):
            raise ValueError("k_tree/v_tree must be [total_nodes, hkv, head_dim]")
        batch = cu_nodes.numel() - 1
        vocab = p_target.shape[1]
        if tuple(p_target.shape) != (total, vocab) or tuple(p_draft.shape) != (total, vocab):
            raise ValueError("p_target/p_draft must be [total_nodes, vocab]")
        if block_table.shape[0] != batch or prefix_len.numel() != batch:
            raise ValueError("block_table / prefix_len must have one row per sequence")
        for t in (parent, token, u_accept, u_resample):
            if t.numel() != total:
                raise ValueError("parent, token, u_accept and u_resample need one entry per node")
        own_rows = 0
        if p_own is not None:
            _need(p_own, "p_own", torch.float32, 2)
            _need(own_row, "own_row", torch.int32, 1)
            if p_own.shape[1] != vocab or own_row.numel() != total:
                raise ValueError("p_own must be [rows, vocab] and own_row [total_nodes]")
            own_rows = p_own.shape[0]
        dev, dt = q.device, dtype_code(q.dtype)
        words = (max_nodes + 63) // 64
        self.anc = torch.empty((total, words), dtype=torch.int64, device=dev)
        self.depth = torch.empty(total, dtype=torch.int32, device=dev)
        self.out = torch.empty_like(q)
        self.lse = torch.empty((total, hq), dtype=torch.float32, device=dev) if want_lse else None
        self.accept = dict(accept_len=torch.empty(batch, dtype=torch.int32, device=dev),
                           path=torch.empty((batch, max_path), dtype=torch.int32, device=dev),
                           resample_node=torch.empty(batch, dtype=torch.int32, device=dev),
                           resample_token=torch.empty(batch, dtype=torch.int32, device=dev),
                           node_ok=torch.empty(total, dtype=torch.uint8, device=dev))
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.accept["err"] = self.err
        need_a = tree_verify_attention_workspace_size(batch, total, max_nodes, max_prefix, hq, hkv, d, dt)
        self.attn_ws = torch.zeros(max(need_a, 1), dtype=torch.uint8, device=dev)  # kept zero
        need_c = tree_accept_workspace_size(batch, vocab)
        self.accept_ws = torch.zeros(max(need_c, 1), dtype=torch.uint8, device=dev)  # kept zero
        # every tensor the struct points at stays referenced by this object
        self._keep = (q, k_cache, v_cache, block_table, prefix_len, k_tree, v_tree, parent,
                      cu_nodes, p_target, p_draft, token, u_accept, u_resample, p_own, own_row)
        a = StepArgs()
        p = lambda t: None if t is None else t.data_ptr()
        a.parent, a.cu_nodes, a.batch, a.total_nodes = p(parent), p(cu_nodes), batch, total
        a.max_nodes, a.words, a.prefix_len = max_nodes, words, p(prefix_len)
        a.anc_bits, a.depth, a.pos = p(self.anc), p(self.depth), None
        a.q, a.k_cache, a.v_cache, a.block_table = p(q), p(k_cache), p(v_cache), p(block_table)
        a.num_blocks, a.max_blocks, a.max_prefix = num_blocks, block_table.shape[1], max_prefix
        a.hq, a.hkv, a.head_dim, a.dtype = hq, hkv, d, dt
        a.softmax_scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        a.k_tree, a.v_tree, a.out, a.lse = p(k_tree), p(v_tree), p(self.out), p(self.lse)
        a.attn_workspace, a.attn_workspace_bytes = p(self.attn_ws), self.attn_ws.numel()
        a.p_target, a.p_draft, a.token = p(p_target), p(p_draft), p(token)
        a.u_accept, a.u_resample, a.p_own, a.own_row = p(u_accept), p(u_resample), p(p_own), p(own_row)
        a.own_rows, a.vocab, a.max_path, a.reserved = own_rows, vocab, max_path, 0
        o = self.accept
        a.accept_len, a.path = p(o["accept_len"]), p(o["path"])
        a.resample_node, a.resample_token, a.node_ok = (p(o["resample_node"]), p(o["resample_token"]),
                                                        p(o["node_ok"]))
        a.accept_workspace, a.accept_workspace_bytes = p(self.accept_ws), self.accept_ws.numel()
        a.err = p(self.err)
        self.args = a
        self._lib = lib

    def run(self, stream=None) -> None:
        _check("tree_verify_step", self._lib.tree_verify_step(ctypes.byref(self.args), _stream(stream)))

    def capture(self, stream=None) -> "VerifyGraph":
        return VerifyGraph(self, stream)


class VerifyGraph:
    """A HIP graph of one VerifyStep's three calls (tree_verify_graph_*)."""

    def __init__(self, step: VerifyStep, stream=None):
        self._lib, self.step = step._lib, step
        h = ctypes.c_void_p()
        s = ctypes.c_void_p(None) if stream is None else _stream(stream)
        _check("tree_verify_graph_create",
               self._lib.tree_verify_graph_create(ctypes.byref(step.args), s, ctypes.byref(h)))
        self._h = h

    def launch(self, stream=None) -> None:
        if self._h is None:
            raise RuntimeError("graph already destroyed")
        _check("tree_verify_graph_launch", self._lib.tree_verify_graph_launch(self._h, _stream(stream)))

    def close(self) -> None:
        if self._h is not None:
            _check("tree_verify_graph_destroy", self._lib.tree_verify_graph_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tree_quantize_rows_e4m3(x, *, codes=None, exps=None, stream=None):
    """Rows of 128 elements (x [..., 128], bf16 or float32) to E4M3 codes with one
    power-of-two scale per row.  Returns (codes [..., 128] uint8, exps [...] uint8:
    value = e4m3(code) * 2^(exps - 127))."""
    lib = load()
    _need(x, "x", (torch.float32, torch.bfloat16))
    if x.shape[-1] != 128:
        raise ValueError("rows must hold 128 elements")
    rows = x.numel() // 128
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if exps is None:
        exps = torch.empty(x.shape[:-1], dtype=torch.uint8, device=x.device)
    _need(codes, "codes", torch.uint8)
    _need(exps, "exps", torch.uint8)
    if codes.numel() != x.numel() or exps.numel() != rows:
        raise ValueError("codes must match x and exps hold one byte per row")
    _check("tree_quantize_rows_e4m3",
           lib.tree_quantize_rows_e4m3(_ptr(x), dtype_code(x.dtype), rows, _ptr(codes), _ptr(exps),
                                       _stream(stream)))
    return codes, exps


def tree_verify_attention_fp8_workspace_size(batch, total_nodes, max_nodes, max_prefix, hq,
                                             hkv) -> int:
    return int(load().tree_verify_attention_fp8_workspace_size(batch, total_nodes, max_nodes,
                                                               max_prefix, hq, hkv))


def tree_verify_attention_fp8(q, k_cache, v_cache, k_exp, v_exp, block_table, prefix_len, k_tree,
                              v_tree, kt_exp, vt_exp, cu_nodes, anc, max_nodes: int,
                              max_prefix: int, scale: float | None = None, *, out=None, lse=None,
                              want_lse: bool = True, workspace=None, err=None, stream=None):
    """Tree attention on the FP8 matrix cores: q bf16 (quantized per row inside);
    k_cache/v_cache [num_blocks, hkv, 64, 128] and k_tree/v_tree [total, hkv, 128] uint8
    E4M3 with k_exp/v_exp [num_blocks, hkv, 64] and kt_exp/vt_exp [total, hkv] uint8 E8M0
    row exponents (tree_quantize_rows_e4m3 writes this format).  Returns (out, lse, err)."""
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, name, torch.uint8, 4)
    for name, t in (("k_exp", k_exp), ("v_exp", v_exp), ("k_tree", k_tree), ("v_tree", v_tree)):
        _need(t, name, torch.uint8, 3)
    for name, t in (("kt_exp", kt_exp), ("vt_exp", vt_exp)):
        _need(t, name, torch.uint8, 2)
    _need(block_table, "block_table", torch.int32, 2)
    _need(prefix_len, "prefix_len", torch.int32, 1)
    _need(cu_nodes, "cu_nodes", torch.int32, 1)
    _need(anc, "anc", torch.int64, 2)
    total, hq, d = q.shape
    num_blocks, hkv, blk, d2 = k_cache.shape
    if d != 128 or blk != TV_BLOCK or d2 != 128 or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [num_blocks, hkv, 64, 128] and head_dim 128")
    if tuple(k_exp.shape) != (num_blocks, hkv, TV_BLOCK) or tuple(v_exp.shape) != tuple(k_exp.shape):
        raise ValueError("k_exp/v_exp must be [num_blocks, hkv, 64]")
    if tuple(k_tree.shape) != (total, hkv, d) or tuple(v_tree.shape) != (total, hkv, d):
        raise ValueError("k_tree/v_tree must be [total_nodes, hkv, 128]")
    if tuple(kt_exp.shape) != (total, hkv) or tuple(vt_exp.shape) != (total, hkv):
        raise ValueError("kt_exp/vt_exp must be [total_nodes, hkv]")
    batch = cu_nodes.numel() - 1
    if block_table.shape[0] != batch or prefix_len.numel() != batch or anc.shape[0] != total:
        raise ValueError("block_table / prefix_len per sequence, anc per node")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((total, hq), dtype=torch.float32, device=q.device)
    need = tree_verify_attention_fp8_workspace_size(batch, total, max_nodes, max_prefix, hq, hkv)
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    err = _err_word(err, q.device)
    _check("tree_verify_attention_fp8",
           lib.tree_verify_attention_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_exp),
                                         _ptr(v_exp), num_blocks, _ptr(block_table),
                                         block_table.shape[1], _ptr(prefix_len), _ptr(k_tree),
                                         _ptr(v_tree), _ptr(kt_exp), _ptr(vt_exp), _ptr(cu_nodes),
                                         _ptr(anc), anc.shape[1], batch, total, max_nodes,
                                         max_prefix, hq, hkv, scale, _ptr(out), _ptr(lse),
                                         _ptr(workspace), ws_bytes, _ptr(err), _stream(stream)))
    return out, lse, err
