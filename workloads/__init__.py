"""Seeded synthetic inputs for the tree-verification step.

This module only draws inputs: tree topologies, Q/K/V tensors, paged block
tables, probability rows, drafted tokens and uniforms.  It holds none of the
verification arithmetic (no attention, no ancestor sets, no acceptance), so
the oracle and the GPU path can both read its output without sharing any of
the method's code.

Every array is a numpy array; bf16 tensors are carried as their raw uint16
bit patterns (round-to-nearest-even from an fp32 draw), so that both sides
see exactly the same bits.

Layouts (what the C-ABI library expects):
  q        [sum_nodes, hq, d]            fp32 or bf16 bits
  k_cache  [num_blocks, hkv, 64, d]      paged prefix keys (64-token blocks)
  v_cache  [num_blocks, hkv, 64, d]
  block_table [batch, max_blocks] int32  physical block of logical block j, -1 unused
  prefix_len  [batch] int32
  k_tree / v_tree [sum_nodes, hkv, d]    keys/values of the draft-tree nodes
  cu_nodes [batch + 1] int32             flattened node offsets per sequence
  parent   [sum_nodes] int32             local parent index, -1 = hangs off the prefix
  p_target / p_draft [sum_nodes, vocab] fp32
  token    [sum_nodes] int32             drafted token of each node (drawn from p_draft)
  u_accept / u_resample [sum_nodes] fp32 uniforms m * 2^-24, m in [0, 2^24)
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK = 64  # tokens per paged KV block
DT_F32 = 0
DT_BF16 = 1


# --------------------------------------------------------------------------
# bf16 bit helpers (input preparation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    """Exact upcast of stored tensor values to fp64."""
    if dtype == DT_BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.default_rng([int(seed)] + [int(t) for t in tags])


# --------------------------------------------------------------------------
# tree topologies (parent arrays, parent[i] < i, -1 = under the prefix)
# --------------------------------------------------------------------------
def level_order(parent: list[int] | np.ndarray) -> np.ndarray:
    """Relabel a parent array so nodes are in level (BFS) order.

    Children keep the relative order of their original indices; parents stay
    before children.  Returns the relabelled parent array.
    """
    parent = [int(p) for p in parent]
    n = len(parent)
    children: dict[int, list[int]] = {}
    for i, p in enumerate(parent):
        children.setdefault(p, []).append(i)
    order: list[int] = []
    frontier = children.get(-1, [])
    while frontier:
        order.extend(frontier)
        nxt: list[int] = []
        for v in frontier:
            nxt.extend(children.get(v, []))
        frontier = nxt
    if len(order) != n:
        raise ValueError("parent array is not a forest rooted at -1")
    new_of = {old: new for new, old in enumerate(order)}
    out = np.empty(n, dtype=np.int32)
    for new, old in enumerate(order):
        p = parent[old]
        out[new] = -1 if p < 0 else new_of[p]
    return out


def tree_heap(n: int) -> np.ndarray:
    """Full binary tree in heap order: node i hangs off node (i-1)//2."""
    return np.array([-1] + [(i - 1) // 2 for i in range(1, n)], dtype=np.int32)


def tree_chain(n: int) -> np.ndarray:
    return np.arange(-1, n - 1, dtype=np.int32)


def tree_star(n: int) -> np.ndarray:
    """n nodes all hanging directly off the prefix (n roots)."""
    return np.full(n, -1, dtype=np.int32)


def tree_kary_levels(k: int, levels: int) -> np.ndarray:
    """Full k-ary forest with k roots under the prefix and `levels` levels."""
    parent: list[int] = []
    prev = [-1]
    for _ in range(levels):
        cur = []
        for p in prev:
            for _ in range(k):
                parent.append(p)
                cur.append(len(parent) - 1)
        prev = cur
    return np.array(parent, dtype=np.int32)


def tree_branch_then_chains(branch: int, branch_levels: int, depth: int, n_total: int) -> np.ndarray:
    """`branch`-ary forest for `branch_levels` levels, then top-1 chains.

    Under the deepest branching nodes, in index order, a chain runs down to
    `depth` levels, until `n_total` nodes exist (the last chain may be short).
    Relabelled to level order.
    """
    parent = list(tree_kary_levels(branch, branch_levels))
    last_level = [i for i in range(len(parent)) if _depth_of(parent, i) == branch_levels]
    chain_len = depth - branch_levels
    for leaf in last_level:
        p = leaf
        for _ in range(chain_len):
            if len(parent) >= n_total:
                break
            parent.append(p)
            p = len(parent) - 1
        if len(parent) >= n_total:
            break
    if len(parent) != n_total:
        raise ValueError("not enough room for the requested node count")
    return level_order(parent)


def _depth_of(parent, i) -> int:
    d = 0
    while i >= 0:
        d += 1
        i = parent[i]
    return d


def tree_random(rng: np.random.Generator, n: int, max_depth: int) -> np.ndarray:
    """Random forest: parent_i uniform over {-1} and earlier nodes of depth < max_depth."""
    parent: list[int] = []
    depth: list[int] = []
    for i in range(n):
        cands = [-1] + [j for j in range(i) if depth[j] < max_depth]
        p = cands[int(rng.integers(0, len(cands)))]
        parent.append(p)
        depth.append(1 if p < 0 else depth[p] + 1)
    return level_order(parent)


def tree_importance_sampled(rng: np.random.Generator, n: int, top_k: int, beta: float,
                            max_depth: int, vocab: int, sigma2: float = 2.0) -> np.ndarray:
    """Draft tree grown by importance sampling over synthetic top-K draft probs.

    Each expanded node draws draft logits ~ N(0, sigma2) over `vocab`, keeps
    its top-K probabilities p and gives its K candidate children the weights
    w = p^beta / sum(p^beta).  A candidate's path weight is the product of the
    weights along its path.  Candidates are taken one at a time, with
    probability proportional to path weight and without replacement, until
    `n` nodes exist; a taken candidate of depth < max_depth adds its own K
    candidates.  Output is in level order.
    """
    sd = math.sqrt(sigma2)

    def child_weights() -> np.ndarray:
        logits = rng.standard_normal(vocab) * sd
        top = np.sort(logits)[-top_k:][::-1]
        p = np.exp(top - logits.max())
        p = p / np.exp(logits - logits.max()).sum()
        w = p ** beta
        return w / w.sum()

    parent: list[int] = []
    # frontier entries: (path_weight, parent_node, depth)
    frontier: list[tuple[float, int, int]] = [(float(w), -1, 1) for w in child_weights()]
    while len(parent) < n and frontier:
        ws = np.array([f[0] for f in frontier])
        j = int(rng.choice(len(frontier), p=ws / ws.sum()))
        pw, p, d = frontier.pop(j)
        parent.append(p)
        me = len(parent) - 1
        if d < max_depth:
            frontier.extend((pw * float(w), me, d + 1) for w in child_weights())
    return level_order(parent)


# --------------------------------------------------------------------------
# probability rows, drafted tokens, uniforms
# --------------------------------------------------------------------------
def _softmax_rows(rng: np.random.Generator, rows: int, vocab: int, sigma2: float) -> np.ndarray:
    x = rng.standard_normal((rows, vocab), dtype=np.float32)
    x *= np.float32(math.sqrt(sigma2))
    x -= x.max(axis=1, keepdims=True)
    np.exp(x, out=x)
    s = x.sum(axis=1, dtype=np.float64, keepdims=True)
    return (x / s).astype(np.float32)


def prob_rows(seed: int, tag: int, rows: int, vocab: int, sigma2: float = 2.0,
              chunk: int = 64, threads: int = 8) -> np.ndarray:
    """[rows, vocab] fp32 rows, each the softmax of N(0, sigma2) logits.

    Row chunk c is drawn from its own seeded stream, so the result does not
    depend on the thread count.
    """
    out = np.empty((rows, vocab), dtype=np.float32)
    starts = list(range(0, rows, chunk))

    def work(c0: int) -> None:
        c1 = min(rows, c0 + chunk)
        out[c0:c1] = _softmax_rows(_rng(seed, 7001, tag, c0), c1 - c0, vocab, sigma2)

    if rows * vocab > 4_000_000 and threads > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, starts))
    else:
        for c0 in starts:
            work(c0)
    return out


def sample_tokens(seed: int, p: np.ndarray, chunk: int = 64) -> np.ndarray:
    """Draw one token per row from the row's distribution (inverse CDF)."""
    rows = p.shape[0]
    tok = np.empty(rows, dtype=np.int32)
    rng = _rng(seed, 7101)
    u = rng.random(rows)
    for c0 in range(0, rows, chunk):
        c1 = min(rows, c0 + chunk)
        cdf = np.cumsum(p[c0:c1], axis=1, dtype=np.float64)
        thr = u[c0:c1, None] * cdf[:, -1:]
        t = (cdf <= thr).sum(axis=1)
        tok[c0:c1] = np.minimum(t, p.shape[1] - 1)
    return tok


def draft_rows(rng: np.random.Generator, batch: int, rows: int, k: int, vocab: int = 32000,
               sigma2: float = 2.0) -> np.ndarray:
    """Synthetic draft-model top-K rows: the K largest probabilities, in descending
    order, of softmax(N(0, sigma2) logits over `vocab`) (softmax in fp64, then fp32).
    Returns [batch, rows, k] float32."""
    out = np.empty((batch, rows, k), np.float32)
    sd = math.sqrt(sigma2)
    for b in range(batch):
        for r in range(rows):
            x = rng.standard_normal(vocab) * sd
            e = np.exp(x - x.max())
            out[b, r] = (np.sort(e)[::-1][:k] / e.sum()).astype(np.float32)
    return out


def grid_uniforms(rng: np.random.Generator, n: int) -> np.ndarray:
    """Uniforms on the 2^-24 grid: exactly representable, in [0, 1)."""
    m = rng.integers(0, 1 << 24, size=n, dtype=np.int64)
    return (m.astype(np.float64) * 2.0 ** -24).astype(np.float32)


# --------------------------------------------------------------------------
# a full verify-step input set
# --------------------------------------------------------------------------
@dataclass
class Case:
    name: str
    batch: int
    hq: int
    hkv: int
    d: int
    dtype: int
    vocab: int
    prefix_len: np.ndarray
    cu_nodes: np.ndarray
    parent: np.ndarray
    block_table: np.ndarray
    num_blocks: int
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    k_tree: np.ndarray
    v_tree: np.ndarray
    p_target: np.ndarray | None = None
    p_draft: np.ndarray | None = None
    token: np.ndarray | None = None
    u_accept: np.ndarray | None = None
    u_resample: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def total_nodes(self) -> int:
        return int(self.cu_nodes[-1])

    @property
    def max_nodes(self) -> int:
        return int(np.diff(self.cu_nodes).max()) if self.batch else 0

    @property
    def max_prefix(self) -> int:
        return int(self.prefix_len.max()) if self.batch else 0

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def local_parent(self, b: int) -> np.ndarray:
        return self.parent[self.cu_nodes[b]:self.cu_nodes[b + 1]]


def _normal_tensor(rng: np.random.Generator, shape, dtype: int) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == DT_BF16 else x


def make_case(name: str, parents: list[np.ndarray], prefix_lens: list[int], hq: int, hkv: int,
              d: int, dtype: int, vocab: int, seed: int, *, alias_prefix: bool = False,
              with_probs: bool = True, spare_blocks: int = 0, sigma2: float = 2.0,
              reserve_tokens: int = 0) -> Case:
    """Draw every input of one verify step for the given trees and prefixes.

    alias_prefix: all sequences' block tables point at the same physical
    blocks (one shared prefix, read through every sequence's table).
    reserve_tokens: each sequence's table also maps the blocks of this many
    positions past its prefix (fresh blocks of the pool, room for a commit).
    """
    assert not (alias_prefix and reserve_tokens), "a shared prefix has no private room"
    batch = len(parents)
    assert len(prefix_lens) == batch
    cu = np.zeros(batch + 1, dtype=np.int32)
    for b, p in enumerate(parents):
        cu[b + 1] = cu[b] + len(p)
    total = int(cu[-1])
    parent = np.concatenate([np.asarray(p, dtype=np.int32) for p in parents]) if total else np.zeros(0, np.int32)
    plen = np.asarray(prefix_lens, dtype=np.int32)
    nblk = [(int(p) + reserve_tokens + BLOCK - 1) // BLOCK for p in plen]
    max_blocks = max([1] + nblk)
    rng_layout = _rng(seed, 11)
    if alias_prefix:
        num_blocks = max([0] + nblk) + spare_blocks
        perm = rng_layout.permutation(num_blocks).astype(np.int32)
        bt = np.full((batch, max_blocks), -1, dtype=np.int32)
        for b in range(batch):
            bt[b, :nblk[b]] = perm[:nblk[b]]
    else:
        num_blocks = sum(nblk) + spare_blocks
        perm = rng_layout.permutation(num_blocks).astype(np.int32)
        bt = np.full((batch, max_blocks), -1, dtype=np.int32)
        o = 0
        for b in range(batch):
            bt[b, :nblk[b]] = perm[o:o + nblk[b]]
            o += nblk[b]
    num_blocks = max(num_blocks, 1)
    q = _normal_tensor(_rng(seed, 21), (total, hq, d), dtype)
    kc = _normal_tensor(_rng(seed, 22), (num_blocks, hkv, BLOCK, d), dtype)
    vc = _normal_tensor(_rng(seed, 23), (num_blocks, hkv, BLOCK, d), dtype)
    kt = _normal_tensor(_rng(seed, 24), (total, hkv, d), dtype)
    vt = _normal_tensor(_rng(seed, 25), (total, hkv, d), dtype)
    case = Case(name=name, batch=batch, hq=hq, hkv=hkv, d=d, dtype=dtype, vocab=vocab,
                prefix_len=plen, cu_nodes=cu, parent=parent, block_table=bt,
                num_blocks=num_blocks, q=q, k_cache=kc, v_cache=vc, k_tree=kt, v_tree=vt)
    if with_probs:
        add_probs(case, seed, sigma2=sigma2)
    return case


def fp8_cache(cache: np.ndarray, dtype: int):
    """An E4M3 copy of a K/V cache [num_blocks, hkv, 64, d] with one fp32 scale per
    (block, head, position) row: scale = max|row| / 448 (1 for an all-zero row);
    the bytes are torch's float8_e4m3fn cast of the row / scale, clamped to +-448.
    Returns (codes uint8, scale float32 [num_blocks, hkv, 64])."""
    import torch
    x = to_f64(cache, dtype).astype(np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = np.clip(x / scale[..., None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scale


def fp8_random_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform E4M3 bytes over every finite code (0x7F and 0xFF, the NaNs, excluded)."""
    c = rng.integers(0, 254, size=shape, dtype=np.int32)
    c = c + (c >= 0x7F)  # skip 0x7F; 253 -> 254 stays below 0xFF
    return c.astype(np.uint8)


def add_probs(case: Case, seed: int, sigma2: float = 2.0) -> None:
    total, vocab = case.total_nodes, case.vocab
    case.p_target = prob_rows(seed, 1, total, vocab, sigma2)
    case.p_draft = prob_rows(seed, 2, total, vocab, sigma2)
    case.token = sample_tokens(seed, case.p_draft) if total else np.zeros(0, np.int32)
    rng = _rng(seed, 31)
    case.u_accept = grid_uniforms(rng, total)
    case.u_resample = grid_uniforms(rng, total)


# --------------------------------------------------------------------------
# the five verify workloads
# --------------------------------------------------------------------------
CONFIG_NAMES = [
    "tiny-fp32: B1 P128 binary-tree-15 H4 D64 fp32 V1000",
    "llava7b-like: B1 P1088 importance-tree-64 MHA32 D128 bf16 V32000",
    "wide-8ary-d3: B8 P4096 tree-584 GQA32/8 D128 bf16 V152064",
    "serving-64: B64 P~U[512,4096] trees 16-96 GQA32/8 D128 bf16 V128256",
    "long-32k: B4 P32768 tree-256 GQA64/8 D128 bf16 V128256",
]


def config_trees(index: int, seed: int):
    """(parents, prefix_lens, hq, hkv, d, dtype, vocab, alias) for workload `index` (0-based)."""
    if index == 0:
        return [tree_heap(15)], [128], 4, 4, 64, DT_F32, 1000, False
    if index == 1:
        t = tree_importance_sampled(_rng(seed, 41), 64, 8, 0.7, 6, 32000)
        return [t], [576 + 512], 32, 32, 128, DT_BF16, 32000, False
    if index == 2:
        t = tree_kary_levels(8, 3)
        return [t] * 8, [4096] * 8, 32, 8, 128, DT_BF16, 152064, False
    if index == 3:
        rng = _rng(seed, 43)
        parents, plens = [], []
        for _ in range(64):
            n = int(rng.integers(16, 97))
            plens.append(int(rng.integers(512, 4097)))
            parents.append(tree_random(rng, n, 8))
        return parents, plens, 32, 8, 128, DT_BF16, 128256, False
    if index == 4:
        t = tree_branch_then_chains(4, 3, 10, 256)
        return [t] * 4, [32768] * 4, 64, 8, 128, DT_BF16, 128256, False
    raise ValueError(index)


def make_config(index: int, seed: int = 1234, with_probs: bool = True) -> Case:
    parents, plens, hq, hkv, d, dt, vocab, alias = config_trees(index, seed)
    return make_case(CONFIG_NAMES[index], parents, plens, hq, hkv, d, dt, vocab, seed,
                     alias_prefix=alias, with_probs=with_probs)


# --------------------------------------------------------------------------
# device upload (torch); the same bytes as the numpy arrays above
# --------------------------------------------------------------------------
def to_torch(a: np.ndarray, dtype: int | None = None, device="cuda"):
    """numpy -> torch tensor on `device`; bf16 bit arrays become torch.bfloat16."""
    import torch
    if dtype == DT_BF16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def case_to_device(case: Case, device="cuda", probs: bool = True) -> dict:
    """Every input of a Case as device tensors, keyed by argument name."""
    dt = case.dtype
    out = dict(
        q=to_torch(case.q, dt, device), k_cache=to_torch(case.k_cache, dt, device),
        v_cache=to_torch(case.v_cache, dt, device), k_tree=to_torch(case.k_tree, dt, device),
        v_tree=to_torch(case.v_tree, dt, device), block_table=to_torch(case.block_table, None, device),
        prefix_len=to_torch(case.prefix_len, None, device), cu_nodes=to_torch(case.cu_nodes, None, device),
        parent=to_torch(case.parent, None, device))
    if probs and case.p_target is not None:
        out.update(p_target=to_torch(case.p_target, None, device),
                   p_draft=to_torch(case.p_draft, None, device),
                   token=to_torch(case.token, None, device),
                   u_accept=to_torch(case.u_accept, None, device),
                   u_resample=to_torch(case.u_resample, None, device))
    return out
