"""Verify-step benchmark on one MI355X.

One step = one pass of the whole verify path over one batch of synthetic,
HBM-resident input: tree_build_index + tree_verify_attention (one attention
layer) + tree_accept.  The step is captured once in a HIP graph and replayed
(launch overhead is what graph capture removes from a verify step); the eager
rate is reported beside it.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config I] [--only]

--config selects the headline workload (0..4, default 4: long-context verify,
batch 4, prefix 32768, 256-node trees, 64 query / 8 KV heads, head_dim 128,
bf16, vocab 128256 -- the largest workload that fits one GPU).  The other four
workloads are measured after it, each with its step time, attention time,
roofline and CPU baseline, under "other_workloads" (--only skips them).

`roofline` is for the attention call (the dominant kernel): algorithmic bytes
(unique prefix K+V, tree K+V, Q, out) or flops (4*D*Hq*sum over nodes of the
visible keys) per launch divided by its average duration, timed with events on
the launch stream over back-to-back graph-replayed launches.  `cpu_baseline`
is the CPU oracle (fp64 numpy + Python) timed on this host on a bounded
sample of the same workload (whole steps, or the first sequences of one).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 matrix
MFMA_FP8_PEAK_TFS = 5000.0     # MI355X dense fp8 matrix
VALU_FP32_PEAK_TFS = 157.3     # MI355X fp32 vector


def node_depths(parent: np.ndarray) -> np.ndarray:
    """Depth of each node of one tree (1 under the prefix); parents precede children."""
    dep = np.zeros(len(parent), dtype=np.int64)
    for i, p in enumerate(parent):
        dep[i] = 1 if p < 0 else dep[p] + 1
    return dep


def attention_cost(case):
    """Algorithmic bytes and flops of one tree-attention launch."""
    esz = 2 if case.dtype == 1 else 4
    d, hq, hkv = case.d, case.hq, case.hkv
    total = case.total_nodes
    prefix_tokens = int(case.prefix_len.sum())
    if case.batch > 1 and np.all(case.block_table == case.block_table[:1]):
        prefix_tokens = int(case.prefix_len.max())  # one physical prefix read through every table
    bytes_ = (prefix_tokens * hkv * d * 2 + total * hkv * d * 2 + 2 * total * hq * d) * esz
    visible = 0
    for b in range(case.batch):
        dep = node_depths(case.local_parent(b))
        visible += int(case.prefix_len[b]) * len(dep) + int(dep.sum())
    flops = 4.0 * d * hq * visible
    return bytes_, flops


ATTN_SOURCES = ("attn_mfma.hip", "attn_mfma_long.hip", "mfma_tile.h", "attn_vec.hip",
                "attention.hip", "attn.h")
COPY_BYTES = 512 << 20  # calibration kernel: reads 512 MiB and writes 512 MiB


def attention_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, "tree_attention_verification_04_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(config: int) -> str:
    return os.path.join(ROOT, "profiles", f"attention_traffic_workload{config}.txt")


def recorded_traffic(config: int):
    """HBM bytes per attention launch from the committed counter summary, if the
    kernel sources still match the ones the counters were taken with."""
    try:
        kv = dict(line.split("=", 1) for line in open(traffic_path(config)).read().split("\n")
                  if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    if kv.get("source_hash", "").strip() != attention_source_hash():
        return None
    return int(kv["hbm_bytes_per_launch"])


def measured_copy_gbps(torch) -> float:
    """Device-to-device copy rate (bytes read + written per second) of 1 GiB, the
    best of 5 copies timed with events: the attainable HBM rate beside the published
    peak (context for the roofline fraction, which stays against the peak)."""
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best = float("inf")
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        best = min(best, a.elapsed_time(b))
    del src, dst
    return round(2 * n * 4 / (best * 1e-3) / 1e9, 1)


def summarize_pmc(config: int, fetch_csv: str, write_csv: str, command: str) -> None:
    """Turn FETCH_SIZE / WRITE_SIZE passes into bytes per attention launch.

    Each counter (KiB per dispatch) is scaled by what it reads for a plain
    elementwise kernel that reads and writes COPY_BYTES (torch.add, same run)."""
    import csv

    def per_kernel(path):
        vals = {}
        for row in csv.DictReader(open(path)):
            vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return vals

    def pick(vals, key):
        rows = [v for k, v in vals.items() if key in k]
        return sum(rows[0]) / len(rows[0]) if rows else None

    f, w = per_kernel(fetch_csv), per_kernel(write_csv)
    copy_f = max((sum(v) / len(v) for k, v in f.items() if "add" in k.lower() and "elementwise" in k), default=None)
    copy_w = max((sum(v) / len(v) for k, v in w.items() if "add" in k.lower() and "elementwise" in k), default=None)
    sf = COPY_BYTES / (copy_f * 1024.0)
    sw = COPY_BYTES / (copy_w * 1024.0)
    # one tree_verify_attention launch: its main kernel plus the split merge, the
    # pair-order kernel and the ticket clear when the plan uses them
    # (the bf16 instances: the FP8 variants' instances carry mode 1 or 2)
    main_keys = ("k_attn_long<false, 0>", "k_attn_long<true, 0>", "k_attn_mfma", "k_attn_vec")
    attn_f = next((v for v in (pick(f, k) for k in main_keys) if v is not None), 0.0)
    attn_w = next((v for v in (pick(w, k) for k in main_keys) if v is not None), 0.0)
    aux = ("k_attn_combine", "k_attn_order", "k_clear_words")
    comb_f = sum(pick(f, k) or 0.0 for k in aux)
    comb_w = sum(pick(w, k) or 0.0 for k in aux)
    fetch = (attn_f + comb_f) * 1024.0 * sf
    write = (attn_w + comb_w) * 1024.0 * sw
    with open(traffic_path(config), "w") as fh:
        fh.write(f"# HBM traffic of one tree_verify_attention launch, workload {config}\n")
        fh.write(f"# command: {command}\n")
        fh.write(f"# FETCH_SIZE KiB/dispatch: attention {attn_f:.1f} merge+order {comb_f:.1f} copy {copy_f:.1f}\n")
        fh.write(f"# WRITE_SIZE KiB/dispatch: attention {attn_w:.1f} merge+order {comb_w:.1f} copy {copy_w:.1f}\n")
        fh.write(f"# scale factors (copy of {COPY_BYTES} B): fetch {sf:.4f} write {sw:.4f}\n")
        fh.write(f"fetch_bytes_per_launch={int(fetch)}\n")
        fh.write(f"write_bytes_per_launch={int(write)}\n")
        fh.write(f"hbm_bytes_per_launch={int(fetch + write)}\n")
        fh.write(f"source_hash={attention_source_hash()}\n")
    print(open(traffic_path(config)).read())


def summarize_trace(config: int, db_path: str, command: str) -> None:
    """Kernel-trace statistics (calls, total, average and share of time per kernel)
    from a rocprofv3 results database, written to profiles/ as markdown."""
    import sqlite3
    import workloads as W
    con = sqlite3.connect(db_path)
    rows = con.execute("select name, count(*), sum(end - start), avg(end - start) from kernels "
                       "group by name order by 3 desc").fetchall()
    total = sum(r[2] for r in rows) or 1
    name = W.CONFIG_NAMES[config]
    out = os.path.join(ROOT, "profiles", f"verify_step_{name.split(':')[0]}_kernel_trace.md")
    with open(out, "w") as fh:
        fh.write(f"# Verify step, workload {config} ({name}): kernel trace\n\n")
        fh.write("Command (run from the repository root on one MI355X):\n\n```\n" + command + "\n```\n\n")
        fh.write("Durations in microseconds from the run's results database; the bench times "
                 "the step, the attention call and the acceptance call alone, and beside them the "
                 "FP8-cache variant, draft-tree construction, probability rows and KV commit.\n\n")
        fh.write("| kernel | calls | total us | average us | % |\n|---|---|---|---|---|\n")
        for n, c, tot, avg in rows:
            fh.write(f"| {n[:140]} | {c} | {tot / 1e3:.1f} | {avg / 1e3:.3f} | {100.0 * tot / total:.1f} |\n")
    print(open(out).read())


def measure_commit(tv, case, dev, acc_out, max_path: int, reps: int) -> dict:
    """tree_commit_kv after this step's acceptance, timed alone (not part of the step).

    The accepted paths of the step are appended to a fresh paged pool whose block
    table reserves reps * max_path positions past each prefix; prefix_len is reset
    before every timed graph replay (outside the timed region).  Algorithmic bytes =
    accepted rows x hkv x head_dim x element size x 2 (K, V) x 2 (read, write)."""
    import torch
    import workloads as W
    elt = 4 if case.dtype == W.DT_F32 else 2
    plen = case.prefix_len.astype(np.int64)
    nblk = (plen + reps * max_path + 63) // 64
    max_blocks = int(nblk.max())
    bt = np.full((case.batch, max_blocks), -1, dtype=np.int32)
    o = 0
    for b in range(case.batch):
        bt[b, :nblk[b]] = np.arange(o, o + nblk[b], dtype=np.int32)
        o += int(nblk[b])
    tdt = dev["k_tree"].dtype
    k_pool = torch.zeros((o, case.hkv, 64, case.d), dtype=tdt, device="cuda")
    v_pool = torch.zeros_like(k_pool)
    bt_d = torch.from_numpy(bt).cuda()
    plen0 = dev["prefix_len"].clone()
    plen_d = plen0.clone()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def commit():
        tv.tree_commit_kv(dev["k_tree"], dev["v_tree"], dev["cu_nodes"], acc_out["accept_len"],
                          acc_out["path"], k_pool, v_pool, bt_d, plen_d, err=err)

    commit()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            commit()
    times = []
    for _ in range(5):
        plen_d.copy_(plen0)
        torch.cuda.synchronize()
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record()
        g.replay()
        e_ev.record()
        torch.cuda.synchronize()
        times.append(s_ev.elapsed_time(e_ev) / reps)
    if int(err.item()) != 0:
        raise SystemExit(f"commit: device error word {int(err.item())}")
    us = float(np.median(times)) * 1e3
    rows = int(acc_out["accept_len"].sum().item())
    bytes_ = rows * case.hkv * case.d * elt * 2 * 2
    gbs = bytes_ / (us * 1e-6) / 1e9
    return dict(us_per_call=round(us, 3), accepted_rows=rows, alg_bytes=bytes_,
                achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(gbs / HBM_PEAK_GBS, 5), bound="hbm",
                note="latency-bound: a few KB to MB per call")


def measure_softmax(tv, case, reps: int) -> dict:
    """tree_softmax_rows for this workload's trees, timed alone (not part of the step).

    Context rows: the prefix end and every node with a child (a node is judged at its
    parent's context); logits ~ N(0, 2) per context row.  Algorithmic bytes = logits
    read once (4 V per context row) + probabilities written (4 V per node)."""
    import torch
    row_of, ctx = [], 0
    for b in range(case.batch):
        par = case.parent[case.cu_nodes[b]:case.cu_nodes[b + 1]]
        m = {-1: ctx}
        ctx += 1
        for p in par:
            if p >= 0 and int(p) not in m:
                m[int(p)] = ctx
                ctx += 1
        row_of += [m[int(p)] for p in par]
    rng = np.random.default_rng(7)
    lg = torch.from_numpy((rng.standard_normal((ctx, case.vocab)) * np.sqrt(2.0)).astype(np.float32)).cuda()
    ro = torch.tensor(row_of, dtype=torch.int32, device="cuda")
    probs = torch.empty((len(row_of), case.vocab), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, int(tv.load().tree_softmax_rows_workspace_size(ctx, case.vocab))),
                     dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    run = lambda: tv.tree_softmax_rows(lg, ro, probs=probs, workspace=ws, err=err)
    run()
    torch.cuda.synchronize()
    n = max(1, min(reps, int(2e9 // max(1, probs.numel() * 4))))  # bound the graph's traffic
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            run()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record()
        g.replay()
        e_ev.record()
        torch.cuda.synchronize()
        times.append(s_ev.elapsed_time(e_ev) / n)
    if int(err.item()) != 0:
        raise SystemExit(f"softmax rows: device error word {int(err.item())}")
    us = float(np.median(times)) * 1e3
    bytes_ = 4 * case.vocab * (ctx + len(row_of))
    gbs = bytes_ / (us * 1e-6) / 1e9
    # the draft's rows over a kept set of 64 tokens per context (tree_softmax_rows_kept):
    # algorithmic bytes = every output row written + its 64 ids and logits read
    keep_max = 64
    keep = torch.from_numpy(np.stack([rng.choice(case.vocab, keep_max, replace=False)
                                      for _ in range(ctx)]).astype(np.int32)).cuda()
    run_k = lambda: tv.tree_softmax_rows_kept(lg, keep, ro, probs=probs, err=err)
    run_k()
    torch.cuda.synchronize()
    us_k = graph_time_us(torch, run_k, n)
    if int(err.item()) != 0:
        raise SystemExit(f"kept rows: device error word {int(err.item())}")
    bytes_k = len(row_of) * (4 * case.vocab + 8 * keep_max)
    gbs_k = bytes_k / (us_k * 1e-6) / 1e9
    kept = dict(us_per_call=round(us_k, 3), keep_max=keep_max, rows=len(row_of), alg_bytes=bytes_k,
                achieved=round(gbs_k, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(gbs_k / HBM_PEAK_GBS, 4), bound="hbm")
    return dict(us_per_call=round(us, 3), context_rows=ctx, rows=len(row_of), vocab=case.vocab,
                alg_bytes=bytes_, achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(gbs / HBM_PEAK_GBS, 4), bound="hbm", kept_rows=kept)


def _graph_us(torch, run, reps: int) -> float:
    run()
    torch.cuda.synchronize()
    return graph_time_us(torch, run, reps)


def fp8_step_time(torch, tv, case, dev, attention_fp8, mn: int, replays: int) -> float:
    """The step with the FP8 matrix-core attention in place of the bf16 one (index,
    attention, acceptance in one captured graph), microseconds per step."""
    anc = torch.empty((case.total_nodes, (mn + 63) // 64), dtype=torch.int64, device="cuda")
    depth = torch.empty(case.total_nodes, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws_acc = torch.zeros(max(tv.tree_accept_workspace_size(case.batch, case.vocab), 1),
                         dtype=torch.uint8, device="cuda")
    outs = {}

    def step():
        tv.tree_build_index(dev["parent"], dev["cu_nodes"], mn, anc=anc, depth=depth, err=err)
        attention_fp8(anc)
        tv.tree_accept(dev["p_target"], dev["p_draft"], dev["token"], dev["u_accept"],
                       dev["u_resample"], dev["parent"], dev["cu_nodes"], mn, 16, outputs=outs,
                       workspace=ws_acc, err=err)

    return _graph_us(torch, step, replays)


def measure_fp8(tv, case, dev, anc, mn: int, bf16_us: float, reps: int) -> dict | None:
    """Both FP8 variants on this workload, each timed alone like the bf16 attention.

    tree_verify_attention_fp8: Q, K and V in E4M3 with power-of-two row scales, scores
    on the FP8 matrix cores.  Its cache and the tree's K/V are quantized by
    tree_quantize_rows_e4m3 before the timed region (the forward pass that writes an
    FP8 cache writes them in that format); q stays bf16 and is quantized inside the
    call.  Algorithmic bytes = the bf16 launch's with every K/V row at 128 + 1 bytes.
    Roof: HBM for the workloads whose bf16 call is HBM-bound, else the matrix cores at
    the peak of its mix (half the flops, Q.K, at the FP8 rate, half, P.V, at the bf16
    rate: 1 / (0.5 / 5000 + 0.5 / 2500) TFLOP/s).

    step_us / step_tokens_per_s: the step with this call in place of the bf16 one.
    tree_verify_attention_fp8kv (E4M3 prefix with fp32 row scales, exact q, tiles
    through registers): its time beside it.  None for a non-bf16 workload."""
    import torch
    import workloads as W
    if case.dtype != W.DT_BF16 or case.d != 128:
        return None
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    # matrix-core variant
    k8, ke = tv.tree_quantize_rows_e4m3(dev["k_cache"])
    v8, ve = tv.tree_quantize_rows_e4m3(dev["v_cache"])
    kt8, kte = tv.tree_quantize_rows_e4m3(dev["k_tree"])
    vt8, vte = tv.tree_quantize_rows_e4m3(dev["v_tree"])
    out = torch.empty_like(dev["q"])
    need = tv.tree_verify_attention_fp8_workspace_size(case.batch, case.total_nodes, mn,
                                                       case.max_prefix, case.hq, case.hkv)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    attention_fp8 = lambda a_bits: tv.tree_verify_attention_fp8(
        dev["q"], k8, v8, ke, ve, dev["block_table"], dev["prefix_len"], kt8, vt8, kte, vte,
        dev["cu_nodes"], a_bits, mn, case.max_prefix, out=out, want_lse=False,
        workspace=ws if need else None, err=err)
    us = _graph_us(torch, lambda: attention_fp8(anc), reps)
    step_us = fp8_step_time(torch, tv, case, dev, attention_fp8, mn, 20)
    # fp32-scale register-path variant
    k8s, ks = W.fp8_cache(case.k_cache, case.dtype)
    v8s, vs = W.fp8_cache(case.v_cache, case.dtype)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    k8s, v8s, ks, vs = t(k8s), t(v8s), t(ks), t(vs)
    need_kv = tv.tree_verify_attention_fp8kv_workspace_size(case.batch, case.total_nodes, mn,
                                                            case.max_prefix, case.hq, case.hkv)
    ws_kv = torch.zeros(max(need_kv, 1), dtype=torch.uint8, device="cuda")
    us_kv = _graph_us(torch, lambda: tv.tree_verify_attention_fp8kv(
        dev["q"], k8s, v8s, ks, vs, dev["block_table"], dev["prefix_len"], dev["k_tree"],
        dev["v_tree"], dev["cu_nodes"], anc, mn, case.max_prefix, out=out, want_lse=False,
        workspace=ws_kv if need_kv else None, err=err), reps)
    if int(err.item()) != 0:
        raise SystemExit(f"fp8 attention: device error word {int(err.item())}")
    bf16_bytes, flops = attention_cost(case)
    prefix_tokens = int(case.prefix_len.sum())
    if case.batch > 1 and np.all(case.block_table == case.block_table[:1]):
        prefix_tokens = int(case.prefix_len.max())
    row_save = 2 * (case.d * 2) - 2 * (case.d + 1)  # K and V rows: bf16 -> E4M3 + exponent
    bytes_ = bf16_bytes - (prefix_tokens + case.total_nodes) * case.hkv * row_save
    gbs = bytes_ / (us * 1e-6) / 1e9
    t_mem = bf16_bytes / (HBM_PEAK_GBS * 1e9)
    t_cmp = flops / (MFMA_BF16_PEAK_TFS * 1e12)
    mix_peak = 1.0 / (0.5 / MFMA_FP8_PEAK_TFS + 0.5 / MFMA_BF16_PEAK_TFS)
    if t_mem >= t_cmp:
        roof = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        ach = flops / (us * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=round(ach, 2), peak=round(mix_peak, 1), unit="TFLOP/s",
                    frac=round(ach / mix_peak, 4), hbm_GBps=round(gbs, 1))
    return dict(us_per_launch=round(us, 3), bf16_us_per_launch=round(bf16_us, 3),
                vs_bf16=round(us / bf16_us, 4), alg_bytes=int(bytes_), **roof,
                step_us=round(step_us, 2),
                step_tokens_per_s=round(case.total_nodes / (step_us * 1e-6), 1),
                kernel="tree_verify_attention_fp8: E4M3 Q.K on the scaled FP8 matrix "
                       "instructions, V converted to bf16 in LDS",
                fp32_scale_variant={"entry": "tree_verify_attention_fp8kv",
                                    "us_per_launch": round(us_kv, 3)})


def measure_draft_tree(tv, case, reps: int) -> dict:
    """tree_draft_build for this workload's batch and tree size (at most 256 nodes),
    top-K 8, beta 0.7, depth <= 6, prune ratio 0.1, on synthetic top-K rows; timed
    alone.  The draws are serial within a sequence: a latency-bound row."""
    import torch
    import workloads as W
    n_max = max(1, min(256, case.max_nodes))
    rng = np.random.default_rng(11)
    probs = torch.from_numpy(W.draft_rows(rng, case.batch, n_max + 1, 8, vocab=4096)).cuda()
    u = torch.from_numpy(np.stack([W.grid_uniforms(rng, n_max) for _ in range(case.batch)])
                         .astype(np.float32)).cuda()
    out = [torch.empty((case.batch, n_max), dtype=torch.int32, device="cuda") for _ in range(2)]
    qd = torch.empty((case.batch, n_max), dtype=torch.float32, device="cuda")
    cnt = torch.empty(case.batch, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    run = lambda: tv.tree_draft_build(probs, u, 6, 0.7, 0.1, parent=out[0], slot=out[1],
                                      q_draft=qd, count=cnt, err=err)
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            run()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record()
        g.replay()
        e_ev.record()
        torch.cuda.synchronize()
        times.append(s_ev.elapsed_time(e_ev) / reps)
    if int(err.item()) != 0:
        raise SystemExit(f"draft tree: device error word {int(err.item())}")
    us = float(np.median(times)) * 1e3
    nodes = int(cnt.sum().item())
    return dict(us_per_call=round(us, 3), batch=case.batch, n_max=n_max, nodes_built=nodes,
                nodes_per_s=round(nodes / (us * 1e-6), 1), bound="latency",
                note="one wavefront per sequence; draws are serial within a sequence")




def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def one_sequence(case, b: int):
    """Sequence b of a case as a batch of one (the paged pool stays shared)."""
    n0, n1 = int(case.cu_nodes[b]), int(case.cu_nodes[b + 1])
    sl = slice(n0, n1)
    return dict(q=case.q[sl], k_tree=case.k_tree[sl], v_tree=case.v_tree[sl],
                block_table=case.block_table[b:b + 1], prefix_len=case.prefix_len[b:b + 1],
                cu_nodes=np.array([0, n1 - n0], dtype=np.int32), parent=case.parent[sl],
                p_target=case.p_target[sl], p_draft=case.p_draft[sl], token=case.token[sl],
                u_accept=case.u_accept[sl], u_resample=case.u_resample[sl])


def cpu_baseline(case, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the workload: whole verify
    steps (index + attention + acceptance) of one sequence at a time, cycling
    through the batch, until about budget_s (at least one sequence)."""
    import oracle
    import workloads as W
    f = lambda a: W.to_f64(a, case.dtype)
    kc, vc = f(case.k_cache), f(case.v_cache)
    seqs, tokens, t0 = 0, 0, time.perf_counter()
    while True:
        s = one_sequence(case, seqs % case.batch)
        n = int(s["cu_nodes"][-1])
        oracle.build_index(s["parent"], s["cu_nodes"], max(1, n), s["prefix_len"])
        oracle.tree_attention(f(s["q"]), kc, vc, s["block_table"], s["prefix_len"], f(s["k_tree"]),
                              f(s["v_tree"]), s["cu_nodes"], s["parent"], case.hq, case.hkv,
                              case.scale)
        oracle.accept(s["p_target"], s["p_draft"], s["token"], s["u_accept"], s["u_resample"],
                      s["parent"], s["cu_nodes"], case.vocab, 16)
        seqs += 1
        tokens += n
        el = time.perf_counter() - t0
        if el >= budget_s or seqs >= 1000:
            break
    whole = seqs // case.batch
    sample = (f"{seqs} sequence-steps ({whole} whole batch steps + {seqs % case.batch} sequences)"
              if case.batch > 1 else f"{seqs} whole verify steps")
    return dict(value=round(tokens / el, 2), unit="tokens/s", cores=blas_threads(),
                host_cpus=os.cpu_count(), kind="oracle",
                sample=f"{sample} of this workload, {tokens} tree tokens in {el:.1f} s: "
                       "index + attention + acceptance per sequence; fp64 numpy (BLAS threads = "
                       "cores) + Python loops")


def measure_uniforms(tv, case, dev, depth, reps: int) -> dict:
    """tree_uniforms over the step's nodes (the counter-based acceptance and resample
    uniforms), timed alone; bytes = 8 per node written."""
    import torch
    req = torch.arange(case.batch, dtype=torch.int64, device="cuda") + 1000
    ua = torch.empty(case.total_nodes, dtype=torch.float32, device="cuda")
    ur = torch.empty_like(ua)

    def fn():
        tv.tree_uniforms(req, depth, dev["cu_nodes"], seed=2026, step=1, u_accept=ua, u_resample=ur)

    fn()
    torch.cuda.synchronize()
    us = graph_time_us(torch, fn, reps)
    return {"us_per_launch": round(us, 3), "nodes": case.total_nodes}


def measure_step_graph(tv, case, dev, replays: int) -> dict:
    """The step through the library's own graph helper (tree_verify_graph_*): the three
    calls captured once, replayed back to back between two events."""
    import torch
    step = tv.VerifyStep(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                         dev["prefix_len"], dev["k_tree"], dev["v_tree"], dev["parent"],
                         dev["cu_nodes"], dev["p_target"], dev["p_draft"], dev["token"],
                         dev["u_accept"], dev["u_resample"], max_nodes=max(1, case.max_nodes),
                         max_prefix=case.max_prefix, max_path=16)
    step.run()
    torch.cuda.synchronize()
    graph = step.capture()
    try:
        stream = torch.cuda.current_stream()
        for _ in range(3):
            graph.launch(stream)
        torch.cuda.synchronize()
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record()
        for _ in range(replays):
            graph.launch(stream)
        e_ev.record()
        torch.cuda.synchronize()
        if int(step.err.item()) != 0:
            raise SystemExit(f"step graph: device error word {int(step.err.item())}")
        us = s_ev.elapsed_time(e_ev) * 1e3 / replays
    finally:
        graph.close()
    return {"us_per_step": round(us, 2), "replays": replays}


def graph_time_us(torch, fn, reps: int, trials: int = 5) -> float:
    """Median over `trials` replays of a graph of `reps` back-to-back calls of fn,
    timed with events on the replay stream; microseconds per call."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(trials):
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record()
        g.replay()
        e_ev.record()
        torch.cuda.synchronize()
        times.append(s_ev.elapsed_time(e_ev) / reps)
    del g
    return float(np.median(times)) * 1e3


def roofline(case, config: int, attn_us: float) -> dict:
    """Bound, achieved rate and fraction of the attention call against its roof."""
    import workloads as W
    bytes_, flops = attention_cost(case)
    if case.dtype == W.DT_F32:
        t_mem, t_cmp = bytes_ / (HBM_PEAK_GBS * 1e9), flops / (VALU_FP32_PEAK_TFS * 1e12)
        cbound, cpeak = "alu", VALU_FP32_PEAK_TFS
    else:
        t_mem, t_cmp = bytes_ / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFS * 1e12)
        cbound, cpeak = "mfma", MFMA_BF16_PEAK_TFS
    gbs = bytes_ / (attn_us * 1e-6) / 1e9
    if t_mem >= t_cmp:
        roof = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        ach = flops / (attn_us * 1e-6) / 1e12
        roof = dict(bound=cbound, achieved=round(ach, 2), peak=cpeak, unit="TFLOP/s",
                    frac=round(ach / cpeak, 4), hbm_GBps=round(gbs, 1))
    traffic = recorded_traffic(config)
    roof["traffic"] = traffic
    roof["traffic_over_alg_bytes"] = round(traffic / bytes_, 3) if traffic else None
    roof.update(kernel="tree_verify_attention", us_per_launch=round(attn_us, 3),
                alg_bytes=int(bytes_), alg_flops=float(flops))
    return roof


def measure_workload(torch, tv, config: int, args, headline: bool) -> dict:
    """Step, attention call and side rows of one workload on the GPU, plus its CPU
    baseline.  The headline workload gets every side row; the others the FP8 variant."""
    import workloads as W
    t_gen = time.perf_counter()
    case = W.make_config(config, args.seed)
    dev = W.case_to_device(case, "cuda:0")
    t_gen = time.perf_counter() - t_gen
    mn = max(1, case.max_nodes)
    words = (mn + 63) // 64
    total, batch = case.total_nodes, case.batch
    dt = tv.dtype_code(dev["q"].dtype)
    max_path = 16
    anc = torch.empty((total, words), dtype=torch.int64, device="cuda")
    depth = torch.empty(total, dtype=torch.int32, device="cuda")
    out = torch.empty_like(dev["q"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws_a = tv.tree_verify_attention_workspace_size(batch, total, mn, case.max_prefix, case.hq,
                                                   case.hkv, case.d, dt)
    ws_attn = torch.zeros(max(ws_a, 1), dtype=torch.uint8, device="cuda")
    ws_acc = torch.zeros(max(tv.tree_accept_workspace_size(batch, case.vocab), 1), dtype=torch.uint8,
                         device="cuda")
    acc_out = dict(accept_len=torch.empty(batch, dtype=torch.int32, device="cuda"),
                   path=torch.empty((batch, max_path), dtype=torch.int32, device="cuda"),
                   resample_node=torch.empty(batch, dtype=torch.int32, device="cuda"),
                   resample_token=torch.empty(batch, dtype=torch.int32, device="cuda"),
                   node_ok=torch.empty(total, dtype=torch.uint8, device="cuda"))

    def attention():
        tv.tree_verify_attention(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                                 dev["prefix_len"], dev["k_tree"], dev["v_tree"], dev["cu_nodes"],
                                 anc, mn, case.max_prefix, out=out, want_lse=False,
                                 workspace=ws_attn if ws_a else None, err=err)

    def accept():
        tv.tree_accept(dev["p_target"], dev["p_draft"], dev["token"], dev["u_accept"],
                       dev["u_resample"], dev["parent"], dev["cu_nodes"], mn, max_path,
                       outputs=acc_out, workspace=ws_acc, err=err)

    def step():
        tv.tree_build_index(dev["parent"], dev["cu_nodes"], mn, anc=anc, depth=depth, err=err)
        attention()
        accept()

    steps = args.steps if headline else min(args.steps, args.other_steps)
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise SystemExit(f"workload {config}: device error word {int(err.item())}")

    # eager rate (host launch overhead included)
    t0 = time.perf_counter()
    n_eager = min(steps, 100)
    for _ in range(n_eager):
        step()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / n_eager

    # graph-captured step, K replays between two events (synchronised on both sides)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / steps
    del graph
    if int(err.item()) != 0:
        raise SystemExit(f"workload {config}: device error word {int(err.item())}")

    # attention alone: back-to-back launches in one graph, timed on its stream
    attn_us = graph_time_us(torch, attention, args.kernel_reps)
    accept_us = graph_time_us(torch, accept, args.kernel_reps)
    roof = roofline(case, config, attn_us)
    torch.cuda.synchronize()
    accepted = int(acc_out["accept_len"].sum().item()) + int((acc_out["resample_token"] >= 0).sum().item())
    res = dict(workload=W.CONFIG_NAMES[config], steps=steps, ms_per_step=round(ms_step, 5),
               us_per_step=round(ms_step * 1e3, 2), us_per_step_eager=round(eager_ms * 1e3, 2),
               tokens_per_s=round(total / (ms_step * 1e-3), 1), attention_us=round(attn_us, 3),
               accept_us=round(accept_us, 3),
               roofline=roof,
               config={"workload": W.CONFIG_NAMES[config], "batch": batch, "tree_nodes": total,
                       "max_prefix": case.max_prefix, "hq": case.hq, "hkv": case.hkv,
                       "head_dim": case.d, "vocab": case.vocab},
               accepted={"tokens_per_step": accepted,
                         "tokens_per_s": round(accepted / (ms_step * 1e-3), 1)},
               wall_s=round(wall, 3), input_gen_s=round(t_gen, 1),
               dtype="bf16" if case.dtype == W.DT_BF16 else "f32")
    fp8 = measure_fp8(tv, case, dev, anc, mn, attn_us, args.kernel_reps)
    if headline:
        res["next_rows"] = {"kv_commit": measure_commit(tv, case, dev, acc_out, max_path, args.kernel_reps),
                            "softmax_rows": measure_softmax(tv, case, args.kernel_reps),
                            "fp8_kv_attention": fp8,
                            "draft_tree": measure_draft_tree(tv, case, args.kernel_reps),
                            "uniforms": measure_uniforms(tv, case, dev, depth, args.kernel_reps),
                            "step_graph": measure_step_graph(tv, case, dev, min(steps, 100))}
        res["measured_copy_GBps"] = measured_copy_gbps(torch)
    elif fp8 is not None:
        res["fp8_kv_attention"] = fp8
    del dev, anc, depth, out, ws_attn, ws_acc, acc_out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(f"# workload {config} done: step {res['us_per_step']} us, attention {attn_us:.2f} us",
          file=sys.stderr, flush=True)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--only", action="store_true", help="measure the headline workload only")
    ap.add_argument("--other-steps", type=int, default=200, help="steps timed per other workload")
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain copy of a known size first (for counter scaling)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"),
                    help="write the traffic summary for --config from two counter passes")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("RESULTS_DB", "COMMAND"),
                    help="write the kernel-trace summary for --config from a rocprofv3 database")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.config, *args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(args.config, *args.summarize_trace)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; the verify path is "
                                   "measured on one GPU's share (--gpus must be 1)"}))
        sys.exit(2)

    import torch
    import tree_attention_verification_04_amd as tv

    tv.load()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1.0, out=dst)  # an elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        del src, dst
    head = measure_workload(torch, tv, args.config, args, headline=True)
    others = {}
    if not args.only:
        for c in range(5):
            if c != args.config:
                r = measure_workload(torch, tv, c, args, headline=False)
                others[r["workload"].split(":")[0]] = r

    cfg = dict(head["config"])
    cfg.update(step="tree_build_index + tree_verify_attention + tree_accept",
               timing="HIP-graph replay, events on the launch stream", wall_s=head["wall_s"])
    roof = dict(head["roofline"])
    roof["measured_copy_GBps"] = head["measured_copy_GBps"]
    res = {
        "metric": "verified tree tokens/s",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "us_per_step": head["us_per_step"],
        "us_per_step_eager": head["us_per_step_eager"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded, HBM-resident; pages' datasets and models are not used)",
        "config": cfg,
        "roofline": roof,
        "attention_us": head["attention_us"],
        "accept_us": head["accept_us"],
        "accepted": dict(head["accepted"], note="accepted path lengths + resampled tokens; the "
                         "synthetic target and draft rows are independent draws, not a model's"),
        "next_rows": head["next_rows"],
    }
    if "cpu_baseline" in head:
        res["cpu_baseline"] = head["cpu_baseline"]
    if others:
        res["other_workloads"] = others
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
