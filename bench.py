"""Benchmark: one vertical-slash sparse prefill layer on one MI355X.

A step is one pass of the whole hot path over one layer's synthetic input
already resident in HBM: online estimation (scores + top-k), index build, and
the sparse prefill kernel.  Prints one JSON line:

  value      = listed sparse-attention TFLOP per layer / layer time
               (effective TFLOP/s; every 64x64 tile of the work lists counts
               4 * 128 * 64 * 64 FLOP, per block and per 64-column chunk; the
               masked tiles that the grouped walk also runs are not counted)
  roofline   = the sparse prefill kernel against the bf16 MFMA peak on the
               tiles it executed (listed tiles, plus every aligned tile 0..b
               of the query blocks the grouped walk ran), timed with HIP events
               on its own stream over the timed steps
  cpu_baseline = the float64 CPU oracle on a bounded sample, extrapolated to
               the layer

The default workload is the 1M-token LLaMA-3-8B-shaped layer (32 q / 8 kv
heads, vertical top-k 1000, slash top-k 6096), with the dense causal kernel
timed at the same shape for the speedup.

usage: python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse prefill ms/layer & eff. TFLOP/s (fraction of MFMA peak), 128K-1M tokens"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TILE_FLOP = 4 * 128 * 64 * 64  # QK^T + PV for one 64x64 tile, head_dim 128


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_sparse_traffic.json")
ATTN_SRC = os.path.join(ROOT, "dynamic_sparse_attention_vertical_amd", "csrc", "attention.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def attn_src_sha():
    import hashlib
    return hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes of one step's sparse prefill (the sum over its key-phase
    launches) from the committed rocprofv3 counter runs (FETCH_SIZE and
    WRITE_SIZE, each scaled by the same counter's reading for a plain copy of
    known size), or None if absent or taken on a different kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload)
    if not entry or rec.get("attention_src_sha") != attn_src_sha():
        return None
    return entry["fetch_kib_per_step"] * 1024 * rec["fetch_calib"] + \
        entry["write_kib_per_step"] * 1024 * rec["write_calib"]


DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


def measured_decode_traffic(workload):
    """HBM bytes of one decode step (scores, stats, top-k and attend kernels)
    from the committed rocprofv3 counter runs, scaled like measured_traffic,
    or None if absent or taken on a different source of those kernels."""
    import hashlib
    try:
        rec = json.load(open(DECODE_TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    csrc = os.path.dirname(ATTN_SRC)
    for name, sha in rec.get("src_sha", {}).items():
        if hashlib.sha256(open(os.path.join(csrc, name), "rb").read()).hexdigest()[:16] != sha:
            return None
    entry = rec.get("workloads", {}).get(workload)
    if not entry:
        return None
    return entry["fetch_kib_per_step"] * 1024 * rec["fetch_calib"] + \
        entry["write_kib_per_step"] * 1024 * rec["write_calib"]


def phase_launches(n):
    """Launches of one sparse prefill at the default phase length: the
    grouped walk, then one per key phase (a single launch when one phase
    covers the sequence)."""
    from dynamic_sparse_attention_vertical_amd.msa import DEFAULT_PHASE_KEYS
    return 1 + -(-n // DEFAULT_PHASE_KEYS) if n > DEFAULT_PHASE_KEYS else 1


def copy_calibration(gib):
    """A plain device copy of a known size, for calibrating HBM byte counters."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4}), flush=True)


def listed_tiles(idx):
    """64-key tiles of the work lists: every block, and the columns in
    chunks of 64 per query block."""
    import torch
    bc = idx.block_count.to(torch.int64)
    cc = idx.column_count.to(torch.int64)
    return int(bc.sum().item() + ((cc + 63) // 64).sum().item())


def executed_tiles(idx, marks):
    """Tiles the sparse prefill ran: the listed ones, except that a query
    block b the grouped walk took ran every aligned tile 0..b (masked to its
    lists).  marks: [Hq, nQB] from msa.sparse_walk_marks, or None."""
    import torch
    bc = idx.block_count.to(torch.int64)
    per = bc + (idx.column_count.to(torch.int64) + 63) // 64
    if marks is not None:
        b = torch.arange(per.shape[1], device=per.device, dtype=torch.int64)[None, :] + 1
        per = torch.where(marks.to(per.device) != 0, b.expand_as(per), per)
    return int(per.sum().item()), (0 if marks is None else int((marks != 0).sum().item()))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def useful_pairs(idx, n):
    """Number of (i, j) pairs the mask allows (j <= i, j listed for i's block)."""
    import torch
    H, nqb, cap = idx.block_offset.shape
    dev = idx.block_count.device
    # a block starting a = st - r0 keys after the query block's first row covers
    # sum_t clamp(t - a + 1, 0, 64) pairs over its 64 rows t
    a = torch.arange(-63, 64, device=dev, dtype=torch.int64)
    t = torch.arange(64, device=dev, dtype=torch.int64)
    table = (t[None, :] - a[:, None] + 1).clamp(0, 64).sum(1)
    r0 = torch.arange(nqb, device=dev, dtype=torch.int64) * 64
    total = 0
    for h in range(H):
        st = idx.block_offset[h].to(torch.int64)
        valid = torch.arange(cap, device=dev)[None, :] < idx.block_count[h][:, None]
        off = (st - r0[:, None]).clamp(-63, 63) + 63
        total += int((table[off] * valid).sum().item())
        ci = idx.column_index[h].to(torch.int64)
        cvalid = torch.arange(ci.shape[1], device=dev)[None, :] < idx.column_count[h][:, None]
        rows = (r0[:, None] + 63 - ci + 1).clamp(min=0, max=64)
        total += int((rows * cvalid).sum().item())
    return total


def cpu_baseline(x, plan, w, target_s=20.0):
    """Time the float64 oracle on a bounded sample and extrapolate to the layer."""
    import numpy as np
    import oracle
    n, hq, G = w.seq_len, w.n_q_heads, w.group
    nqb = n // 64
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    q, k, v = x["q"].cpu(), x["k"].cpu(), x["v"].cpu()
    v_idx, s_idx = plan.v_idx.cpu().numpy(), plan.s_idx.cpu().numpy()
    # estimator for one head
    t0 = time.perf_counter()
    oracle.estimate_vs(q, k, last_q=64, heads=[0])
    t_est = (time.perf_counter() - t0) * hq
    # index build, all heads (plain C)
    t0 = time.perf_counter()
    ridx = oracle.build_index(v_idx, s_idx, n)
    t_idx = time.perf_counter() - t0
    # masked attention on sampled query blocks of head 0 until ~target_s
    rng = np.random.default_rng(0)
    order = [nqb - 1, 0, 1] + rng.permutation(np.arange(2, nqb - 1)).tolist()
    done, keys_done, t_att = [], 0, 0.0
    for b in order:
        t0 = time.perf_counter()
        oracle.masked_attention_blocks(q, k, v, ridx, [(0, b)])
        t_att += time.perf_counter() - t0
        done.append(b)
        keys_done += 64 * b + 64
        if t_est / hq + t_idx + t_att > target_s or len(done) >= 64:
            break
    keys_total = hq * sum(64 * b + 64 for b in range(nqb))
    t_layer = t_est + t_idx + t_att * keys_total / keys_done
    tiles = int(ridx.block_count.sum() + ((ridx.column_count + 63) // 64).sum())
    return {
        "value": round(tiles * TILE_FLOP / t_layer / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"float64 oracle: estimator on 1 of {hq} heads, index build on all heads, masked "
                   f"attention on {len(done)} of {nqb} query blocks of head 0; layer time extrapolated "
                   f"by heads and by keys scanned ({t_layer:.1f} s/layer, {t_est / hq:.2f} s estimator "
                   f"per head, {t_idx:.2f} s index, {t_att:.2f} s attention measured)"),
    }


def time_graph(step, outs, steps, warmup):
    """Capture step() once as a HIP graph (graphs.StepGraph) and time `steps`
    replays back to back with events on the stream they run on; also whether
    the replays left outs (the eager step's results on the same inputs)
    bit-identical."""
    import torch
    from dynamic_sparse_attention_vertical_amd.graphs import StepGraph

    before = [t.clone() for t in outs]
    g = StepGraph(step)
    for t in outs:      # so that equal results after the replays show that the replays computed them
        t.fill_(float("nan") if t.is_floating_point() else -1)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    same = all(torch.equal(a, b) for a, b in zip(before, outs))
    del before, g
    return {"ms_per_step": round(ms, 4), "replays": steps, "replay_equals_eager": same}


def bench_decode(args, dw):
    """One decode step over a batch of key caches (msa_decode_sparse): scores
    for every cached key, the top-k per head, attention over them.  Bound by
    HBM: the algorithmic bytes are the K caches read once plus the selected V
    rows.  A dense decode step reads K and V whole; both floors at 8 TB/s are
    reported beside the measured time."""
    import torch
    import dynamic_sparse_attention_vertical_amd as msa
    from synth import make_decode_inputs

    log(f"[bench] decode workload {dw.name}: batch {dw.batch}, {dw.n_q_heads}q/{dw.n_kv_heads}kv heads, "
        f"cache {dw.cache_len}, top-{dw.topk}")
    x = make_decode_inputs(dw, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    lens = x.get("cache_lens")                # sequences of different lengths: msa_decode_sparse_varlen
    hq, hkv, n = q.shape[0], k.shape[0], dw.cache_len
    stream = torch.cuda.current_stream()
    ws = torch.empty(msa.decode_sparse_workspace_bytes(hq, hkv, n, q.dtype), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    idx = torch.empty((hq, dw.topk), dtype=torch.int32, device="cuda")
    rec = torch.empty(hq, dtype=torch.float32, device="cuda")

    def step():     # on torch's current stream (a graph capture makes its own stream current)
        msa.decode_sparse(q, k, v, dw.topk, idx=idx, out=out, recovery=rec, cache_lens=lens, workspace=ws,
                          stream=torch.cuda.current_stream())

    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    reps = max(args.steps, 20)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    graph = None
    if args.graph:
        graph = time_graph(step, [out, idx, rec], reps, args.warmup)
        log(f"[bench] decode step as one HIP graph {graph['ms_per_step']:.4f} ms")
    recovery = rec.clone()
    k_bytes = sum(dw.length(b) for b in range(dw.batch)) * dw.n_kv_heads * 128 * 2   # the keys that exist
    v_bytes = hq * dw.topk * 128 * 2
    alg = k_bytes + v_bytes
    gbs = alg / (ms * 1e-3) / 1e9
    log(f"[bench] decode step {ms:.4f} ms")
    res = {
        "metric": "decode_sparse_step_hbm_GBps",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": dw.name, "batch": dw.batch, "q_heads": dw.n_q_heads, "kv_heads": dw.n_kv_heads,
                   "cache_len": n, "topk": dw.topk, "head_dim": 128,
                   **({"cache_lens": list(dw.lengths)} if dw.lengths else {})},
        "breakdown": {
            "ms_floor_sparse_step": round(alg / PEAK_HBM_GBS / 1e6, 4),
            "ms_floor_dense_decode": round(2 * k_bytes / PEAK_HBM_GBS / 1e6, 4),
            "kept_attention_share": {"mean": round(float(recovery.mean()), 4),
                                     "min": round(float(recovery.min()), 4),
                                     "note": "synthetic iid queries and keys: near-flat attention"},
            "k_cache_bytes": k_bytes, "selected_v_bytes": v_bytes,
            **({"graph": {**graph, "speedup_vs_eager": round(ms / graph["ms_per_step"], 3)}} if graph else {}),
        },
        "roofline": {"bound": "hbm", "kernel": "decode_scores_kernel + top-k + decode_attend_kernel (one step)",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_decode_traffic(dw.name),
                     "traffic_source": ("rocprofv3 FETCH_SIZE + WRITE_SIZE of the same source, committed in "
                                        "profiles/decode_traffic.json (null when the decode, top-k or layout "
                                        "source has changed since)")},
    }
    print(json.dumps(res), flush=True)


def bench_packed(args, pw):
    """One packed prefill layer: sequences of different lengths packed along
    the rows, each estimated, indexed and attended as on its own, in one
    launch chain (the msa_*_varlen calls); the dense causal kernel over the
    same packed batch for the speedup; and, for reference, the same sequences
    as one call chain each (what a packed batch cost before the variable-length
    calls).  TFLOP/s on the work lists' tiles, as for one sequence."""
    import torch
    import dynamic_sparse_attention_vertical_amd as msa
    from dynamic_sparse_attention_vertical_amd.layer import LayerPlan, vertical_slash_layer
    from synth import make_packed_inputs

    lens = list(pw.lengths)
    hq, hkv, nseq = pw.n_q_heads, pw.n_kv_heads, len(lens)
    rows, max_len = sum(lens), max(lens)
    log(f"[bench] packed workload {pw.name}: {nseq} sequences of {min(lens)}..{max_len} tokens ({rows} in all), "
        f"{hq}q/{hkv}kv heads")
    x = make_packed_inputs(pw, device="cuda")
    q, k, v, cu = x["q"], x["k"], x["v"], x["cu_seqlens"]
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    kv, ks = min(pw.vertical_topk, max_len), min(pw.slash_topk, max_len)
    heads = nseq * hq
    stream = torch.cuda.current_stream()
    est_ws = torch.empty(msa.estimate_vs_varlen_workspace_bytes(hq, hkv, rows, cu_d, max_len, q.dtype),
                         dtype=torch.uint8, device="cuda")
    v_idx = torch.empty((heads, kv), dtype=torch.int32, device="cuda")
    s_idx = torch.empty((heads, ks), dtype=torch.int32, device="cuda")
    cb, cc = msa.index_caps(max_len, kv, ks, heads)
    idx = msa.alloc_index(heads, max_len, cb, cc, "cuda")
    att_bytes = msa.sparse_prefill_varlen_workspace_bytes(hq, hkv, rows, cu_d, max_len, q.dtype)
    att_ws = torch.empty(max(att_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        msa.estimate_vs_varlen(q, k, cu_d, max_len, kv, ks, workspace=est_ws, v_idx=v_idx, s_idx=s_idx,
                               stream=stream)
        if ev is not None:
            ev[1].record(stream)
        msa.build_index_varlen(v_idx, s_idx, cu_d, max_len, hq, rows=rows, out=idx, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        msa.sparse_prefill_varlen(q, k, v, idx, cu_d, max_len, out=out, workspace=att_ws, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    per = [[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in events]
    ms_est, ms_idx, ms_att = (sum(p[j] for p in per) / len(per) for j in range(3))
    log(f"[bench] timed {args.steps} steps: {ms_step:.2f} ms/layer (estimate {ms_est:.3f}, index {ms_idx:.3f}, "
        f"sparse prefill {ms_att:.3f})")

    # tiles of the query blocks each sequence has (entries past its end are unwritten)
    nqb_max = (max_len + 63) // 64
    seq_nqb = torch.tensor([(n + 63) // 64 for n in lens], device="cuda").repeat_interleave(hq)
    live = torch.arange(nqb_max, device="cuda")[None, :] < seq_nqb[:, None]
    bc = idx.block_count.to(torch.int64) * live
    per_blk = bc + ((idx.column_count.to(torch.int64) + 63) // 64) * live
    tiles = int(per_blk.sum().item())
    marks = msa.sparse_walk_marks(att_ws, heads, hkv * nseq, max_len, q.dtype) if att_bytes else None
    run_per = per_blk
    walk_blocks = 0
    if marks is not None:
        marks = (marks != 0) & live
        b1 = torch.arange(nqb_max, device="cuda", dtype=torch.int64)[None, :] + 1
        run_per = torch.where(marks, b1.expand_as(per_blk), per_blk)
        walk_blocks = int(marks.sum().item())
    run_tiles = int(run_per.sum().item())
    causal_tiles = hq * sum(((n + 63) // 64) * ((n + 63) // 64 + 1) // 2 for n in lens)
    att_tflops = run_tiles * TILE_FLOP / (ms_att * 1e-3) / 1e12

    # dense over the same packed batch, and the per-sequence loop
    dense_out = torch.empty_like(q)
    msa.dense_prefill_varlen(q, k, v, cu_d, max_len, out=dense_out, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    msa.dense_prefill_varlen(q, k, v, cu_d, max_len, out=dense_out, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_dense = e0.elapsed_time(e1)
    plans = {}

    def loop():
        for a, b in zip(cu, cu[1:]):
            n = b - a
            if n not in plans:
                plans[n] = LayerPlan(hq, hkv, n, min(kv, n), min(ks, n), "cuda", q.dtype)
            pl = plans[n]
            vertical_slash_layer(q[:, a:b], k[:, a:b], v[:, a:b], pl.vertical_topk, pl.slash_topk, plan=pl,
                                 out=dense_out[:, a:b], stream=stream)
    loop()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop()
    torch.cuda.synchronize()
    ms_loop = (time.perf_counter() - t0) * 1e3
    log(f"[bench] dense over the packed batch {ms_dense:.2f} ms; one call chain per sequence {ms_loop:.2f} ms")
    res = {
        "metric": METRIC,
        "value": round(tiles * TILE_FLOP / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": pw.name, "step": "packed lists", "sequences": nseq, "total_tokens": rows,
                   "max_seqlen": max_len, "min_seqlen": min(lens), "q_heads": hq, "kv_heads": hkv, "head_dim": 128,
                   "vertical_topk": pw.vertical_topk, "slash_topk": pw.slash_topk, "last_q": 64, "block": 64},
        "breakdown": {
            "ms_estimate": round(ms_est, 4), "ms_build_index": round(ms_idx, 4),
            "ms_sparse_prefill": round(ms_att, 4),
            "listed_tiles": tiles, "executed_tiles": run_tiles, "causal_tiles": causal_tiles,
            "grouped_walk_blocks": walk_blocks,
            "listed_density": round(tiles / causal_tiles, 5), "executed_density": round(run_tiles / causal_tiles, 5),
            "sparse_prefill_tflops": round(att_tflops, 2),
            "ms_dense_prefill": round(ms_dense, 3),
            "dense_prefill_tflops": round(causal_tiles * TILE_FLOP / (ms_dense * 1e-3) / 1e12, 2),
            "speedup_vs_dense": round(ms_dense / ms_step, 3),
            "ms_one_chain_per_sequence": round(ms_loop, 3),
            "speedup_vs_one_chain_per_sequence": round(ms_loop / ms_step, 3),
        },
        "roofline": {"bound": "mfma",
                     "kernel": "attn_fwd_kernel<bf16, packed> sparse: grouped walk + per-head key phases",
                     "launches_per_step": phase_launches(max_len),
                     "achieved": round(att_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(pw.name),
                     "traffic_source": ("rocprofv3 FETCH_SIZE + WRITE_SIZE of the same source, committed in "
                                        "profiles/attn_sparse_traffic.json (null when the kernel source "
                                        "has changed since)")},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3_8b_1m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--exact", action="store_true",
                    help="with --fused: the exact union mask (selected columns and diagonals only, "
                         "same tiles masked)")
    ap.add_argument("--fused", action="store_true",
                    help="time estimate + msa_sparse_prefill_fused (work lists walked inside the attention "
                         "kernel) as the step instead of estimate + build_index + sparse_prefill")
    ap.add_argument("--graph", action="store_true",
                    help="also capture the step as one HIP graph and time its replays (layer and decode "
                         "workloads; breakdown.graph)")
    ap.add_argument("--copy-calib", type=float, default=0.0,
                    help="only run a plain copy of this many GiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.copy_calib > 0:
        copy_calibration(args.copy_calib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the sparse prefill path has no multi-GPU mode "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dynamic_sparse_attention_vertical_amd as msa
    from dynamic_sparse_attention_vertical_amd.layer import LayerPlan, MixedPlan, mixed_index
    from synth import DECODE_WORKLOADS, PACKED_WORKLOADS, WORKLOADS, make_inputs

    if args.workload in DECODE_WORKLOADS:
        bench_decode(args, DECODE_WORKLOADS[args.workload])
        return
    if args.workload in PACKED_WORKLOADS:
        bench_packed(args, PACKED_WORKLOADS[args.workload])
        return
    w = WORKLOADS[args.workload]
    mixed = bool(w.head_patterns)
    n, hq, hkv = w.seq_len, w.n_q_heads, w.n_kv_heads
    log(f"[bench] workload {w.name}: {hq}q/{hkv}kv heads, N={n}, k={w.vertical_topk}/{w.slash_topk}")
    t0 = time.perf_counter()
    x = make_inputs(w, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] inputs generated on the GPU in {time.perf_counter() - t0:.1f} s")
    q, k, v = x["q"], x["k"], x["v"]
    if mixed:
        # heads with three patterns (A-shape, vertical-slash, block-sparse): all
        # work lists are built in one stage (timed as "estimate"), then one
        # sparse prefill over all heads
        plan = MixedPlan(w.head_patterns, hkv, n, w.vertical_topk, w.slash_topk, w.sink, w.window, w.bs_topk)
    else:
        plan = LayerPlan(hq, hkv, n, w.vertical_topk, w.slash_topk, "cuda", q.dtype)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    fused = args.fused
    exact = args.exact
    if exact and not fused:
        print("--exact needs --fused", file=sys.stderr)
        sys.exit(2)
    if fused and mixed:
        print("--fused applies to vertical-slash layers only", file=sys.stderr)
        sys.exit(2)
    fused_ws = None
    if fused:
        nbytes = msa.sparse_prefill_fused_workspace_bytes(hq, hkv, n, w.vertical_topk, q.dtype, exact=exact)
        fused_ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None

    def step(ev=None):
        # torch's current stream at call time: the timed loop's stream, or the
        # capture stream when the step is recorded as a graph
        stream = torch.cuda.current_stream()
        if ev is not None:
            ev[0].record(stream)
        if mixed:
            mixed_index(q, k, plan, stream=stream)
            if ev is not None:
                ev[1].record(stream)
                ev[2].record(stream)
        else:
            msa.estimate_vs(q, k, w.vertical_topk, w.slash_topk, workspace=plan.workspace, v_idx=plan.v_idx,
                            s_idx=plan.s_idx, stream=stream)
            if ev is not None:
                ev[1].record(stream)
            if not fused:
                msa.build_index(plan.v_idx, plan.s_idx, n, out=plan.index, stream=stream)
            if ev is not None:
                ev[2].record(stream)
        if fused:
            msa.sparse_prefill_fused(q, k, v, plan.v_idx, plan.s_idx, out=out, exact=exact, workspace=fused_ws,
                                     stream=stream)
        else:
            msa.sparse_prefill(q, k, v, plan.index, out=out, workspace=plan.attn_workspace, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in events]
    ms_est = sum(p[0] for p in per) / len(per)
    ms_idx = sum(p[1] for p in per) / len(per)
    ms_att = sum(p[2] for p in per) / len(per)
    ms_step = wall * 1e3 / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_step:.2f} ms/layer (estimate {ms_est:.3f}, index {ms_idx:.3f}, "
        f"sparse prefill {ms_att:.3f})")
    graph = None
    if args.graph and mixed:
        log("[bench] --graph: timed for vertical-slash layers only")
    elif args.graph:
        graph = time_graph(step, [out], args.steps, args.warmup)
        log(f"[bench] the step as one HIP graph: {graph['ms_per_step']:.3f} ms/layer")

    if fused:       # the lists the fused kernel walked, built once (untimed) to count their tiles
        msa.build_index(plan.v_idx, plan.s_idx, n, out=plan.index, stream=stream)
        torch.cuda.synchronize()
    tiles = listed_tiles(plan.index)
    nqb = n // 64
    causal_tiles = hq * nqb * (nqb + 1) // 2
    listed_flop = tiles * TILE_FLOP
    marks = None
    if plan.attn_workspace is not None and not fused:
        marks = msa.sparse_walk_marks(plan.attn_workspace, hq, hkv, n, q.dtype)
    run_tiles, walk_blocks = executed_tiles(plan.index, marks)
    exec_flop = run_tiles * TILE_FLOP
    pairs = useful_pairs(plan.index, n)
    causal_pairs = hq * n * (n + 1) // 2
    att_tflops = exec_flop / (ms_att * 1e-3) / 1e12

    # HBM-bound steps: algorithmic bytes over the measured time.  Estimator: K
    # read by both passes plus the two score arrays written (the top-k
    # selection inside the same call is timed with it).  Index builder: the
    # entries and counts written.
    if mixed:
        breakdown = {"ms_work_lists": round(ms_est + ms_idx, 4),
                     "head_patterns": {p: sum(x == p for x in w.head_patterns) for p in ("a", "vs", "bs")}}
    else:
        est_bytes = 2 * hkv * n * 128 * 2 + 2 * hq * n * 4
        idx_bytes = 4 * (int(plan.index.block_count.sum()) + int(plan.index.column_count.sum())) + 8 * hq * nqb
        est_gbs = est_bytes / (ms_est * 1e-3) / 1e9
        breakdown = {
            "ms_estimate": round(ms_est, 4),
            "estimate_gbs": round(est_gbs, 1), "estimate_hbm_frac": round(est_gbs / PEAK_HBM_GBS, 4)}
        if fused:
            breakdown["work_lists"] = ("walked inside the attention kernel (msa_sparse_prefill_fused); "
                                       f"{idx_bytes / 1e9:.2f} GB of lists not written")
        else:
            idx_gbs = idx_bytes / (ms_idx * 1e-3) / 1e9
            breakdown.update({"ms_build_index": round(ms_idx, 4), "build_index_gbs": round(idx_gbs, 1),
                              "build_index_hbm_frac": round(idx_gbs / PEAK_HBM_GBS, 4)})
    breakdown.update({
        "ms_sparse_prefill": round(ms_att, 4),
        "listed_tiles": tiles, "executed_tiles": run_tiles, "causal_tiles": causal_tiles,
        "grouped_walk_blocks": walk_blocks,
        "listed_density": round(tiles / causal_tiles, 5),
        "executed_density": round(run_tiles / causal_tiles, 5),
        "useful_density": round(pairs / causal_pairs, 5),
        "listed_tflop": round(listed_flop / 1e12, 4),
        "executed_tflop": round(exec_flop / 1e12, 4),
        "sparse_prefill_tflops": round(att_tflops, 2),
        "sparse_prefill_listed_tflops": round(listed_flop / (ms_att * 1e-3) / 1e12, 2),
    })
    if graph:
        breakdown["graph"] = {**graph, "speedup_vs_eager": round(ms_step / graph["ms_per_step"], 3)}
    if not args.no_dense:
        dense_out = torch.empty_like(q)
        lse_d = torch.empty((hq, n), dtype=torch.float32, device=q.device)
        msa.dense_prefill(q, k, v, out=dense_out, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        msa.dense_prefill(q, k, v, out=dense_out, lse=lse_d, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_dense = e0.elapsed_time(e1)
        # attention recall: the share of each row's dense softmax mass that the
        # sparse index keeps, exp(lse_sparse - lse_dense), from one more
        # (untimed) sparse call
        lse_s = torch.empty_like(lse_d)
        msa.sparse_prefill(q, k, v, plan.index, out=dense_out, lse=lse_s, workspace=plan.attn_workspace,
                           stream=stream)
        rec = torch.exp(lse_s - lse_d).flatten()
        breakdown["attention_recall"] = {
            "mean": round(float(rec.mean()), 4), "p05": round(float(torch.quantile(rec[::max(1, rec.numel() // 1000000)], 0.05)), 4),
            "min": round(float(rec.min()), 4), "rows": "every row of every head"}
        del lse_s, lse_d, rec
        dense_flop = causal_tiles * TILE_FLOP
        breakdown.update({"ms_dense_prefill": round(ms_dense, 3),
                          "dense_prefill_tflops": round(dense_flop / (ms_dense * 1e-3) / 1e12, 2),
                          "speedup_vs_dense": round(ms_dense / ms_step, 3)})
        del dense_out
        log(f"[bench] dense prefill {ms_dense:.2f} ms")

    res = {
        "metric": METRIC,
        "value": round(listed_flop / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "step": ("fused-exact" if exact else "fused") if fused else "lists",
                   "seq_len": n, "q_heads": hq, "kv_heads": hkv, "head_dim": 128,
                   "vertical_topk": w.vertical_topk, "slash_topk": w.slash_topk, "last_q": 64, "block": 64},
        "breakdown": breakdown,
        # the step's sparse prefill is one grouped-walk launch and n / phase_keys
        # key-phase launches (one kernel template, attention.hip): achieved =
        # the FLOPs of the tiles they executed over their summed time
        "roofline": {"bound": "mfma",
                     "kernel": ("attn_fwd_kernel<bf16> fused: per-head key phases walking the cover" if fused
                                else "attn_fwd_kernel<bf16> sparse: grouped walk + per-head key phases"),
                     "launches_per_step": phase_launches(n) - (1 if fused and phase_launches(n) > 1 else 0),
                     "achieved": round(att_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if fused else measured_traffic(w.name),
                     "traffic_source": ("rocprofv3 FETCH_SIZE + WRITE_SIZE of the same source, committed in "
                                        "profiles/attn_sparse_traffic.json (null when the kernel source "
                                        "has changed since)")},
    }
    if mixed:
        log("[bench] the CPU oracle baseline is sampled on vertical-slash layers only")
    elif not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline(x, plan, w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
