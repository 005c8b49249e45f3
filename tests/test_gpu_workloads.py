"""GPU parity at the named workloads' full sizes, in the launch
configuration bench.py times (LayerPlan buffers, one call per step on the
current stream).  What each workload checks against the oracle:

  * index arrays (block and column counts, block starts, column keys) of
    every q head, bit for bit, against oracle.build_index run on the GPU's
    own top-k sets (head by head, compared on the GPU);
  * estimator scores (element by element) and top-k sets (tie band) of
    sampled heads: three at 128K, one per kv head at 512K and 1M;
  * sparse attention outputs and lse on sampled query blocks (0, 1, the
    last, and seeded random ones) of the sampled heads;
  * dense attention on sampled query blocks, 1M included;
  * the fused sparse prefill (work lists walked inside the kernel) on the
    layer's own sets: bitwise equal to the list path on every (q head,
    query block) the grouped walk did not take, graded tolerances on the
    rest; and its exact union mask (MSA_FUSED_EXACT) against the oracle's
    exact_attention_blocks on sampled query blocks (128K, 1M, 1M-band);
  * mixed 256K: every A-shape and vertical-slash head's arrays exact, every
    row of every block-sparse head within the tie band, attention sampled.
"""

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_vertical_amd as msa
import oracle
from dynamic_sparse_attention_vertical_amd.layer import LayerPlan, MixedPlan, mixed_layer
from parity import (SCORE_RTOL, check_band, compare_index, compare_lse, compare_out,
                    to_oracle_index)
from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def sample_blocks(nqb, k, seed):
    r = np.random.default_rng(seed)
    extra = r.choice(np.arange(2, nqb - 1), size=min(k, nqb - 3), replace=False).tolist()
    return sorted(set([0, 1, nqb - 1] + extra))


def check_vs_heads(x, w, plan, heads):
    """Scores and index sets of sampled heads against the oracle."""
    q, k = x["q"], x["k"]
    n = w.seq_len
    G = w.group
    for h in heads:
        g = h // G
        vsc = torch.empty((G, n), dtype=torch.float32, device="cuda")
        ssc = torch.empty((G, n), dtype=torch.float32, device="cuda")
        vi, si = msa.estimate_vs(q[g * G:(g + 1) * G], k[g:g + 1], w.vertical_topk, w.slash_topk,
                                 v_score=vsc, s_score=ssc)
        hh = h - g * G
        # the group-local call selects the same sets as the full-layer call
        assert torch.equal(vi[hh], plan.v_idx[h]) and torch.equal(si[hh], plan.s_idx[h])
        qc = q[h:h + 1, n - 64:].cpu()
        qfull = torch.zeros((1, n, 128), dtype=q.dtype)
        qfull[0, n - 64:] = qc[0]
        rv, rs = oracle.estimate_vs(qfull, k[g:g + 1].cpu(), last_q=64)
        for gs, r, name in ((vsc[hh], rv[0], "v"), (ssc[hh], rs[0], "s")):
            gg = gs.cpu().numpy().astype(np.float64)
            bad = np.abs(gg - r) > SCORE_RTOL * r + 1e-6
            assert not bad.any(), f"head {h} {name}: {bad.sum()} scores off (max {np.abs(gg - r).max():.3e})"
        check_band(plan.v_idx[h].cpu().numpy(), rv[0], w.vertical_topk, f"head {h} v_idx")
        check_band(plan.s_idx[h].cpu().numpy(), rs[0], w.slash_topk, f"head {h} s_idx")
        log(f"  head {h}: scores and sets within tolerance")


def check_index_heads(plan_idx, v_idx, s_idx, n, heads):
    """Index arrays of the sampled heads against the oracle (CPU compare);
    returns the oracle's index of those heads."""
    vi = v_idx.cpu().numpy()
    si = s_idx.cpu().numpy()
    ridx = oracle.build_index(vi[heads], si[heads], n)
    sub = msa.IndexTensors(plan_idx.block_count[heads], plan_idx.block_offset[heads],
                           plan_idx.column_count[heads], plan_idx.column_index[heads])
    compare_index(sub, ridx, "index")
    return ridx


def compare_head_arrays_gpu(gidx, h, ridx, r, what):
    """Row r of an oracle index against head h of a GPU index, exactly, up
    to each count (the compare runs on the GPU: a 1M head is 400 MB)."""
    dev = gidx.block_count.device
    rbc = torch.from_numpy(ridx.block_count[r]).to(dev)
    rcc = torch.from_numpy(ridx.column_count[r]).to(dev)
    assert torch.equal(gidx.block_count[h], rbc), f"{what}: block counts differ"
    assert torch.equal(gidx.column_count[h], rcc), f"{what}: column counts differ"
    for cnt, garr, rarr, name in ((rbc, gidx.block_offset[h], ridx.block_offset[r], "block starts"),
                                  (rcc, gidx.column_index[h], ridx.column_index[r], "columns")):
        wd = int(cnt.max().item()) if cnt.numel() else 0
        if wd == 0:
            continue
        ref = torch.from_numpy(np.ascontiguousarray(rarr[:, :wd])).to(dev)
        valid = torch.arange(wd, device=dev)[None, :] < cnt[:, None]
        diff = (garr[:, :wd] != ref) & valid
        assert not bool(diff.any()), f"{what}: {int(diff.sum())} {name} differ"


def check_index_all_heads(plan_idx, v_idx, s_idx, n, what):
    """Every head's arrays against oracle.build_index on that head's sets."""
    vi = v_idx.cpu().numpy()
    si = s_idx.cpu().numpy()
    for h in range(vi.shape[0]):
        ridx = oracle.build_index(vi[h:h + 1], si[h:h + 1], n)
        compare_head_arrays_gpu(plan_idx, h, ridx, 0, f"{what} head {h}")
    log(f"  {what}: index arrays of all {vi.shape[0]} heads exact")


def check_attention(x, out, lse, idx_rows, items, what):
    q, k, v = x["q"].cpu(), x["k"].cpu(), x["v"].cpu()
    ref = oracle.masked_attention_blocks(q, k, v, idx_rows[0], items, head_rows=idx_rows[1])
    for (h, b), (o, l) in ref.items():
        compare_out(out[h, 64 * b: 64 * b + 64].float().cpu().numpy(), o, False, f"{what} h{h} b{b}")
        compare_lse(lse[h, 64 * b: 64 * b + 64].cpu().numpy(), l, f"{what} h{h} b{b}")
    log(f"  {what}: {len(items)} sampled query blocks within tolerance")


def check_dense(x, n, items):
    q, k, v = x["q"], x["k"], x["v"]
    out, lse = msa.dense_prefill(q, k, v, lse=True)
    torch.cuda.synchronize()
    ref = oracle.dense_attention_blocks(q.cpu(), k.cpu(), v.cpu(), items)
    for (h, b), (o, l) in ref.items():
        compare_out(out[h, 64 * b: 64 * b + 64].float().cpu().numpy(), o, False, f"dense h{h} b{b}")
        compare_lse(lse[h, 64 * b: 64 * b + 64].cpu().numpy(), l, f"dense h{h} b{b}")
    log(f"  dense: {len(items)} sampled query blocks within tolerance")


def check_fused(x, w, plan, out, lse, items):
    """msa_sparse_prefill_fused on the layer's sets against the list path's
    output: the same tiles in the same order except where the grouped walk
    ran."""
    q, k, v = x["q"], x["k"], x["v"]
    hq, n = q.shape[0], q.shape[1]
    nbytes = msa.sparse_prefill_fused_workspace_bytes(hq, w.n_kv_heads, n, w.vertical_topk, q.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
    fout = torch.empty_like(out)
    flse = torch.empty_like(lse)
    msa.sparse_prefill_fused(q, k, v, plan.v_idx, plan.s_idx, out=fout, lse=flse, workspace=ws)
    torch.cuda.synchronize()
    del ws
    marks = msa.sparse_walk_marks(plan.attn_workspace, hq, w.n_kv_heads, n, q.dtype) \
        if plan.attn_workspace is not None else None
    rows = torch.ones((hq, n), dtype=torch.bool, device="cuda") if marks is None else \
        (marks == 0).repeat_interleave(64, dim=1)[:, :n]
    for h in range(hq):
        r = rows[h]
        assert torch.equal(fout[h][r], out[h][r]), f"fused head {h}: outputs differ where the walk did not run"
        assert torch.equal(flse[h][r], lse[h][r]), f"fused head {h}: lse differs where the walk did not run"
        if not bool(r.all()):
            compare_out(fout[h][~r].float().cpu().numpy(), out[h][~r].float().cpu().numpy(), False, f"fused h{h}")
            compare_lse(flse[h][~r].cpu().numpy(), lse[h][~r].cpu().numpy(), f"fused h{h}")
    walked = 0 if marks is None else int((marks != 0).sum())
    log(f"  fused: bitwise equal on {hq * (n // 64) - walked} of {hq * (n // 64)} (head, query block) items, "
        f"the rest within tolerance")
    # the exact union mask on the same sets, sampled against the oracle
    nbytes = msa.sparse_prefill_fused_workspace_bytes(hq, w.n_kv_heads, n, w.vertical_topk, q.dtype, exact=True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    msa.sparse_prefill_fused(q, k, v, plan.v_idx, plan.s_idx, out=fout, lse=flse, exact=True, workspace=ws)
    torch.cuda.synchronize()
    del ws
    vi, si = plan.v_idx.cpu().numpy(), plan.s_idx.cpu().numpy()
    ref = oracle.exact_attention_blocks(q.cpu(), k.cpu(), v.cpu(), vi, si, items)
    for (h, b), (o, l) in ref.items():
        compare_out(fout[h, 64 * b: 64 * b + 64].float().cpu().numpy(), o, False, f"exact h{h} b{b}")
        compare_lse(flse[h, 64 * b: 64 * b + 64].cpu().numpy(), l, f"exact h{h} b{b}")
    log(f"  fused exact union mask: {len(items)} sampled query blocks within tolerance")


def run_vs_workload(name, heads, n_blocks, dense_blocks=6, attn_heads=None, fused=False):
    """The layer as bench.py runs it, then: estimator scores and sets of
    `heads`; every head's index arrays; sparse attention on n_blocks sampled
    query blocks of `attn_heads` (default: the first two of `heads`); dense
    attention on dense_blocks of them for the first head."""
    w = WORKLOADS[name]
    n, hq = w.seq_len, w.n_q_heads
    log(f"[{name}] generating inputs")
    x = make_inputs(w, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    plan = LayerPlan(hq, w.n_kv_heads, n, w.vertical_topk, w.slash_topk, "cuda", q.dtype)
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    out, plan = msa.vertical_slash_layer(q, k, v, w.vertical_topk, w.slash_topk, plan=plan, lse=lse)
    out = out[0]
    torch.cuda.synchronize()
    log(f"[{name}] layer done")
    check_vs_heads(x, w, plan, heads)
    check_index_all_heads(plan.index, plan.v_idx, plan.s_idx, n, name)
    attn_heads = heads[:2] if attn_heads is None else attn_heads
    ridx = check_index_heads(plan.index, plan.v_idx, plan.s_idx, n, attn_heads)
    nqb = n // 64
    blocks = sample_blocks(nqb, n_blocks, seed=n)
    items = [(h, b) for h in attn_heads for b in blocks]
    check_attention(x, out, lse, (ridx, {h: i for i, h in enumerate(attn_heads)}), items, "sparse")
    if dense_blocks:
        check_dense(x, n, [(attn_heads[0], b) for b in blocks[:dense_blocks]])
    if fused:
        check_fused(x, w, plan, out, lse, [(h, b) for h in attn_heads for b in blocks[:4]])
    return plan


def test_single_head_4k_full_parity():
    """Whole-array parity at the single-head 4K workload, float32 and bfloat16."""
    w = WORKLOADS["single_head_4k"]
    n = w.seq_len
    x = make_inputs(w)
    for fp32 in (True, False):
        sfx = "32" if fp32 else ""
        q, k, v = x["q" + sfx], x["k" + sfx], x["v" + sfx]
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        vsc = torch.empty((1, n), dtype=torch.float32, device="cuda")
        ssc = torch.empty((1, n), dtype=torch.float32, device="cuda")
        vi, si = msa.estimate_vs(qd, kd, w.vertical_topk, w.slash_topk, v_score=vsc, s_score=ssc)
        rv, rs = oracle.estimate_vs(q, k, last_q=64)
        for gs, r in ((vsc, rv), (ssc, rs)):
            gg = gs.cpu().numpy().astype(np.float64)
            assert np.all(np.abs(gg - r) <= SCORE_RTOL * r + 1e-6)
        check_band(vi[0].cpu().numpy(), rv[0], w.vertical_topk, "v")
        check_band(si[0].cpu().numpy(), rs[0], w.slash_topk, "s")
        idx = msa.build_index(vi, si, n)
        ridx = oracle.build_index(vi.cpu().numpy(), si.cpu().numpy(), n)
        compare_index(idx, ridx, "index")
        out, lse = msa.sparse_prefill(qd, kd, vd, idx, lse=True)
        ref, rlse = oracle.attention_with_mask(q, k, v, oracle.index_mask(ridx, n))
        compare_out(out.float().cpu().numpy(), ref, fp32, "sparse")
        compare_lse(lse.cpu().numpy(), rlse, "sparse")
        dout, dlse = msa.dense_prefill(qd, kd, vd, lse=True)
        dref, drlse = oracle.dense_attention(q, k, v)
        compare_out(dout.float().cpu().numpy(), dref, fp32, "dense")
        compare_lse(dlse.cpu().numpy(), drlse, "dense")
        log(f"single_head_4k {'fp32' if fp32 else 'bf16'}: full parity")


def test_llama3_8b_128k():
    run_vs_workload("llama3_8b_128k", heads=[0, 13, 31], n_blocks=10, attn_heads=[0, 13, 31], fused=True)


# one q head per kv head (G = 4), the first of each group but for two groups
ONE_PER_KV = [0, 5, 10, 15, 16, 22, 26, 31]


def test_llama3_8b_512k():
    run_vs_workload("llama3_8b_512k", heads=ONE_PER_KV, n_blocks=8, attn_heads=[0, 22])


def test_llama3_8b_1m():
    run_vs_workload("llama3_8b_1m", heads=ONE_PER_KV, n_blocks=6, attn_heads=[5, 31], fused=True)


def test_llama3_8b_1m_band():
    """The 1M layer with clustered slashes: long runs of adjacent diagonals, so
    the index is mostly long contiguous block runs plus the leftover columns."""
    plan = run_vs_workload("llama3_8b_1m_band", heads=[2, 27], n_blocks=6, dense_blocks=0, fused=True)
    # the clustering is what this workload is for: far fewer blocks than the
    # iid 1M layer's (about one per selected diagonal there)
    assert plan.index.block_count.float().mean().item() < 0.5 * 6096


def test_mixed_256k():
    w = WORKLOADS["mixed_256k"]
    n, hq = w.seq_len, w.n_q_heads
    x = make_inputs(w, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    plan = MixedPlan(w.head_patterns, w.n_kv_heads, n, w.vertical_topk, w.slash_topk, w.sink, w.window,
                     w.bs_topk, "cuda", q.dtype)
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    out, lse = mixed_layer(q, k, v, plan, lse=lse)
    torch.cuda.synchronize()
    log("[mixed_256k] layer done")
    nqb = n // 64
    a_heads, vs_heads, bs_heads = w.heads_with("a"), w.heads_with("vs"), w.heads_with("bs")
    # A-shape heads: static index, exact, every head
    av, as_ = oracle.a_shape_sets(n, w.sink, w.window)
    ra = oracle.build_index(av[None], as_[None], n)
    for h in a_heads:
        compare_head_arrays_gpu(plan.index, h, ra, 0, f"a-shape head {h}")
    # vertical-slash heads: arrays exact for every head (given its sets), sets
    # within the band for two of them
    vs_rows = {h: i for i, h in enumerate(vs_heads)}
    for h in vs_heads:
        r = vs_rows[h]
        ridx = oracle.build_index(plan.v_idx[r:r + 1].cpu().numpy(), plan.s_idx[r:r + 1].cpu().numpy(), n)
        compare_head_arrays_gpu(plan.index, h, ridx, 0, f"vs head {h}")
    sample_vs = [vs_heads[0], vs_heads[-1]]
    for h in sample_vs:
        r = vs_rows[h]
        qfull = torch.zeros((1, n, 128), dtype=q.dtype)
        qfull[0, n - 64:] = q[h, n - 64:].cpu()
        rv, rs = oracle.estimate_vs(qfull, k[h // w.group: h // w.group + 1].cpu(), last_q=64)
        check_band(plan.v_idx[r].cpu().numpy(), rv[0], w.vertical_topk, f"vs head {h} v")
        check_band(plan.s_idx[r].cpu().numpy(), rs[0], w.slash_topk, f"vs head {h} s")
    # block-sparse heads: every query block's chosen key blocks within the band
    # of the row softmax of the oracle's block scores, every head
    qc, kc = q.cpu(), k.cpu()
    for h in bs_heads:
        u = oracle.block_scores(qc, kc, h)
        bc = plan.index.block_count[h].cpu().numpy()
        bo = plan.index.block_offset[h].cpu().numpy()
        assert np.all(plan.index.column_count[h].cpu().numpy() == 0)
        for b in range(nqb):
            kk = min(w.bs_topk, b + 1)
            assert bc[b] == kk
            row = u[b, : b + 1]
            pr = np.exp(row - row.max())
            check_band(bo[b, :kk] // 64, pr / pr.sum(), kk, f"bs head {h} block {b}")
            assert np.all(bo[b, :kk] % 64 == 0)
        log(f"  bs head {h}: all {nqb} query blocks within the band")
    log("[mixed_256k] index checks passed")
    # attention on sampled blocks of every pattern, with the GPU's (validated) index
    heads = [a_heads[0], sample_vs[0], bs_heads[-1]]
    gi = to_oracle_index(msa.IndexTensors(plan.index.block_count[heads], plan.index.block_offset[heads],
                                          plan.index.column_count[heads], plan.index.column_index[heads]))
    blocks = sample_blocks(nqb, 5, seed=7)
    items = [(h, b) for h in heads for b in blocks]
    check_attention(x, out, lse, (gi, {h: i for i, h in enumerate(heads)}), items, "mixed")
