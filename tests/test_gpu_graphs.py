"""HIP-graph replay of whole call chains (graphs.StepGraph, layer_graph,
decode_graph): a vertical-slash layer (estimate, index, sparse prefill in
several key phases) and decode steps (one cache length, and per-sequence
lengths read from the device) and a packed batch (device cu_seqlens, host
max_seqlen, sequence boundaries changed between replays), each captured once
and replayed three times
with new inputs copied into the captured buffers, eager torch work and
synchronisations between the replays.  Every replay must equal, bit for bit,
the eager chain on the same inputs in buffers of its own (the kernels are
deterministic: no floating-point atomics); the layer's replays are also checked
against the oracle on the index they built."""

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_vertical_amd as msa
import oracle
from dynamic_sparse_attention_vertical_amd.graphs import StepGraph, decode_graph, layer_graph
from dynamic_sparse_attention_vertical_amd.layer import LayerPlan
from parity import compare_out, to_oracle_index
from synth import make_inputs, small_workload

pytestmark = pytest.mark.gpu

REPLAYS = 3


def inputs(hq, hkv, n, seed):
    x = make_inputs(small_workload(n_q_heads=hq, n_kv_heads=hkv, seq_len=n, seed=seed))
    return x["q"], x["k"], x["v"]


def index_arrays(idx):
    """The written part of the work lists: counts, then the entries below each
    count (slots past a count are left as they were)."""
    bm = torch.arange(idx.block_offset.shape[2], device=idx.block_offset.device) < idx.block_count[..., None]
    cm = torch.arange(idx.column_index.shape[2], device=idx.column_index.device) < idx.column_count[..., None]
    return [idx.block_count, idx.column_count, idx.block_offset[bm], idx.column_index[cm]]


def test_layer_chain_in_key_phases_replays_like_eager():
    """estimate_vs + build_index + sparse_prefill with 1024-key phases (three
    phase launches at 3000 keys, after the grouped walk) as one graph."""
    hq, hkv, n, kv, ks, phase = 8, 2, 64 * 46 + 37, 48, 160, 1024
    q0, k0, v0 = inputs(hq, hkv, n, seed=901)
    q, k, v = q0.cuda(), k0.cuda(), v0.cuda()
    plan = LayerPlan(hq, hkv, n, kv, ks, "cuda", q.dtype)
    aws = torch.empty(msa.sparse_prefill_workspace_bytes(hq, hkv, n, q.dtype, phase_keys=phase),
                      dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")

    def chain(p, o, l, ws):
        msa.estimate_vs(q, k, kv, ks, workspace=p.workspace, v_idx=p.v_idx, s_idx=p.s_idx)
        msa.build_index(p.v_idx, p.s_idx, n, out=p.index)
        msa.sparse_prefill(q, k, v, p.index, out=o, lse=l, phase_keys=phase, workspace=ws)
        return o, l

    g = StepGraph(lambda: chain(plan, out, lse, aws))
    ref_plan = LayerPlan(hq, hkv, n, kv, ks, "cuda", q.dtype)
    ref_ws = torch.empty_like(aws)
    for r in range(REPLAYS):
        qr, kr, vr = inputs(hq, hkv, n, seed=910 + r)
        q.copy_(qr), k.copy_(kr), v.copy_(vr)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [out.clone(), lse.clone(), plan.v_idx.clone(), plan.s_idx.clone()] + \
              [t.clone() for t in index_arrays(plan.index)]
        ref_out, ref_lse = chain(ref_plan, torch.empty_like(q), torch.empty_like(lse), ref_ws)
        torch.cuda.synchronize()
        ref = [ref_out, ref_lse, ref_plan.v_idx, ref_plan.s_idx] + index_arrays(ref_plan.index)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs from the eager chain"
        want, _ = oracle.attention_with_mask(qr, kr, vr, oracle.index_mask(to_oracle_index(plan.index), n))
        compare_out(got[0].float().cpu().numpy(), want, False, f"graph replay {r}")


def test_layer_graph_helper():
    hq, hkv, n, kv, ks = 4, 1, 64 * 15 + 5, 40, 100
    q0, k0, v0 = inputs(hq, hkv, n, seed=921)
    q, k, v = q0.cuda(), k0.cuda(), v0.cuda()
    g, plan = layer_graph(q, k, v, kv, ks)
    for r in range(REPLAYS):
        qr, kr, vr = inputs(hq, hkv, n, seed=930 + r)
        q.copy_(qr), k.copy_(kr), v.copy_(vr)
        torch.cuda.synchronize()
        out, lse = g.replay()
        torch.cuda.synchronize()
        got_out, got_lse = out.clone(), lse.clone()
        (ref_out, ref_lse), _ = msa.vertical_slash_layer(q, k, v, kv, ks, lse=True)
        torch.cuda.synchronize()
        assert torch.equal(got_out, ref_out) and torch.equal(got_lse, ref_lse), f"replay {r}"


@pytest.mark.parametrize("varlen", [False, True])
def test_decode_graph_replays_like_eager(varlen):
    hq, hkv, n, topk = 16, 4, 5000, 300
    _, k0, v0 = inputs(hq, hkv, n, seed=941)
    q = torch.empty((hq, 128), dtype=torch.bfloat16, device="cuda")
    k, v = k0.cuda(), v0.cuda()
    lens = torch.full((hkv,), n, dtype=torch.int32, device="cuda") if varlen else None
    g = decode_graph(q, k, v, topk, cache_lens=lens, lse=True, recovery=True)
    rng = np.random.default_rng(942)
    for r in range(REPLAYS):
        qr, kr, vr = inputs(hq, hkv, n, seed=950 + r)
        q.copy_(qr[:, -1]), k.copy_(kr), v.copy_(vr)
        if varlen:      # lengths change between replays; the graph reads them on the device
            lens.copy_(torch.from_numpy(rng.integers(0, n + 1, size=hkv).astype(np.int32)))
        torch.cuda.synchronize()
        outs = g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        ref = msa.decode_sparse(q, k, v, topk, lse=True, recovery=True, cache_lens=lens)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs"


def test_packed_chain_replays_like_eager():
    """estimate_vs_varlen + build_index_varlen + sparse_prefill_varlen (512-key
    phases) as one graph over a fixed capacity of rows and a host max_seqlen;
    the device cu_seqlens change between replays."""
    hq, hkv, rows, max_len, kv, ks, phase = 4, 1, 3000, 2000, 40, 120, 512
    splits = [[1000, 1200, 800], [2000, 500, 500], [700, 700, 1600]]

    def packed(lens, seed):
        parts = [inputs(hq, hkv, n, seed + i) for i, n in enumerate(lens)]
        return [torch.cat([p[j] for p in parts], dim=1).cuda() for j in range(3)]

    def offsets(lens):
        return torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)

    q, k, v = packed(splits[0], 960)
    cu = offsets(splits[0]).cuda()
    nb = msa.sparse_prefill_varlen_workspace_bytes(hq, hkv, rows, cu, max_len, q.dtype, phase_keys=phase)

    def chain(ws):
        v_idx, s_idx = msa.estimate_vs_varlen(q, k, cu, max_len, kv, ks)
        idx = msa.build_index_varlen(v_idx, s_idx, cu, max_len, hq, rows=rows)
        out, lse = msa.sparse_prefill_varlen(q, k, v, idx, cu, max_len, lse=True, workspace=ws,
                                             phase_keys=phase)
        return out, lse, v_idx, s_idx

    ws_graph = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    ws_eager = torch.empty_like(ws_graph)
    g = StepGraph(lambda: chain(ws_graph))
    for r, lens in enumerate(splits):
        qr, kr, vr = packed(lens, 970 + 10 * r)
        q.copy_(qr), k.copy_(kr), v.copy_(vr), cu.copy_(offsets(lens))
        torch.cuda.synchronize()
        got = [t.clone() for t in g.replay()]
        torch.cuda.synchronize()
        ref = chain(ws_eager)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {r} (lengths {lens}): output {i} differs from the eager chain"
