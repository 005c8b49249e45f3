"""GPU checks of the README-style calls (vertical_slash_sparse_attention,
block_sparse_attention, streaming_forward) on batched [B, H, N, D] inputs:
each batch element against the oracle on the same index, and the batched call
against the per-element composition of the C-ABI steps."""

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_vertical_amd as msa
import oracle
from parity import compare_out, to_oracle_index
from synth import make_inputs, small_workload

pytestmark = pytest.mark.gpu


def batch_inputs(B, hq, hkv, n, seed):
    qs, ks, vs = [], [], []
    for bi in range(B):
        x = make_inputs(small_workload(n_q_heads=hq, n_kv_heads=hkv, seq_len=n, seed=seed + bi))
        qs.append(x["q"]), ks.append(x["k"]), vs.append(x["v"])
    return torch.stack(qs), torch.stack(ks), torch.stack(vs)


def test_vertical_slash_sparse_attention_batched():
    B, hq, hkv, n, kv, ks = 2, 4, 1, 1024, 40, 100
    q, k, v = batch_inputs(B, hq, hkv, n, seed=31)
    out = msa.vertical_slash_sparse_attention(q.cuda(), k.cuda(), v.cuda(), kv, ks)
    assert out.shape == q.shape
    for bi in range(B):
        ref_gpu, plan = msa.vertical_slash_layer(q[bi].cuda(), k[bi].cuda(), v[bi].cuda(), kv, ks)
        assert torch.equal(out[bi], ref_gpu)                  # same kernels, same index
        idx = to_oracle_index(plan.index)
        ref, _ = oracle.attention_with_mask(q[bi], k[bi], v[bi], oracle.index_mask(idx, n))
        compare_out(out[bi].float().cpu().numpy(), ref, False, f"vertical-slash batch {bi}")
    # a 3-D call is the same as one batch element
    one = msa.vertical_slash_sparse_attention(q[1].cuda(), k[1].cuda(), v[1].cuda(), kv, ks)
    assert torch.equal(one, out[1])


def test_block_sparse_attention_batched():
    B, hq, hkv, n, topk = 2, 4, 2, 640, 3
    q, k, v = batch_inputs(B, hq, hkv, n, seed=41)
    out = msa.block_sparse_attention(q.cuda(), k.cuda(), v.cuda(), topk)
    for bi in range(B):
        cnt, offs, _ = oracle.block_sparse_select(q[bi], k[bi], range(hq), topk=topk)
        idx = oracle.IndexArrays(cnt, offs, np.zeros_like(cnt), np.zeros((hq, n // 64, 0), np.int32))
        ref, _ = oracle.attention_with_mask(q[bi], k[bi], v[bi], oracle.index_mask(idx, n))
        compare_out(out[bi].float().cpu().numpy(), ref, False, f"block-sparse batch {bi}")


@pytest.mark.parametrize("init_num,window", [(128, 256), (64, 64), (1, 1000)])
def test_streaming_forward_batched(init_num, window):
    B, hq, hkv, n = 2, 4, 2, 1024
    q, k, v = batch_inputs(B, hq, hkv, n, seed=51)
    out = msa.streaming_forward(q.cuda(), k.cuda(), v.cuda(), init_num, window)
    vs_, ss_ = oracle.a_shape_sets(n, init_num, window)
    idx = oracle.build_index(np.tile(vs_, (hq, 1)), np.tile(ss_, (hq, 1)), n)
    M = oracle.index_mask(idx, n)
    for bi in range(B):
        ref, _ = oracle.attention_with_mask(q[bi], k[bi], v[bi], M)
        compare_out(out[bi].float().cpu().numpy(), ref, False, f"streaming batch {bi}")


def test_batch_layouts_fold_or_loop():
    """A contiguous batch runs as one problem of B*H heads; a batch whose
    heads are not evenly spaced across elements (here [H, B, N, D] memory
    seen as [B, H, N, D]) runs element by element.  Both give bitwise the
    same outputs as the per-element calls (at this length every element's
    estimate uses the same key ranges either way)."""
    B, hq, hkv, n = 3, 4, 2, 768
    q, k, v = batch_inputs(B, hq, hkv, n, seed=91)
    qp, kp, vp = (t.transpose(0, 1).contiguous().cuda().transpose(0, 1) for t in (q, k, v))
    assert qp.stride(0) != qp.shape[1] * qp.stride(1)           # not foldable
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    for call, args in ((msa.vertical_slash_sparse_attention, (24, 70)), (msa.block_sparse_attention, (3,)),
                       (msa.streaming_forward, (64, 128))):
        folded = call(qc, kc, vc, *args)
        looped = call(qp, kp, vp, *args)
        assert folded.shape == looped.shape == q.shape
        for bi in range(B):
            one = call(qc[bi], kc[bi], vc[bi], *args)
            assert torch.equal(folded[bi], one), (call.__name__, "folded", bi)
            assert torch.equal(looped[bi], one), (call.__name__, "looped", bi)


def test_api_ragged_lengths():
    """Lengths that are not a multiple of 64 through the whole path: estimate,
    index, sparse prefill; block-sparse; streaming."""
    hq, hkv, n = 4, 1, 64 * 11 + 29
    q, k, v = batch_inputs(1, hq, hkv, n, seed=61)
    out = msa.vertical_slash_sparse_attention(q.cuda(), k.cuda(), v.cuda(), 30, 90)
    ref_gpu, plan = msa.vertical_slash_layer(q[0].cuda(), k[0].cuda(), v[0].cuda(), 30, 90)
    assert torch.equal(out[0], ref_gpu)
    ref, _ = oracle.attention_with_mask(q[0], k[0], v[0], oracle.index_mask(to_oracle_index(plan.index), n))
    compare_out(out[0].float().cpu().numpy(), ref, False, "vertical-slash ragged")
    out = msa.block_sparse_attention(q.cuda(), k.cuda(), v.cuda(), 3)
    cnt, offs, _ = oracle.block_sparse_select(q[0], k[0], range(hq), topk=3)
    nb = (n + 63) // 64
    idx = oracle.IndexArrays(cnt, offs, np.zeros_like(cnt), np.zeros((hq, nb, 0), np.int32))
    ref, _ = oracle.attention_with_mask(q[0], k[0], v[0], oracle.index_mask(idx, n))
    compare_out(out[0].float().cpu().numpy(), ref, False, "block-sparse ragged")
    out = msa.streaming_forward(q.cuda(), k.cuda(), v.cuda(), 64, 200)
    vs_, ss_ = oracle.a_shape_sets(n, 64, 200)
    sidx = oracle.build_index(np.tile(vs_, (hq, 1)), np.tile(ss_, (hq, 1)), n)
    ref, _ = oracle.attention_with_mask(q[0], k[0], v[0], oracle.index_mask(sidx, n))
    compare_out(out[0].float().cpu().numpy(), ref, False, "streaming ragged")


def test_batched_shape_errors():
    q = torch.zeros((2, 4, 256, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(msa.MsaError):
        msa.vertical_slash_sparse_attention(q, q[:, :1, :, :][0], q[:, :1], 8, 8)
    with pytest.raises(msa.MsaError):
        msa.streaming_forward(q, q[:, :1], q[:, :1], 0, 64)


def _packed_inputs(hq, hkv, lens, seed):
    parts = [batch_inputs(1, hq, hkv, n, seed=seed + i) for i, n in enumerate(lens)]
    q = torch.cat([p[0][0] for p in parts], dim=1).cuda()
    k = torch.cat([p[1][0] for p in parts], dim=1).cuda()
    v = torch.cat([p[2][0] for p in parts], dim=1).cuda()
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    return q, k, v, cu


def test_strided_views_match_contiguous():
    """A sequence that is a slice of packed [heads, total, 128] tensors (head
    stride = total rows) gives bitwise the same results as a contiguous copy,
    in every entry point."""
    hq, hkv, lens = 4, 2, [300, 64 * 5, 777]
    q, k, v, cu = _packed_inputs(hq, hkv, lens, seed=71)
    a, b = cu[2], cu[3]
    qv, kv_, vv = q[:, a:b], k[:, a:b], v[:, a:b]
    qc, kc, vc = qv.contiguous(), kv_.contiguous(), vv.contiguous()
    n = b - a
    o1, l1 = msa.dense_prefill(qv, kv_, vv, lse=True)
    o2, l2 = msa.dense_prefill(qc, kc, vc, lse=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    vi1, si1 = msa.estimate_vs(qv, kv_, 30, 80)
    vi2, si2 = msa.estimate_vs(qc, kc, 30, 80)
    assert torch.equal(vi1, vi2) and torch.equal(si1, si2)
    idx = msa.build_index(vi1, si1, n)
    o1, l1 = msa.sparse_prefill(qv, kv_, vv, idx, lse=True, phase_keys=128)
    o2, l2 = msa.sparse_prefill(qc, kc, vc, idx, lse=True, phase_keys=128)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    b1 = msa.estimate_bs(qv, kv_, 3)
    b2 = msa.estimate_bs(qc, kc, 3)
    assert torch.equal(b1.block_count, b2.block_count)
    live = torch.arange(b1.cap_blocks, device="cuda")[None, None, :] < b1.block_count[:, :, None]
    assert torch.equal(b1.block_offset[live], b2.block_offset[live])       # entries past a count are unspecified


def test_packed_batch_calls():
    """cu_seqlens: each packed sequence equals the same call on that sequence alone."""
    hq, hkv, lens = 4, 1, [200, 64 * 6, 641]
    q, k, v, cu = _packed_inputs(hq, hkv, lens, seed=81)
    for call, args in ((msa.vertical_slash_sparse_attention, (30, 90)), (msa.block_sparse_attention, (3,)),
                       (msa.streaming_forward, (64, 128))):
        out = call(q, k, v, *args, cu_seqlens=cu)
        for i in range(len(lens)):
            a, b = cu[i], cu[i + 1]
            one = call(q[:, a:b].contiguous(), k[:, a:b].contiguous(), v[:, a:b].contiguous(),
                       *[min(x, b - a) for x in args])
            assert torch.equal(out[:, a:b], one), (call.__name__, i)
    with pytest.raises(msa.MsaError):
        msa.streaming_forward(q, k, v, 64, 128, cu_seqlens=[0, 100, 50, q.shape[1]])


def test_index_rows_not_16_byte_aligned():
    """Work lists whose block_offset starts 4 bytes into an allocation (rows
    4-byte aligned only) take the element-wise stores and hold the same lists."""
    hq, n, kv, ks = 2, 64 * 40 + 9, 24, 40
    g = torch.Generator().manual_seed(91)
    vi = torch.sort(torch.randperm(n, generator=g)[:kv])[0].repeat(hq, 1).int().cuda()
    si = torch.sort(torch.randperm(n, generator=g)[:ks])[0].repeat(hq, 1).int().cuda()
    ref = msa.build_index(vi, si, n)
    cb, cc = ref.cap_blocks, ref.cap_cols
    assert cb % 4 == 0
    nqb = ref.block_count.shape[1]
    buf = torch.full((hq * nqb * cb + 1,), -7, dtype=torch.int32, device="cuda")
    odd = msa.IndexTensors(torch.empty_like(ref.block_count), buf[1:].view(hq, nqb, cb),
                           torch.empty_like(ref.column_count), torch.empty_like(ref.column_index))
    assert odd.block_offset.data_ptr() % 16 == 4
    msa.build_index(vi, si, n, out=odd)
    assert torch.equal(odd.block_count, ref.block_count) and torch.equal(odd.column_count, ref.column_count)
    live = torch.arange(cb, device="cuda")[None, None, :] < ref.block_count[:, :, None]
    assert torch.equal(odd.block_offset[live], ref.block_offset[live])
    assert int(buf[0]) == -7                                    # nothing written before the array
    livec = torch.arange(cc, device="cuda")[None, None, :] < ref.column_count[:, :, None]
    assert torch.equal(odd.column_index[livec], ref.column_index[livec])


def test_side_stream_calls():
    """Calls on a side stream (their temporaries allocated on it, torch ops
    ordered with the launches) give the default stream's results."""
    hq, hkv, n = 4, 2, 1024 + 17
    x = make_inputs(small_workload(n_q_heads=hq, n_kv_heads=hkv, seq_len=n, seed=97))
    q, k, v = x["q"].cuda(), x["k"].cuda(), x["v"].cuda()
    ref = [msa.vertical_slash_sparse_attention(q, k, v, 30, 90), msa.block_sparse_attention(q, k, v, 3),
           msa.streaming_forward(q, k, v, 64, 128), msa.dense_prefill(q, k, v)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(torch.cuda.Stream()):     # a third stream current: the calls must not use it
        got = [msa.vertical_slash_sparse_attention(q, k, v, 30, 90, stream=side),
               msa.block_sparse_attention(q, k, v, 3, stream=side),
               msa.streaming_forward(q, k, v, 64, 128, stream=side), msa.dense_prefill(q, k, v, stream=side)]
    side.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
