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
