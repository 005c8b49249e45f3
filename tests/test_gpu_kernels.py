"""GPU parity of each kernel against the CPU oracle, at sizes the oracle
finishes in seconds that span several tiles (ragged block counts included).
Every call goes through the C ABI (via the ctypes binding)."""

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_vertical_amd as msa
import oracle
from parity import (check_band, compare_index, compare_lse, compare_out, to_oracle_index,
                    SCORE_RTOL)
from synth import make_inputs, small_workload

pytestmark = pytest.mark.gpu


def inputs(hq, hkv, n, seed=0, fp32=False, **kw):
    w = small_workload(n_q_heads=hq, n_kv_heads=hkv, seq_len=n, seed=seed,
                       dtypes=("fp32", "bf16") if fp32 else ("bf16",), **kw)
    x = make_inputs(w)
    if fp32:
        return w, x["q32"], x["k32"], x["v32"]
    return w, x["q"], x["k"], x["v"]


def cuda(*ts):
    return [t.to("cuda") for t in ts]


def random_sets(h, n, kv, ks, seed=0):
    r = np.random.default_rng(seed)
    v = np.stack([np.sort(r.choice(n, size=kv, replace=False)) for _ in range(h)]).astype(np.int32)
    s = np.stack([np.sort(r.choice(n, size=ks, replace=False)) for _ in range(h)]).astype(np.int32)
    return v, s


@pytest.mark.parametrize("hq,hkv,n,fp32", [(1, 1, 64, False), (4, 1, 256, False), (4, 2, 320, False),
                                           (8, 2, 1024, False), (2, 1, 320, True), (1, 1, 512, True),
                                           # GQA groups of 8, 3 and 6 (four, one and two heads per workgroup)
                                           (8, 1, 512, False), (6, 2, 384, False), (6, 1, 256, False)])
def test_dense_prefill(hq, hkv, n, fp32):
    w, q, k, v = inputs(hq, hkv, n, seed=n + hq, fp32=fp32)
    out, lse = msa.dense_prefill(*cuda(q, k, v), lse=True)
    ref, rlse = oracle.dense_attention(q, k, v)
    compare_out(out.float().cpu().numpy(), ref, fp32, "dense")
    compare_lse(lse.cpu().numpy(), rlse, "dense")


@pytest.mark.parametrize("hq,hkv,n,kv,ks,fp32", [(4, 1, 256, 7, 9, False), (4, 2, 640, 20, 30, False),
                                                 (2, 1, 1024, 100, 40, False), (2, 2, 384, 5, 200, False),
                                                 (2, 1, 320, 9, 13, True),
                                                 # GQA groups of 8 and 3
                                                 (8, 1, 512, 20, 30, False), (6, 2, 448, 15, 25, False)])
def test_sparse_prefill_given_index(hq, hkv, n, kv, ks, fp32):
    w, q, k, v = inputs(hq, hkv, n, seed=n, fp32=fp32)
    vi, si = random_sets(hq, n, kv, ks, seed=n + 1)
    ridx = oracle.build_index(vi, si, n)
    gidx = msa.alloc_index(hq, n, ridx.block_offset.shape[2], ridx.column_index.shape[2])
    gidx.block_count.copy_(torch.from_numpy(ridx.block_count))
    gidx.block_offset.copy_(torch.from_numpy(ridx.block_offset))
    gidx.column_count.copy_(torch.from_numpy(ridx.column_count))
    gidx.column_index.copy_(torch.from_numpy(ridx.column_index))
    out, lse = msa.sparse_prefill(*cuda(q, k, v), gidx, lse=True)
    ref, rlse = oracle.attention_with_mask(q, k, v, oracle.index_mask(ridx, n))
    compare_out(out.float().cpu().numpy(), ref, fp32, "sparse")
    compare_lse(lse.cpu().numpy(), rlse, "sparse")


@pytest.mark.parametrize("hq,hkv,n,kv,ks,phase,fp32", [
    (4, 2, 1216, 40, 60, 64, False),      # one phase per query block, ragged lists
    (2, 1, 1216, 100, 300, 320, False),   # phase edges inside block tiles (unaligned starts)
    (2, 1, 2048, 7, 2048, 512, False),    # every diagonal: blocks in every phase
    (2, 1, 640, 9, 13, 192, True),        # fp32; most phases hold nothing for most blocks
    (1, 1, 256, 1, 1, 64, False),         # a single diagonal and column
    # (the cases above hold fewer than 16 tiles per block and phase, so every
    # phase but a block's own leaves its tiles to the next: they check that
    # path.  Below, phases of 16 tiles carry the softmax state between launches)
    (2, 1, 4096, 9, 4096, 1024, False),   # every diagonal: 16 tiles in each full phase
    (1, 1, 4096, 5, 4096, 1024, True),    # the same in fp32
    (2, 1, 4096, 30, 1200, 1024, False),  # about 16 per phase: some carried, some left over
])
def test_sparse_prefill_phases(hq, hkv, n, kv, ks, phase, fp32):
    """Key phases (one launch per phase, state in the workspace) against the
    oracle and against one phase over the same lists."""
    w, q, k, v = inputs(hq, hkv, n, seed=n + phase, fp32=fp32)
    vi, si = random_sets(hq, n, kv, ks, seed=n + phase + 1)
    ridx = oracle.build_index(vi, si, n)
    gidx = msa.alloc_index(hq, n, ridx.block_offset.shape[2], ridx.column_index.shape[2])
    gidx.block_count.copy_(torch.from_numpy(ridx.block_count))
    gidx.block_offset.copy_(torch.from_numpy(ridx.block_offset))
    gidx.column_count.copy_(torch.from_numpy(ridx.column_count))
    gidx.column_index.copy_(torch.from_numpy(ridx.column_index))
    dt = torch.float32 if fp32 else torch.bfloat16
    need = msa.sparse_prefill_workspace_bytes(hq, hkv, n, dt, phase_keys=phase)
    assert need == hq * (n // 64) * (2 * (64 * 64 + 128) * 4 + 12)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")     # no initial contents assumed
    qs, ks_, vs = cuda(q, k, v)
    out, lse = msa.sparse_prefill(qs, ks_, vs, gidx, lse=True, phase_keys=phase, workspace=ws)
    ref, rlse = oracle.attention_with_mask(q, k, v, oracle.index_mask(ridx, n))
    compare_out(out.float().cpu().numpy(), ref, fp32, "sparse phases")
    compare_lse(lse.cpu().numpy(), rlse, "sparse phases")
    one, one_lse = msa.sparse_prefill(qs, ks_, vs, gidx, lse=True, phase_keys=n)
    compare_out(out.float().cpu().numpy(), one.float().cpu().numpy(), fp32, "phases vs one phase")
    compare_lse(lse.cpu().numpy(), one_lse.cpu().numpy(), "phases vs one phase")


def test_recall_from_lse():
    """Attention recall measured on the GPU as exp(lse_sparse - lse_dense)
    against the oracle's share of the dense softmax mass under the mask."""
    hq, hkv, n = 4, 2, 640
    w, q, k, v = inputs(hq, hkv, n, seed=17)
    vi, si = random_sets(hq, n, 12, 40, seed=18)
    idx = msa.build_index(*cuda(torch.from_numpy(vi), torch.from_numpy(si)), n)
    qs, ks_, vs = cuda(q, k, v)
    _, lse_s = msa.sparse_prefill(qs, ks_, vs, idx, lse=True)
    _, lse_d = msa.dense_prefill(qs, ks_, vs, lse=True)
    got = torch.exp(lse_s - lse_d).cpu().numpy()
    want = oracle.attention_recall(q, k, oracle.index_mask(to_oracle_index(idx), n))
    assert np.abs(got - want).max() <= 3e-4


# ------------------------------------------------ lengths not a multiple of 64

@pytest.mark.parametrize("hq,hkv,n,fp32", [(4, 2, 64 * 5 + 23, False), (1, 1, 37, False),
                                           (2, 1, 64 * 4 + 1, True), (8, 2, 1000, False)])
def test_dense_prefill_ragged(hq, hkv, n, fp32):
    w, q, k, v = inputs(hq, hkv, n, seed=n + 3, fp32=fp32)
    out, lse = msa.dense_prefill(*cuda(q, k, v), lse=True)
    ref, rlse = oracle.dense_attention(q, k, v)
    compare_out(out.float().cpu().numpy(), ref, fp32, "dense ragged")
    compare_lse(lse.cpu().numpy(), rlse, "dense ragged")


@pytest.mark.parametrize("hq,n,kv,ks,seed", [(2, 64 * 5 + 23, 7, 40, 0), (3, 1000, 50, 300, 1),
                                             (1, 37, 5, 20, 2)])
def test_build_index_ragged(hq, n, kv, ks, seed):
    vi, si = random_sets(hq, n, kv, ks, seed)
    ridx = oracle.build_index(vi, si, n)
    gidx = msa.build_index(*cuda(torch.from_numpy(vi), torch.from_numpy(si)), n)
    compare_index(gidx, ridx, "build_index ragged")


@pytest.mark.parametrize("hq,hkv,n,kv,ks,phase,fp32", [
    (4, 2, 64 * 7 + 23, 20, 60, 0, False),
    (2, 1, 64 * 9 + 63, 30, 100, 128, False),     # key phases, short last block
    (2, 1, 50, 5, 10, 0, False),                  # shorter than one block
    (2, 1, 64 * 3 + 40, 9, 13, 0, True),
])
def test_sparse_prefill_ragged(hq, hkv, n, kv, ks, phase, fp32):
    w, q, k, v = inputs(hq, hkv, n, seed=n + 5, fp32=fp32)
    vi, si = random_sets(hq, n, kv, ks, seed=n + 6)
    ridx = oracle.build_index(vi, si, n)
    gidx = msa.build_index(*cuda(torch.from_numpy(vi), torch.from_numpy(si)), n)
    compare_index(gidx, ridx, "index ragged")
    out, lse = msa.sparse_prefill(*cuda(q, k, v), gidx, lse=True, phase_keys=phase)
    ref, rlse = oracle.attention_with_mask(q, k, v, oracle.index_mask(ridx, n))
    compare_out(out.float().cpu().numpy(), ref, fp32, "sparse ragged")
    compare_lse(lse.cpu().numpy(), rlse, "sparse ragged")


def test_sparse_all_selected_equals_dense():
    n = 512
    w, q, k, v = inputs(4, 2, n, seed=3)
    all_ = torch.arange(n, dtype=torch.int32, device="cuda").expand(4, -1).contiguous()
    idx = msa.build_index(all_, all_, n)
    qs, ks_, vs = cuda(q, k, v)
    out = msa.sparse_prefill(qs, ks_, vs, idx)
    dense = msa.dense_prefill(qs, ks_, vs)
    ref, _ = oracle.dense_attention(q, k, v)
    compare_out(out.float().cpu().numpy(), ref, False, "all-selected")
    assert torch.equal(out, dense)      # same tiles in the same order: bitwise equal


def test_sparse_empty_rows_give_zero():
    n = 256
    w, q, k, v = inputs(1, 1, n, seed=4)
    vi = np.array([[n - 1]], np.int32)
    si = np.array([[n - 1]], np.int32)
    idx = msa.build_index(*cuda(torch.from_numpy(vi), torch.from_numpy(si)), n)
    out, lse = msa.sparse_prefill(*cuda(q, k, v), idx, lse=True)
    assert int(idx.block_count[0, 0]) == 0 and int(idx.column_count[0, 0]) == 0
    assert torch.all(out[0, :64] == 0)
    assert torch.all(torch.isneginf(lse[0, :64]))


@pytest.mark.parametrize("hq,n,kv,ks,seed", [(2, 256, 7, 9, 0), (3, 1024, 50, 300, 1), (2, 4096, 64, 256, 2),
                                             (1, 2048, 1, 2048, 3), (2, 16384, 1000, 13000, 4)])
def test_build_index_exact(hq, n, kv, ks, seed):
    vi, si = random_sets(hq, n, kv, ks, seed)
    ridx = oracle.build_index(vi, si, n)
    gidx = msa.build_index(*cuda(torch.from_numpy(vi), torch.from_numpy(si)), n)
    compare_index(gidx, ridx, "build_index")


@pytest.mark.parametrize("hq,n,kv,ks,cap_b,cap_c,seed", [
    (2, 448, 5, 10, None, None, 5),       # minimal caps 7 and 5: rows not 16-byte aligned
    (3, 1024, 40, 200, 37, 53, 6),        # caller caps above the minimum, odd
    (2, 2048, 30, 2000, 33, 30, 7),       # many blocks per item, odd row pitch
])
def test_build_index_odd_capacities(hq, n, kv, ks, cap_b, cap_c, seed):
    vi, si = random_sets(hq, n, kv, ks, seed)
    ridx = oracle.build_index(vi, si, n)
    mb, mc = msa.index_caps(n, kv, ks)
    out = msa.alloc_index(hq, n, cap_b or mb, cap_c or mc)
    gidx = msa.build_index(*cuda(torch.from_numpy(vi), torch.from_numpy(si)), n, out=out)
    compare_index(gidx, ridx, "build_index odd caps")


def test_build_index_many_columns():
    # more selected columns than the kernel stages in LDS
    vi, si = random_sets(2, 8192, 5000, 120, 8)
    ridx = oracle.build_index(vi, si, 8192)
    gidx = msa.build_index(*cuda(torch.from_numpy(vi), torch.from_numpy(si)), 8192)
    compare_index(gidx, ridx, "build_index many columns")


def test_build_index_a_shape():
    n = 64 * 120
    av, as_ = oracle.a_shape_sets(n, 128, 4096)
    ridx = oracle.build_index(av[None], as_[None], n)
    gidx = msa.build_index(*cuda(torch.from_numpy(av[None].copy()), torch.from_numpy(as_[None].copy())), n)
    compare_index(gidx, ridx, "a-shape")


@pytest.mark.parametrize("hq,hkv,n,fp32", [(4, 1, 256, False), (4, 2, 1024, False), (8, 2, 4096, False),
                                           (2, 1, 2048, True), (1, 1, 64, False), (4, 4, 8192, False),
                                           # lengths not a multiple of 64: keys tiled in a shifted frame
                                           (4, 1, 64 * 4 + 23, False), (2, 1, 64 * 9 + 1, True),
                                           (4, 2, 100, False), (1, 1, 127, False),
                                           (8, 2, 64 * 70 + 40, False),    # 18 key ranges
                                           # GQA groups above four: each wave serves a second q head
                                           # in a second pass over the range (8: both passes full;
                                           # 5: one wave busy in the second); 3: one wave idle
                                           (8, 1, 1024, False), (5, 1, 512, True), (6, 2, 64 * 6 + 17, False)])
def test_estimate_scores(hq, hkv, n, fp32):
    w, q, k, _ = inputs(hq, hkv, n, seed=n + 5, fp32=fp32)
    qs, ks_ = cuda(q, k)
    vsc = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    ssc = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    kv, ks = min(32, n), min(64, n)
    vi, si = msa.estimate_vs(qs, ks_, kv, ks, v_score=vsc, s_score=ssc)
    rv, rs = oracle.estimate_vs(q, k, last_q=64)
    for g, r, name in ((vsc, rv, "v"), (ssc, rs, "s")):
        g = g.cpu().numpy().astype(np.float64)
        bad = np.abs(g - r) > SCORE_RTOL * r + 1e-6
        assert not bad.any(), f"{name} scores: {bad.sum()} entries off, max {np.abs(g - r).max():.3e}"
    for h in range(hq):
        check_band(vi[h].cpu().numpy(), rv[h], kv, f"v_idx head {h}")
        check_band(si[h].cpu().numpy(), rs[h], ks, f"s_idx head {h}")


def test_topk_exact_ties_go_to_lower_index():
    """Identical key rows make every column reachable by all 64 rows score
    exactly the same (each column sums the same values in the same order), so
    the vertical selection must be the lowest indices.  Diagonal sums split at
    tile boundaries differently per offset, so the slash ties are only equal up
    to rounding: they are checked against the tie band."""
    n, hq = 2048, 2
    w, q, k, _ = inputs(hq, 1, n, seed=9)
    k = k[:, :1].expand(1, n, 128).contiguous()
    vi, si = msa.estimate_vs(*cuda(q, k), 100, 300)
    rv, rs = oracle.estimate_vs(q, k, last_q=64)
    for h in range(hq):
        assert vi[h].cpu().tolist() == list(range(100))
        check_band(si[h].cpu().numpy(), rs[h], 300, "tied slash")


def test_deterministic():
    n = 2048
    w, q, k, v = inputs(4, 1, n, seed=11)
    qs, ks_, vs = cuda(q, k, v)
    a, pa = msa.vertical_slash_layer(qs, ks_, vs, 64, 128)
    va, sa = pa.v_idx.clone(), pa.s_idx.clone()
    b, pb = msa.vertical_slash_layer(qs, ks_, vs, 64, 128)
    assert torch.equal(a, b) and torch.equal(va, pb.v_idx) and torch.equal(sa, pb.s_idx)


@pytest.mark.parametrize("fp32", [False, True])
def test_layer_end_to_end_small(fp32):
    n, hq, hkv, kv, ks = 2048, 4, 2, 48, 96
    w, q, k, v = inputs(hq, hkv, n, seed=21, fp32=fp32)
    out, plan = msa.vertical_slash_layer(*cuda(q, k, v), kv, ks)
    rv, rs = oracle.estimate_vs(q, k, last_q=64)
    vi, si = plan.v_idx.cpu().numpy(), plan.s_idx.cpu().numpy()
    for h in range(hq):
        check_band(vi[h], rv[h], kv, "v")
        check_band(si[h], rs[h], ks, "s")
    ridx = oracle.build_index(vi, si, n)
    compare_index(plan.index, ridx, "layer index")
    ref, _ = oracle.attention_with_mask(q, k, v, oracle.index_mask(ridx, n))
    compare_out(out.float().cpu().numpy(), ref, fp32, "layer")


@pytest.mark.parametrize("n,topk", [(1024, 3), (2048, 100), (640, 4),
                                    (64 * 5 + 23, 3), (100, 1), (64 * 10 + 1, 4),   # short last blocks
                                    (64 * 1100 + 5, 7)])   # two scoring chunks of query blocks
def test_estimate_bs(n, topk):
    hq, hkv = 4, 2
    w, q, k, v = inputs(hq, hkv, n, seed=n)
    idx = msa.estimate_bs(*cuda(q, k), topk)
    cnt, offs, scores = oracle.block_sparse_select(q, k, range(hq), topk=topk)
    bc = idx.block_count.cpu().numpy()
    bo = idx.block_offset.cpu().numpy()
    assert np.array_equal(bc, cnt)
    assert np.all(idx.column_count.cpu().numpy() == 0)
    nb = (n + 63) // 64
    for h in range(hq):
        for b in range(nb):
            kk = bc[h, b]
            c = bo[h, b, :kk] // 64
            assert np.all(bo[h, b, :kk] % 64 == 0) and np.all(np.diff(c) > 0)
            u = scores[h, b, : b + 1]
            pr = np.exp(u - u.max())
            pr /= pr.sum()
            check_band(c, pr, kk, f"bs head {h} block {b}")


@pytest.mark.parametrize("fp32", [False, True])
def test_explicit_softmax_scale(fp32):
    """A caller-given sm_scale (here 0.05, not 1/sqrt(128)) reaches every step:
    estimator scores, sparse and dense attention, against the oracle with the
    same scale."""
    hq, hkv, n, scale = 4, 2, 64 * 6 + 9, 0.05
    w, q, k, v = inputs(hq, hkv, n, seed=77, fp32=fp32)
    qs, ks_, vs = cuda(q, k, v)
    vsc = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    ssc = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    vi, si = msa.estimate_vs(qs, ks_, 16, 32, v_score=vsc, s_score=ssc, sm_scale=scale)
    rv, rs = oracle.estimate_vs(q, k, last_q=64, scale=scale)
    for g, r, name in ((vsc, rv, "v"), (ssc, rs, "s")):
        g = g.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(g - r) <= SCORE_RTOL * r + 1e-6), f"{name} scores with sm_scale"
    ridx = oracle.build_index(vi.cpu().numpy(), si.cpu().numpy(), n)
    out, lse = msa.sparse_prefill(qs, ks_, vs, msa.build_index(vi, si, n), lse=True, sm_scale=scale)
    ref, rlse = oracle.attention_with_mask(q, k, v, oracle.index_mask(ridx, n), scale=scale)
    compare_out(out.float().cpu().numpy(), ref, fp32, "sparse, sm_scale")
    compare_lse(lse.cpu().numpy(), rlse, "sparse, sm_scale")
    dout, dlse = msa.dense_prefill(qs, ks_, vs, lse=True, sm_scale=scale)
    dref, drlse = oracle.dense_attention(q, k, v, scale=scale)
    compare_out(dout.float().cpu().numpy(), dref, fp32, "dense, sm_scale")
    compare_lse(dlse.cpu().numpy(), drlse, "dense, sm_scale")


def test_estimate_bs_long_rows():
    """Block-sparse selection for query blocks past 15360 (rows of block
    scores longer than the LDS copy the selection keeps): 10^6 tokens, so
    15625 key blocks and a short last one.  Chosen blocks within the tie band
    of the oracle's row softmax, on rows both below and past 15360."""
    n, topk = 1_000_000, 100
    w = small_workload(n_q_heads=2, n_kv_heads=1, seq_len=n, seed=99, n_planted=3)
    x = make_inputs(w, device="cuda")
    q, k = x["q"], x["k"]
    idx = msa.estimate_bs(q, k, topk)
    torch.cuda.synchronize()
    nb = -(-n // 64)
    rows = [0, 99, 100, 5000, 15359, 15360, 15361, 15500, nb - 2, nb - 1]
    qc, kc = q.cpu(), k.cpu()
    for h in range(2):
        u = oracle.block_scores(qc, kc, h)
        bc = idx.block_count[h].cpu().numpy()
        bo = idx.block_offset[h].cpu().numpy()
        assert np.all(idx.column_count[h].cpu().numpy() == 0)
        for b in rows:
            kk = min(topk, b + 1)
            assert bc[b] == kk
            row = u[b, : b + 1]
            pr = np.exp(row - row.max())
            check_band(bo[b, :kk] // 64, pr / pr.sum(), kk, f"head {h} block {b}")
            assert np.all(bo[b, :kk] % 64 == 0)


@pytest.mark.parametrize("hq,hkv,n,fp32", [(8, 2, 64 * 40 + 17, False), (4, 2, 64 * 24, False),
                                           (3, 3, 64 * 20 + 1, False), (4, 1, 64 * 16 + 33, True)])
def test_sparse_grouped_walk(hq, hkv, n, fp32):
    """Lists that leave few keys out: every diagonal but two runs of 200 (so
    query blocks far enough down have two holes, partly filled by columns).
    The last head instead keeps the diagonals below n - 400, which leaves too
    much out for the late query blocks.  The q heads of a kv group whose lists
    all qualify run as one aligned-tile walk, the rest per head: against the
    oracle, and against the per-head kernel alone (one phase, no workspace)."""
    w, q, k, v = inputs(hq, hkv, n, seed=n + hq, fp32=fp32)
    rng = np.random.default_rng(n + 7)
    vi = np.sort(np.stack([rng.choice(n, 12, replace=False) for _ in range(hq)]), axis=1).astype(np.int32)
    rows = []
    for h in range(hq):
        if h == hq - 1:
            rows.append(np.arange(n - 400))
        else:
            a = 200 + 37 * h
            drop = np.r_[np.arange(a, a + 200), np.arange(a + 400, a + 600)]
            rows.append(np.setdiff1d(np.arange(n), drop))
    si = np.stack(rows).astype(np.int32)
    ridx = oracle.build_index(vi, si, n)
    gidx = msa.alloc_index(hq, n, ridx.block_offset.shape[2], ridx.column_index.shape[2])
    gidx.block_count.copy_(torch.from_numpy(ridx.block_count))
    gidx.block_offset.copy_(torch.from_numpy(ridx.block_offset))
    gidx.column_count.copy_(torch.from_numpy(ridx.column_count))
    gidx.column_index.copy_(torch.from_numpy(ridx.column_index))
    qs, ks_, vs = cuda(q, k, v)
    ws = walk_workspace(hq, hkv, n, qs.dtype)
    out, lse = msa.sparse_prefill(qs, ks_, vs, gidx, lse=True, phase_keys=512, workspace=ws)
    ref, rlse = oracle.attention_with_mask(q, k, v, oracle.index_mask(ridx, n))
    compare_out(out.float().cpu().numpy(), ref, fp32, "grouped walk")
    compare_lse(lse.cpu().numpy(), rlse, "grouped walk")
    one, one_lse = msa.sparse_prefill(qs, ks_, vs, gidx, lse=True, phase_keys=-(-n // 64) * 64)
    compare_out(out.float().cpu().numpy(), one.float().cpu().numpy(), fp32, "grouped vs per-head")
    compare_lse(lse.cpu().numpy(), one_lse.cpu().numpy(), "grouped vs per-head")
    # which units the walk took: the first query blocks (rows below 200, where
    # every head keeps all diagonals up to its last row) for every kv group;
    # never the last query block of the group holding the last head, whose
    # diagonals stop at n - 400 and leave hundreds of keys out
    marks = walk_marks(ws, hq, hkv, n)
    assert np.all(marks[:, :3] == 1), marks[:, :3]
    assert marks[-1, -1] == 0


def walk_workspace(hq, hkv, n, dtype, phase_keys=512):
    nbytes = msa.sparse_prefill_workspace_bytes(hq, hkv, n, dtype, phase_keys=phase_keys)
    assert nbytes > 0
    return torch.full((nbytes,), 0x7f, dtype=torch.uint8, device="cuda")


def walk_marks(ws, hq, hkv, n):
    """The grouped walk's marks, one per group of q heads sharing a unit and
    query block (1: the unit ran as one aligned-tile walk)."""
    torch.cuda.synchronize()
    m = msa.sparse_walk_marks(ws, hq, hkv, n, phase_keys=512).cpu().numpy()
    G = hq // hkv
    kh = 4 if G % 4 == 0 else (2 if G % 2 == 0 else 1)
    assert np.array_equal(m, np.repeat(m[::kh], kh, axis=0))      # one mark per unit
    return m[::kh]


@pytest.mark.parametrize("hq,hkv,fp32", [(4, 1, False), (4, 2, False), (4, 2, True)])
def test_sparse_columns_in_any_order(hq, hkv, fp32):
    """Column lists are sets: any order gives the same attention.  Per query
    block b >= 1 every head lists the aligned tiles 0..b except one, plus 10
    columns inside that tile; the even heads list them in descending order on
    odd query blocks.  The grouped walk reads columns in ascending order, so it
    must leave every unit holding such a list to the per-head kernel; it takes
    the others whose uncovered keys (64 - 10) are at most 1/8 of [0, r1], i.e.
    b = 0 and b >= 6."""
    n = 64 * 24
    nqb = n // 64
    w, q, k, v = inputs(hq, hkv, n, seed=77 + hq + hkv, fp32=fp32)
    rng = np.random.default_rng(5)
    bc = np.zeros((hq, nqb), np.int32)
    bo = np.full((hq, nqb, nqb), -1, np.int32)
    cc = np.zeros((hq, nqb), np.int32)
    ci = np.full((hq, nqb, 10), -1, np.int32)
    for h in range(hq):
        for b in range(nqb):
            hole = (7 * b + h) % (b + 1) if b > 0 else -1
            starts = [64 * t for t in range(b + 1) if t != hole]
            bc[h, b] = len(starts)
            bo[h, b, : len(starts)] = starts
            if hole >= 0:
                cols = np.sort(rng.choice(64, 10, replace=False)) + 64 * hole
                if h % 2 == 0 and b % 2 == 1:
                    cols = cols[::-1]
                cc[h, b] = 10
                ci[h, b] = cols
    ridx = oracle.IndexArrays(bc, bo, cc, ci)
    gidx = msa.alloc_index(hq, n, nqb, 10)
    for name in ("block_count", "block_offset", "column_count", "column_index"):
        getattr(gidx, name).copy_(torch.from_numpy(getattr(ridx, name)))
    qs, ks_, vs = cuda(q, k, v)
    ws = walk_workspace(hq, hkv, n, qs.dtype)
    out, lse = msa.sparse_prefill(qs, ks_, vs, gidx, lse=True, phase_keys=512, workspace=ws)
    ref, rlse = oracle.attention_with_mask(q, k, v, oracle.index_mask(ridx, n))
    compare_out(out.float().cpu().numpy(), ref, fp32, "columns in any order")
    compare_lse(lse.cpu().numpy(), rlse, "columns in any order")
    marks = walk_marks(ws, hq, hkv, n)
    b = np.arange(nqb)
    want = ((b == 0) | (b >= 6)) & (b % 2 == 0)
    np.testing.assert_array_equal(marks, np.broadcast_to(want.astype(np.int32), marks.shape))
    # the same lists in one phase (no walk, no workspace) agree
    one, one_lse = msa.sparse_prefill(qs, ks_, vs, gidx, lse=True, phase_keys=n)
    compare_out(one.float().cpu().numpy(), ref, fp32, "columns in any order, one phase")
    compare_lse(one_lse.cpu().numpy(), rlse, "columns in any order, one phase")
