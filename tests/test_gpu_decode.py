"""GPU parity of the decode-side top-k attention (msa_decode_sparse) against
the float64 oracle (oracle.decode_sparse_attention): the selected key sets
exactly, except keys whose oracle score lies within 1e-4 of the k-th largest
(the fp32 / fp64 tie band); outputs, lse and the kept share of the attention
mass on the GPU's own sets at the graded tolerances.  Caches of different lengths
(msa_decode_sparse_varlen) are checked the same way against the oracle with
the same lengths, with NaN in every row past a length.  Every call goes
through the C ABI."""

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_vertical_amd as msa
import oracle
from parity import compare_out
from synth import DECODE_WORKLOADS, WORKLOADS, make_decode_inputs, make_inputs, small_workload

pytestmark = pytest.mark.gpu

SCORE_BAND = 1e-4     # absolute, on sm_scale * <q, k>
LSE_ATOL = 1e-4
REC_ATOL = 1e-5


def cache(hq, hkv, n, seed, fp32=False):
    """Decode inputs of the synthetic recipe: the caches are a prefill's K and
    V, the decode queries its last query row."""
    w = small_workload(n_q_heads=hq, n_kv_heads=hkv, seq_len=n, seed=seed,
                       dtypes=("fp32", "bf16") if fp32 else ("bf16",))
    x = make_inputs(w)
    sfx = "32" if fp32 else ""
    return x["q" + sfx][:, -1].contiguous(), x["k" + sfx], x["v" + sfx]


def check_sets(idx, s, topk, what):
    """idx [Hq, topk] ascending; every key scoring above the k-th largest
    (by more than the band) chosen, none scoring below it by more."""
    for h in range(s.shape[0]):
        got = idx[h]
        assert len(np.unique(got)) == topk and np.all(np.diff(got) > 0), f"{what} h{h}: not ascending distinct"
        kth = np.sort(s[h])[::-1][topk - 1]
        must = np.nonzero(s[h] > kth + SCORE_BAND)[0]
        assert np.isin(must, got).all(), f"{what} h{h}: a key above the band is missing"
        assert np.all(s[h][got] >= kth - SCORE_BAND), f"{what} h{h}: a key below the band was chosen"


def check_decode(q, k, v, topk, fp32, what, given=None):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    if given is None:
        out, idx, lse, rec = msa.decode_sparse(qd, kd, vd, topk, lse=True, recovery=True)
    else:
        out, idx, lse, rec = msa.decode_sparse(qd, kd, vd, topk, idx=given.cuda(), given=True, lse=True,
                                               recovery=True)
    idx = idx.cpu().numpy()
    s = oracle.decode_scores(q, k)
    if given is None:
        check_sets(idx, s, topk, what)
    else:
        np.testing.assert_array_equal(idx, given.numpy())
    ro, rl, rr, _ = oracle.decode_sparse_attention(q, k, v, topk, idx=idx)
    compare_out(out.float().cpu().numpy(), ro, fp32, what)
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=0, atol=LSE_ATOL, err_msg=what)
    np.testing.assert_allclose(rec.cpu().numpy(), rr, rtol=0, atol=REC_ATOL, err_msg=what)
    return out, idx, rec.cpu().numpy()


@pytest.mark.parametrize("hq,hkv,n,topk,fp32", [
    (4, 1, 1000, 100, False),
    (8, 2, 4096 + 37, 300, False),     # ragged: the last score chunk and top-k slice are partial
    (6, 2, 2500, 64, False),           # GQA group of 3
    (16, 1, 2048, 128, False),         # group of 16: two scoring passes over K
    (2, 2, 777, 1, False),             # one key
    (2, 1, 513, 513, False),           # every key: dense decode attention
    (4, 2, 1500, 200, True),           # fp32
    (128, 32, 3000 + 5, 200, False),   # 128 rows: one top-k workgroup per row
    (256, 64, 1100, 1100, False),      # every key, one workgroup per row
    (128, 32, 20000, 15000, False),    # one workgroup per row, more entries than it stages in LDS
    (8, 2, 70, 9, False),              # a cache shorter than one scoring chunk
    (128, 32, 101, 17, False),         # the same with one workgroup per row
])
def test_decode_topk(hq, hkv, n, topk, fp32):
    q, k, v = cache(hq, hkv, n, seed=n + topk, fp32=fp32)
    _, _, rec = check_decode(q, k, v, topk, fp32, f"decode {hq}/{hkv} n={n} k={topk}")
    if topk == n:
        np.testing.assert_allclose(rec, 1.0, atol=REC_ATOL)


def test_decode_static_set_keeps_less():
    """A static choice (the first 16 keys and the last topk - 16) against the
    dynamic top-k of the same size: the dynamic set keeps at least as much of
    every head's attention mass (the top-k maximise the kept share), and both
    match the oracle."""
    hq, hkv, n, topk = 8, 2, 3000, 200
    q, k, v = cache(hq, hkv, n, seed=9)
    _, _, rec_dyn = check_decode(q, k, v, topk, False, "dynamic")
    static = np.r_[np.arange(16), np.arange(n - (topk - 16), n)].astype(np.int32)
    given = torch.from_numpy(np.tile(static, (hq, 1)))
    _, _, rec_st = check_decode(q, k, v, topk, False, "static", given=given)
    assert np.all(rec_dyn >= rec_st - REC_ATOL)


def test_decode_strided_cache_and_batch():
    """Caches inside a longer buffer (rows between heads = the buffer's
    length), and a batch of two sequences folded into the heads."""
    hq, hkv, n, cap, topk = 4, 2, 900, 1200, 50
    qa, ka, va = cache(hq, hkv, n, seed=21)
    qb, kb, vb = cache(hq, hkv, n, seed=22)
    kbuf = torch.zeros((2 * hkv, cap, 128), dtype=ka.dtype)
    vbuf = torch.zeros((2 * hkv, cap, 128), dtype=va.dtype)
    kbuf[:hkv, :n], kbuf[hkv:, :n] = ka, kb
    vbuf[:hkv, :n], vbuf[hkv:, :n] = va, vb
    q = torch.cat([qa, qb])
    out, idx, lse, rec = msa.decode_sparse(q.cuda(), kbuf.cuda()[:, :n], vbuf.cuda()[:, :n], topk, lse=True,
                                           recovery=True)
    for part, (qq, kk, vv) in enumerate(((qa, ka, va), (qb, kb, vb))):
        rows = slice(part * hq, (part + 1) * hq)
        i = idx[rows].cpu().numpy()
        check_sets(i, oracle.decode_scores(qq, kk), topk, f"batch {part}")
        ro, rl, rr, _ = oracle.decode_sparse_attention(qq, kk, vv, topk, idx=i)
        compare_out(out[rows].float().cpu().numpy(), ro, False, f"batch {part}")
        np.testing.assert_allclose(lse[rows].cpu().numpy(), rl, atol=LSE_ATOL)
        np.testing.assert_allclose(rec[rows].cpu().numpy(), rr, atol=REC_ATOL)


def test_decode_128k_cache():
    """The 128K workload's caches (32 q heads, 8 kv heads, 131,072 keys), the
    top-1000 keys per head, every head against the oracle."""
    w = WORKLOADS["llama3_8b_128k"]
    x = make_inputs(w, device="cuda")
    q = x["q"][:, -1].contiguous()
    out, idx, lse, rec = msa.decode_sparse(q, x["k"], x["v"], 1000, lse=True, recovery=True)
    torch.cuda.synchronize()
    qc, kc, vc = q.cpu(), x["k"].cpu(), x["v"].cpu()
    i = idx.cpu().numpy()
    check_sets(i, oracle.decode_scores(qc, kc), 1000, "128K")
    ro, rl, rr, _ = oracle.decode_sparse_attention(qc, kc, vc, 1000, idx=i)
    compare_out(out.float().cpu().numpy(), ro, False, "128K")
    np.testing.assert_allclose(lse.cpu().numpy(), rl, atol=LSE_ATOL)
    np.testing.assert_allclose(rec.cpu().numpy(), rr, atol=REC_ATOL)
    print(f"128K decode: kept share of the attention mass, top-1000: mean {rr.mean():.3f}, min {rr.min():.3f}")


def tie_cache(hq, hkv, n, seed):
    """Keys at seven score levels, key j at level j % 7, every q head equal
    to the direction of its kv head's keys: keys of one level score exactly
    alike (identical rows), levels lie far apart."""
    g = torch.Generator().manual_seed(seed)
    w = torch.randn(hkv, 128, generator=g)
    levels = torch.tensor([-1.5, -1.0, -0.5, 0.0, 0.5, 1.0, 1.5])
    c = levels[torch.arange(n) % 7]
    k = (c[None, :, None] * w[:, None, :]).to(torch.bfloat16)
    q = w.repeat_interleave(hq // hkv, 0).to(torch.bfloat16)
    v = torch.randn(hkv, n, 128, generator=g).to(torch.bfloat16)
    return q, k, v


@pytest.mark.parametrize("hq,hkv", [(8, 2), (128, 32)])      # slices across the chip; one workgroup per row
def test_decode_topk_exact_ties(hq, hkv):
    """The top level's 300 keys, then the 17 lowest-index keys of the next
    level, whose 300 keys all tie: the selected sets equal the oracle's
    exactly (ties go to the lower index)."""
    n, topk = 2100, 300 + 17
    q, k, v = tie_cache(hq, hkv, n, seed=5)
    out, idx, lse, rec = msa.decode_sparse(q.cuda(), k.cuda(), v.cuda(), topk, lse=True, recovery=True)
    ro, rl, rr, ref_idx = oracle.decode_sparse_attention(q, k, v, topk)
    expect = np.sort(np.r_[np.arange(6, n, 7), np.arange(5, 5 + 7 * 17, 7)])
    assert np.array_equal(ref_idx[0], expect)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    compare_out(out.float().cpu().numpy(), ro, False, "ties")
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=0, atol=LSE_ATOL)


def varlen_cache(hq, hkv, n, lens, seed, fp32=False):
    """The recipe's caches with kv head g holding lens[g] keys: the rows past
    each length are NaN, so a kernel that read one would show it."""
    q, k, v = cache(hq, hkv, n, seed, fp32)
    for g, L in enumerate(lens):
        k[g, L:] = float("nan")
        v[g, L:] = float("nan")
    return q, k, v


def check_decode_varlen(q, k, v, lens, topk, fp32, what, given=None, per_sequence=None):
    """Against the oracle with the same cache lengths: a head whose cache
    holds at least topk keys selects within it (tie band as above); a shorter
    one selects all its keys and then the lowest positions past its end."""
    hq, hkv = q.shape[0], k.shape[0]
    G = hq // hkv
    lens_arg = torch.tensor(per_sequence if per_sequence is not None else lens, dtype=torch.int32).cuda()
    kw = dict(lse=True, recovery=True, cache_lens=lens_arg)
    if given is not None:
        kw.update(idx=given.cuda(), given=True)
    out, idx, lse, rec = msa.decode_sparse(q.cuda(), k.cuda(), v.cuda(), topk, **kw)
    idx = idx.cpu().numpy()
    s = oracle.decode_scores(q, k)
    for h in range(hq):
        L = int(lens[h // G])
        if given is not None:
            np.testing.assert_array_equal(idx[h], given[h].numpy())
        elif L >= topk:
            assert np.all(idx[h] < L), f"{what} h{h}: a key past the cache's end"
            check_sets(idx[h:h + 1], s[h:h + 1, :L], topk, f"{what} h{h}")
        else:
            np.testing.assert_array_equal(idx[h], np.arange(topk), err_msg=f"{what} h{h}")
    ro, rl, rr, _ = oracle.decode_sparse_attention(q, k, v, topk, idx=idx, cache_len=np.asarray(lens))
    o = out.float().cpu().numpy()
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    compare_out(o, ro, fp32, what)
    lg = lse.cpu().numpy()
    np.testing.assert_array_equal(np.isneginf(lg), np.isneginf(rl), err_msg=what)
    fin = np.isfinite(rl)
    np.testing.assert_allclose(lg[fin], rl[fin], rtol=0, atol=LSE_ATOL, err_msg=what)
    np.testing.assert_allclose(rec.cpu().numpy(), rr, rtol=0, atol=REC_ATOL, err_msg=what)


@pytest.mark.parametrize("hq,hkv,n,topk,lens,fp32", [
    (8, 2, 3000, 200, (1234, 3000), False),           # one cache shorter than the capacity
    (8, 2, 3001, 200, (1235, 3001), False),           # rows of keys not 16-byte aligned
    (8, 4, 2500, 100, (0, 1, 99, 100), False),        # empty, one key, fewer than topk, exactly topk
    (4, 2, 1500, 50, (640, 1013), True),              # fp32: two steps per chunk; the cache ends on a step
    (4, 2, 1500, 50, (700, 0), True),
    (8, 2, 70, 9, (3, 69), False),                    # caches shorter than one scoring chunk
])
def test_decode_varlen(hq, hkv, n, topk, lens, fp32):
    q, k, v = varlen_cache(hq, hkv, n, lens, seed=n + topk, fp32=fp32)
    check_decode_varlen(q, k, v, lens, topk, fp32, f"varlen {hq}/{hkv} n={n} k={topk} lens={lens}")


@pytest.mark.parametrize("n", [5000, 8000])
def test_decode_varlen_rows_topk(n):
    """128 q heads (one top-k workgroup per row) over 32 caches of assorted
    lengths: empty, below, at and above topk, on and off the 256-key step,
    and full.  At capacity 8000 a short cache leaves more tied positions past
    its end than the select stages in LDS."""
    hq, hkv, topk = 128, 32, 300
    rng = np.random.default_rng(11)
    lens = rng.integers(0, n + 1, hkv)
    lens[:10] = (0, 1, 299, 300, 301, 256, 257, n - 1, n, 4096)
    q, k, v = varlen_cache(hq, hkv, n, lens, seed=31)
    check_decode_varlen(q, k, v, lens, topk, False, f"varlen rows n={n}")


def test_decode_varlen_given_keys_and_batch_lengths():
    """Given keys at or past a cache's end carry no weight; lengths given per
    sequence of a folded batch serve each sequence's kv heads."""
    hq, hkv, n, topk = 8, 2, 1000, 64
    lens = (500, 1000)
    q, k, v = varlen_cache(hq, hkv, n, lens, seed=41)
    given = torch.from_numpy(np.tile(np.r_[np.arange(0, 960, 30), np.arange(470, 534)][:topk].astype(np.int32),
                                     (hq, 1)))
    given = torch.sort(given, dim=1).values.contiguous()
    check_decode_varlen(q, k, v, lens, topk, False, "varlen given", given=given)
    # two sequences of two kv heads each, one length per sequence
    hq, hkv = 8, 4
    lens = (600, 600, 900, 900)
    q, k, v = varlen_cache(hq, hkv, n, lens, seed=42)
    check_decode_varlen(q, k, v, lens, 100, False, "varlen per sequence", per_sequence=(600, 900))


def test_decode_varlen_many_sequences():
    """Eight sequences (16 q / 2 kv heads each, one top-k workgroup per row)
    with capacity 100,000 and lengths from 1,000 to 100,000, top-1000."""
    n, topk = 100_000, 1000
    rng = np.random.default_rng(12)
    seq = rng.integers(1000, n + 1, 8)
    seq[0], seq[1] = n, 1000
    lens = np.repeat(seq, 2)
    w = small_workload(n_q_heads=16, n_kv_heads=2, seq_len=n, seed=77)
    x = make_inputs(w)
    q = x["q"][:, -1].repeat(8, 1).contiguous()
    k = x["k"].repeat(8, 1, 1)
    v = x["v"].repeat(8, 1, 1)
    for g, L in enumerate(lens):
        k[g, L:] = float("nan")
        v[g, L:] = float("nan")
    check_decode_varlen(q, k, v, lens, topk, False, "varlen 8 x 100K", per_sequence=seq)


def test_decode_varlen_workload_sampled():
    """The benchmark's variable-length decode batch as the benchmark runs it
    (8 sequences of 32 q / 8 kv heads, capacity 131,072, 4,096 to 131,072
    tokens, top-1000): three sequences' heads against the oracle on caches
    cut to their lengths."""
    dw = DECODE_WORKLOADS["llama3_8b_decode_varlen"]
    x = make_decode_inputs(dw, device="cuda")
    out, idx, lse, rec = msa.decode_sparse(x["q"], x["k"], x["v"], dw.topk, lse=True, recovery=True,
                                           cache_lens=x["cache_lens"])
    torch.cuda.synchronize()
    for b in (0, 5, 7):
        hs, gs, L = slice(b * 32, (b + 1) * 32), slice(b * 8, (b + 1) * 8), dw.length(b)
        q, k, v = x["q"][hs].cpu(), x["k"][gs, :L].cpu(), x["v"][gs, :L].cpu()
        i = idx[hs].cpu().numpy()
        what = f"varlen workload sequence {b} ({L} tokens)"
        assert np.all(i < L), what
        check_sets(i, oracle.decode_scores(q, k), dw.topk, what)
        ro, rl, rr, _ = oracle.decode_sparse_attention(q, k, v, dw.topk, idx=i)
        compare_out(out[hs].float().cpu().numpy(), ro, False, what)
        np.testing.assert_allclose(lse[hs].cpu().numpy(), rl, atol=LSE_ATOL, err_msg=what)
        np.testing.assert_allclose(rec[hs].cpu().numpy(), rr, atol=REC_ATOL, err_msg=what)


def test_decode_varlen_lengths_clamped():
    """Cache lengths outside [0, capacity] are clamped on the device: a
    negative length is an empty cache, one past the capacity the full one."""
    hq, hkv, n, topk = 8, 2, 900, 50
    q, k, v = cache(hq, hkv, n, seed=51)
    lens_dev = torch.tensor([-3, 1 << 30], dtype=torch.int32).cuda()
    out, idx, lse, rec = msa.decode_sparse(q.cuda(), k.cuda(), v.cuda(), topk, lse=True, recovery=True,
                                           cache_lens=lens_dev)
    i = idx.cpu().numpy()
    ro, rl, rr, _ = oracle.decode_sparse_attention(q, k, v, topk, idx=i, cache_len=np.array([0, n]))
    np.testing.assert_array_equal(i[:4], np.tile(np.arange(topk), (4, 1)))     # empty: the first positions
    check_sets(i[4:], oracle.decode_scores(q[4:], k[1:]), topk, "full cache")
    compare_out(out.float().cpu().numpy(), ro, False, "clamped lengths")
    lg = lse.cpu().numpy()
    assert np.isneginf(lg[:4]).all() and np.isfinite(lg[4:]).all()
    np.testing.assert_allclose(lg[4:], rl[4:], atol=LSE_ATOL)
    np.testing.assert_allclose(rec.cpu().numpy(), rr, atol=REC_ATOL)
