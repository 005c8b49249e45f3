"""GPU parity of the packed variable-length calls (msa_estimate_vs_varlen,
msa_build_index_varlen, msa_sparse_prefill_varlen, msa_dense_prefill_varlen):
every sequence of a packed [heads, total, 128] batch against the float64
oracle on that sequence's own rows.

Per sequence: the vertical and slash sets within the 1e-3 tie band of the
oracle's scores (a sequence of at most k tokens: all its positions, then the
positions past its end); the work lists bit-exact against the oracle's
builder on the GPU's sets; the sparse and dense outputs and lse at the graded
tolerances (whole sequences where the oracle's mask fits, sampled query
blocks for the long one).  Sequences shorter than the 64-row window are
estimated with all their rows as the window.  Every call goes through the C
ABI."""

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_vertical_amd as msa
import oracle
from parity import check_band, compare_index, compare_lse, compare_out
from synth import make_inputs, small_workload

pytestmark = pytest.mark.gpu


def packed_inputs(hq, hkv, lens, seed, fp32=False):
    """Sequences of the synthetic recipe concatenated along the rows."""
    parts = []
    for i, n in enumerate(lens):
        w = small_workload(n_q_heads=hq, n_kv_heads=hkv, seq_len=n, seed=seed + i,
                           dtypes=("fp32", "bf16") if fp32 else ("bf16",))
        x = make_inputs(w)
        sfx = "32" if fp32 else ""
        parts.append((x["q" + sfx], x["k" + sfx], x["v" + sfx]))
    q, k, v = (torch.cat([p[i] for p in parts], dim=1).contiguous() for i in range(3))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64).tolist()
    return q, k, v, cu


def run_varlen(q, k, v, cu, kv, ks, phase_keys=0):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    max_len = max(b - a for a, b in zip(cu, cu[1:]))
    kv, ks = min(kv, max_len), min(ks, max_len)
    v_idx, s_idx = msa.estimate_vs_varlen(qd, kd, cu_d, max_len, kv, ks)
    idx = msa.build_index_varlen(v_idx, s_idx, cu_d, max_len, q.shape[0], rows=q.shape[1])
    nb = msa.sparse_prefill_varlen_workspace_bytes(q.shape[0], k.shape[0], q.shape[1], cu_d, max_len, q.dtype,
                                                   phase_keys=phase_keys)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    out, lse = msa.sparse_prefill_varlen(qd, kd, vd, idx, cu_d, max_len, lse=True, workspace=ws,
                                         phase_keys=phase_keys)
    dout, dlse = msa.dense_prefill_varlen(qd, kd, vd, cu_d, max_len, lse=True)
    torch.cuda.synchronize()
    nseq = len(cu) - 1
    marks = msa.sparse_walk_marks(ws, nseq * q.shape[0], nseq * k.shape[0], max_len, q.dtype,
                                  phase_keys=phase_keys) if nb else None
    return dict(v_idx=v_idx.cpu().numpy(), s_idx=s_idx.cpu().numpy(), idx=idx, out=out, lse=lse, dout=dout,
                dlse=dlse, kv=kv, ks=ks, marks=marks)


def sequence_index(idx, rows, nqb):
    return msa.IndexTensors(idx.block_count[rows, :nqb], idx.block_offset[rows, :nqb],
                            idx.column_count[rows, :nqb], idx.column_index[rows, :nqb])


def check_sets(gpu_set, scores, k, n, what):
    if n <= k:                                        # all positions, then those past the end
        np.testing.assert_array_equal(gpu_set, np.arange(k), err_msg=what)
    else:
        check_band(gpu_set, scores, k, what)


def check_sequence(q, k, v, cu, r, s, fp32, sample=None):
    """Sequence s of the packed batch against the oracle (sample: query
    blocks to check instead of the whole sequence)."""
    hq = q.shape[0]
    a, b = cu[s], cu[s + 1]
    n = b - a
    qs, ks_, vs = q[:, a:b], k[:, a:b], v[:, a:b]
    rows = slice(s * hq, (s + 1) * hq)
    what = f"sequence {s} ({n} tokens)"
    vsc, ssc = oracle.estimate_vs(qs, ks_, last_q=min(64, n))
    vi, si = r["v_idx"][rows], r["s_idx"][rows]
    for h in range(hq):
        check_sets(vi[h], vsc[h], r["kv"], n, f"{what} vertical h{h}")
        check_sets(si[h], ssc[h], r["ks"], n, f"{what} slash h{h}")
    nqb = (n + 63) // 64
    ref_idx = oracle.build_index(vi, si, n)
    compare_index(sequence_index(r["idx"], rows, nqb), ref_idx, what)
    out = r["out"][:, a:b].float().cpu().numpy()
    lse = r["lse"][:, a:b].cpu().numpy()
    dout = r["dout"][:, a:b].float().cpu().numpy()
    dlse = r["dlse"][:, a:b].cpu().numpy()
    if sample is None:
        ro, rl = oracle.attention_with_mask(qs, ks_, vs, oracle.index_mask(ref_idx, n))
        compare_out(out, ro, fp32, what)
        compare_lse(lse, rl, what)
        do, dl = oracle.dense_attention(qs, ks_, vs)
        compare_out(dout, do, fp32, what + " dense")
        compare_lse(dlse, dl, what + " dense")
    else:
        items = [(h, bb) for h in range(hq) for bb in sample]
        ref = oracle.masked_attention_blocks(qs, ks_, vs, ref_idx, items)
        dref = oracle.dense_attention_blocks(qs, ks_, vs, items)
        for (h, bb), (o, l) in ref.items():
            r0, r1 = bb * 64, min(bb * 64 + 64, n)
            compare_out(out[h, r0:r1], o, fp32, f"{what} h{h} b{bb}")
            compare_lse(lse[h, r0:r1], l, f"{what} h{h} b{bb}")
            do, dl = dref[(h, bb)]
            compare_out(dout[h, r0:r1], do, fp32, f"{what} dense h{h} b{bb}")
            compare_lse(dlse[h, r0:r1], dl, f"{what} dense h{h} b{bb}")


@pytest.mark.parametrize("hq,hkv,lens,kv,ks,fp32", [
    (4, 2, [300, 320, 777, 40, 64, 1], 30, 90, False),   # ragged, shorter than the window, one token
    (2, 1, [200, 513], 20, 60, True),                    # fp32
    (8, 1, [65, 129, 1000, 63], 100, 300, False),        # GQA 8; sets longer than some sequences
])
def test_packed_varlen(hq, hkv, lens, kv, ks, fp32):
    q, k, v, cu = packed_inputs(hq, hkv, lens, seed=sum(lens) + kv, fp32=fp32)
    r = run_varlen(q, k, v, cu, kv, ks)
    for s in range(len(lens)):
        check_sequence(q, k, v, cu, r, s, fp32)


@pytest.mark.parametrize("fp32", [False, True])
def test_packed_varlen_short_phases(fp32):
    """Key phases of 256 keys over a packed batch (so every sequence longer
    than that crosses phases, with its state carried in the workspace, and
    the grouped walk takes the units it qualifies), bf16 and fp32, every
    sequence against the oracle."""
    hq, hkv, lens = 4, 1, [700, 130, 1000, 257]
    q, k, v, cu = packed_inputs(hq, hkv, lens, seed=1001, fp32=fp32)
    r = run_varlen(q, k, v, cu, 40, 150, phase_keys=256)
    assert r["marks"] is not None
    for s_ in range(len(lens)):
        check_sequence(q, k, v, cu, r, s_, fp32)


def test_packed_varlen_key_phases():
    """The longest sequence takes key phases and the grouped walk (13,000
    tokens over phases of 12,288 keys); the shorter ones finish in the first
    phase.  Sampled query blocks of the long sequence, whole short ones."""
    hq, hkv, lens = 4, 1, [700, 13000, 5000]
    q, k, v, cu = packed_inputs(hq, hkv, lens, seed=501)
    r = run_varlen(q, k, v, cu, 300, 1000)
    # the grouped walk ran in the packed batch: every sequence has units it took
    marks = r["marks"].cpu().numpy()
    for s_, n in enumerate(lens):
        assert marks[s_ * hq:(s_ + 1) * hq, :(n + 63) // 64].any(), f"sequence {s_}: no unit in the grouped walk"
    check_sequence(q, k, v, cu, r, 0, False)
    check_sequence(q, k, v, cu, r, 1, False, sample=[0, 1, 95, 191, 192, 200, 203])
    check_sequence(q, k, v, cu, r, 2, False, sample=[0, 40, 77, 78])


def test_packed_varlen_equals_single_calls():
    """Sequences of a packed batch of 24 (lengths 64 to 900, GQA 4) against
    the one-sequence calls on their rows.  Here both split the estimate's
    keys into the same 256-key ranges and run one key phase, so the sets (a
    sequence of at most k tokens: its positions, then the ones past its end),
    the work lists and the outputs are bit for bit those of the single calls;
    the README call with cu_seqlens is the same as the steps."""
    rng = np.random.default_rng(7)
    lens = rng.integers(64, 901, 24).tolist()
    lens[3] = 40                                      # and one below the kv set size
    hq, hkv, kv, ks = 4, 1, 48, 120
    q, k, v, cu = packed_inputs(hq, hkv, lens, seed=601)
    r = run_varlen(q, k, v, cu, kv, ks)
    out_readme = msa.vertical_slash_sparse_attention(q.cuda(), k.cuda(), v.cuda(), kv, ks, cu_seqlens=cu)
    assert torch.equal(out_readme, r["out"])
    for s in (0, 3, 5, 11, 23):
        a, b = cu[s], cu[s + 1]
        n = b - a
        if n < 64:
            continue                                  # the one-sequence estimate needs the 64-row window
        qs, ks_, vs = q[:, a:b].cuda(), k[:, a:b].cuda(), v[:, a:b].cuda()
        vi, si = msa.estimate_vs(qs, ks_, min(kv, n), min(ks, n))
        rows = slice(s * hq, (s + 1) * hq)
        gv, gs = r["v_idx"][rows], r["s_idx"][rows]
        np.testing.assert_array_equal(gv[:, :min(kv, n)], vi.cpu().numpy(), err_msg=f"sequence {s} vertical")
        np.testing.assert_array_equal(gs[:, :min(ks, n)], si.cpu().numpy(), err_msg=f"sequence {s} slash")
        idx = msa.build_index(vi, si, n)
        nqb = (n + 63) // 64
        mine = sequence_index(r["idx"], rows, nqb)
        assert torch.equal(idx.block_count, mine.block_count) and torch.equal(idx.column_count, mine.column_count)
        one, lse = msa.sparse_prefill(qs, ks_, vs, idx, lse=True)
        assert torch.equal(one, r["out"][:, a:b]), f"sequence {s}"
        assert torch.equal(lse, r["lse"][:, a:b]), f"sequence {s} lse"
        assert torch.equal(msa.dense_prefill(qs, ks_, vs), r["dout"][:, a:b]), f"sequence {s} dense"


def test_packed_block_sparse_varlen():
    """The block-sparse estimate of a packed batch: each sequence's lists
    against the oracle's selection on its own rows (top-3 and top-100 key
    blocks of the mean-pooled scores, ties in a band), and its attention over
    them."""
    hq, hkv, lens = 4, 2, [150, 64 * 7, 2000, 30, 64 * 40 + 5]
    q, k, v, cu = packed_inputs(hq, hkv, lens, seed=801)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    max_len = max(lens)
    for topk in (3, 100):
        idx = msa.estimate_bs_varlen(qd, kd, cu_d, max_len, topk)
        out = msa.sparse_prefill_varlen(qd, kd, vd, idx, cu_d, max_len)
        bc, bo, cc = (t.cpu().numpy() for t in (idx.block_count, idx.block_offset, idx.column_count))
        for s_, (a, b) in enumerate(zip(cu, cu[1:])):
            n = b - a
            nqb = (n + 63) // 64                      # entries past a sequence's blocks are not written
            qs, ks_, vs = q[:, a:b], k[:, a:b], v[:, a:b]
            rows = slice(s_ * hq, (s_ + 1) * hq)
            what = f"block-sparse top-{topk} sequence {s_} ({n} tokens)"
            assert (cc[rows][:, :nqb] == 0).all(), what
            cnt, _, scores = oracle.block_sparse_select(qs, ks_, range(hq), topk=topk)
            assert np.array_equal(bc[rows][:, :nqb], cnt), what
            for h in range(hq):
                for qb in range(nqb):
                    kk = cnt[h, qb]
                    starts = bo[rows][h, qb, :kk]
                    assert np.all(starts % 64 == 0) and np.all(np.diff(starts) > 0), what
                    u = scores[h, qb, : qb + 1]          # the band on the row's softmax (scores may be negative)
                    pr = np.exp(u - u.max())
                    check_band(starts // 64, pr / pr.sum(), kk, f"{what} h{h} b{qb}")
            ref_idx = oracle.IndexArrays(bc[rows][:, :nqb], bo[rows][:, :nqb],
                                         np.zeros((hq, nqb), np.int32), np.zeros((hq, nqb, 0), np.int32))
            ro, _ = oracle.attention_with_mask(qs, ks_, vs, oracle.index_mask(ref_idx, n))
            compare_out(out[:, a:b].float().cpu().numpy(), ro, False, what)


def test_packed_streaming_and_block_sparse():
    """streaming_forward and block_sparse_attention with cu_seqlens: each
    sequence as the one-sequence call computes it."""
    hq, hkv, lens = 4, 2, [150, 64 * 7, 901, 30]
    q, k, v, cu = packed_inputs(hq, hkv, lens, seed=701)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for call, args in ((msa.streaming_forward, (64, 128)), (msa.block_sparse_attention, (3,))):
        out = call(qd, kd, vd, *args, cu_seqlens=cu)
        for i in range(len(lens)):
            a, b = cu[i], cu[i + 1]
            one = call(qd[:, a:b].contiguous(), kd[:, a:b].contiguous(), vd[:, a:b].contiguous(),
                       *[min(x, b - a) for x in args])
            assert torch.equal(out[:, a:b], one), (call.__name__, i)


def test_packed_workload_sampled():
    """The benchmark's packed batch as the benchmark runs it (64 prompts of
    1,062 to 32,444 tokens, 32 q / 8 kv heads, vertical 1000 / slash 6096):
    the shortest, a middle and the longest sequence against the oracle
    (sets of four heads within the tie band, their work lists bit-exact,
    sampled query blocks of the sparse output)."""
    from synth import PACKED_WORKLOADS, make_packed_inputs
    pw = PACKED_WORKLOADS["llama3_8b_packed_64"]
    x = make_packed_inputs(pw, device="cuda")
    q, k, v, cu = x["q"], x["k"], x["v"], x["cu_seqlens"]
    lens = list(pw.lengths)
    hq, max_len = pw.n_q_heads, max(lens)
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    v_idx, s_idx = msa.estimate_vs_varlen(q, k, cu_d, max_len, pw.vertical_topk, pw.slash_topk)
    idx = msa.build_index_varlen(v_idx, s_idx, cu_d, max_len, hq, rows=q.shape[1])
    out = msa.sparse_prefill_varlen(q, k, v, idx, cu_d, max_len)
    torch.cuda.synchronize()
    heads = [0, 5, 17, 31]
    for s in (int(np.argmin(lens)), 9, int(np.argmax(lens))):
        a, b = cu[s], cu[s + 1]
        n = b - a
        what = f"packed sequence {s} ({n} tokens)"
        qs, ks_, vs = q[:, a:b].cpu(), k[:, a:b].cpu(), v[:, a:b].cpu()
        vsc, ssc = oracle.estimate_vs(qs, ks_, heads=heads)
        vi = v_idx[s * hq:(s + 1) * hq].cpu().numpy()[heads]
        si = s_idx[s * hq:(s + 1) * hq].cpu().numpy()[heads]
        for j, h in enumerate(heads):
            check_sets(vi[j], vsc[j], pw.vertical_topk, n, f"{what} vertical h{h}")
            check_sets(si[j], ssc[j], pw.slash_topk, n, f"{what} slash h{h}")
        nqb = (n + 63) // 64
        ref_idx = oracle.build_index(vi, si, n)
        rows = [s * hq + h for h in heads]
        mine = msa.IndexTensors(idx.block_count[rows, :nqb], idx.block_offset[rows, :nqb],
                                idx.column_count[rows, :nqb], idx.column_index[rows, :nqb])
        compare_index(mine, ref_idx, what)
        blocks = sorted({0, nqb // 3, nqb // 2, nqb - 1})
        items = [(h, bb) for h in heads for bb in blocks]
        ref = oracle.masked_attention_blocks(qs, ks_, vs, ref_idx, items, head_rows={h: j for j, h in enumerate(heads)})
        o = out[:, a:b].float().cpu().numpy()
        for (h, bb), (ro, _) in ref.items():
            compare_out(o[h, bb * 64:min(bb * 64 + 64, n)], ro, False, f"{what} h{h} b{bb}")


def test_packed_bad_offsets_stay_in_bounds():
    """cu_seqlens contents that break the rules (falling, past the packed
    length) are clamped on the device: the calls complete and every output
    is finite.  Here sequence 1 clamps to empty and sequence 2 to rows
    100..599, overlapping sequence 0, so only rows 0..99 are sequence 0's
    alone and must equal the well-formed batch's."""
    hq, hkv, lens = 4, 2, [300, 200, 500]
    q, k, v, cu = packed_inputs(hq, hkv, lens, seed=901)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    good = run_varlen(q, k, v, cu, 30, 90)
    total = q.shape[1]
    bad = torch.tensor([0, 300, 100, 1 << 30], dtype=torch.int32, device="cuda")   # falling, then past the end
    v_idx, s_idx = msa.estimate_vs_varlen(qd, kd, bad, 500, 30, 90)
    idx = msa.build_index_varlen(v_idx, s_idx, bad, 500, hq, rows=total)
    out = torch.zeros_like(qd)
    msa.sparse_prefill_varlen(qd, kd, vd, idx, bad, 500, out=out)
    dout = torch.zeros_like(qd)
    msa.dense_prefill_varlen(qd, kd, vd, bad, 500, out=dout)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(dout.float()).all()
    assert torch.equal(out[:, :100], good["out"][:, :100])
    assert torch.equal(dout[:, :100], good["dout"][:, :100])


def test_packed_block_sparse_chunks():
    """The block-sparse scores of a packed batch go through the workspace in
    chunks of 1024 query blocks: a 70,000-token sequence (1,094 blocks, two
    chunks) packed with short ones, fp32, its lists and the short ones'
    against the oracle's selection (two heads each)."""
    hq, hkv, lens = 2, 1, [70000, 300, 1500]
    q, k, v, cu = packed_inputs(hq, hkv, lens, seed=1101, fp32=True)
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    idx = msa.estimate_bs_varlen(q.cuda(), k.cuda(), cu_d, max(lens), 100)
    bc, bo = idx.block_count.cpu().numpy(), idx.block_offset.cpu().numpy()
    for s_, (a, b) in enumerate(zip(cu, cu[1:])):
        n = b - a
        nqb = (n + 63) // 64
        cnt, _, scores = oracle.block_sparse_select(q[:, a:b], k[:, a:b], range(hq), topk=100)
        rows = slice(s_ * hq, (s_ + 1) * hq)
        assert np.array_equal(bc[rows][:, :nqb], cnt), f"sequence {s_}"
        for h in range(hq):
            for qb in sorted({0, nqb // 2, 1023 % nqb, 1024 % nqb, nqb - 1}):
                kk = cnt[h, qb]
                u = scores[h, qb, : qb + 1]
                pr = np.exp(u - u.max())
                check_band(bo[rows][h, qb, :kk] // 64, pr / pr.sum(), kk, f"sequence {s_} h{h} b{qb}")
