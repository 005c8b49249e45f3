"""GPU parity of the fused sparse prefill (work lists walked inside the
attention kernel, msa_sparse_prefill_fused) against the oracle and against
msa_build_index + msa_sparse_prefill on the same sets.

Both paths visit the same blocks in the same key phases, then every column in
a query block's final phase, in the same order; only the list path's grouped
walk (which runs some query blocks as aligned-tile walks) differs.  So the
outputs must be bitwise equal on every query block that walk did not take,
and agree at the graded tolerances on the rest."""

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_vertical_amd as msa
import oracle
from parity import compare_lse, compare_out
from synth import make_inputs, small_workload

pytestmark = pytest.mark.gpu


def inputs(hq, hkv, n, seed=0, fp32=False):
    w = small_workload(n_q_heads=hq, n_kv_heads=hkv, seq_len=n, seed=seed,
                       dtypes=("fp32", "bf16") if fp32 else ("bf16",))
    x = make_inputs(w)
    if fp32:
        return x["q32"], x["k32"], x["v32"]
    return x["q"], x["k"], x["v"]


def random_sets(h, n, kv, ks, seed=0):
    r = np.random.default_rng(seed)
    v = np.stack([np.sort(r.choice(n, size=kv, replace=False)) for _ in range(h)]).astype(np.int32)
    s = np.stack([np.sort(r.choice(n, size=ks, replace=False)) for _ in range(h)]).astype(np.int32)
    return v.reshape(h, kv), s.reshape(h, ks)


def one_phase(n):
    return -(-n // 64) * 64


def dev(*ts):
    return [t.to("cuda") for t in ts]


def list_path(qs, ks_, vs, vi, si, n, **kw):
    idx = msa.build_index(*dev(torch.from_numpy(vi), torch.from_numpy(si)), n)
    return msa.sparse_prefill(qs, ks_, vs, idx, lse=True, **kw)


def list_path_phases(qs, ks_, vs, vi, si, n, phase):
    """The list path in key phases, and which (q head, query block) its
    grouped walk took."""
    hq, hkv = qs.shape[0], ks_.shape[0]
    nbytes = msa.sparse_prefill_workspace_bytes(hq, hkv, n, qs.dtype, phase_keys=phase)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")
    out, lse = list_path(qs, ks_, vs, vi, si, n, phase_keys=phase, workspace=ws)
    torch.cuda.synchronize()
    marks = msa.sparse_walk_marks(ws, hq, hkv, n, qs.dtype, phase_keys=phase).cpu().numpy()
    return out, lse, marks


def equal_where_not_walked(out, lse, ref, ref_lse, marks, fp32, what):
    """Bitwise equal on the query blocks the grouped walk left to the per-head
    kernel; graded tolerances on the ones it took."""
    n = out.shape[1]
    rows = np.repeat(marks == 0, 64, axis=1)[:, :n]
    rows_t = torch.from_numpy(rows).to(out.device)
    assert torch.equal(out[rows_t], ref[rows_t]), f"{what}: outputs differ where the walk did not run"
    assert torch.equal(lse[rows_t], ref_lse[rows_t]), f"{what}: lse differs where the walk did not run"
    compare_out(out.float().cpu().numpy(), ref.float().cpu().numpy(), fp32, what)
    compare_lse(lse.cpu().numpy(), ref_lse.cpu().numpy(), what)
    return int((marks != 0).sum())


@pytest.mark.parametrize("hq,hkv,n,kv,ks,fp32", [
    (4, 1, 256, 7, 9, False),
    (4, 2, 64 * 7 + 23, 20, 60, False),     # ragged last query block
    (2, 1, 1024, 100, 40, False),
    (2, 2, 384, 5, 200, False),
    (2, 1, 50, 5, 10, False),               # shorter than one block
    (2, 1, 320, 9, 13, True),
    (8, 1, 512, 20, 30, False),             # GQA group of 8
    (6, 2, 448, 15, 25, False),             # GQA group of 3
    (2, 1, 4096, 1024, 300, False),         # the most columns the fused kernel holds
    (2, 1, 4096, 9, 4096, False),           # every diagonal: blocks tile [0, r1]
    (2, 1, 8192, 300, 2000, False),
])
def test_fused_one_launch_equals_lists(hq, hkv, n, kv, ks, fp32):
    q, k, v = inputs(hq, hkv, n, seed=n + kv, fp32=fp32)
    vi, si = random_sets(hq, n, kv, ks, seed=n + ks)
    qs, ks_, vs = dev(q, k, v)
    pk = one_phase(n)
    out, lse = msa.sparse_prefill_fused(qs, ks_, vs, *dev(torch.from_numpy(vi), torch.from_numpy(si)),
                                        lse=True, phase_keys=pk)
    ref_out, ref_lse = list_path(qs, ks_, vs, vi, si, n, phase_keys=pk)
    assert torch.equal(out, ref_out)
    assert torch.equal(lse, ref_lse)
    if n <= 4096:
        ridx = oracle.build_index(vi, si, n)
        ref, rlse = oracle.attention_with_mask(q, k, v, oracle.index_mask(ridx, n))
        compare_out(out.float().cpu().numpy(), ref, fp32, "fused")
        compare_lse(lse.cpu().numpy(), rlse, "fused")


@pytest.mark.parametrize("hq,hkv,n,kv,ks,phase,fp32", [
    (4, 2, 1216, 40, 60, 64, False),      # one phase per query block, ragged lists
    (2, 1, 1216, 100, 300, 320, False),   # phase edges inside block tiles (unaligned starts)
    (2, 1, 2048, 7, 2048, 512, False),    # every diagonal: blocks in every phase
    (2, 1, 640, 9, 13, 192, True),        # fp32; most phases hold nothing for most blocks
    (1, 1, 256, 1, 1, 64, False),         # a single diagonal and column
    (2, 1, 4096, 9, 4096, 1024, False),   # every diagonal: 16 tiles in each full phase
    (1, 1, 4096, 5, 4096, 1024, True),    # the same in fp32
    (2, 1, 4096, 30, 1200, 1024, False),  # about 16 per phase: some carried, some left over
    (2, 1, 4096, 800, 600, 256, False),   # many columns, found across the phases, all run in the last
    (2, 1, 64 * 9 + 63, 30, 100, 128, False),   # short last block
])
def test_fused_phases(hq, hkv, n, kv, ks, phase, fp32):
    q, k, v = inputs(hq, hkv, n, seed=n + phase, fp32=fp32)
    vi, si = random_sets(hq, n, kv, ks, seed=n + phase + 1)
    qs, ks_, vs = dev(q, k, v)
    dt = torch.float32 if fp32 else torch.bfloat16
    need = msa.sparse_prefill_fused_workspace_bytes(hq, hkv, n, kv, dt, phase_keys=phase)
    assert need == msa.sparse_prefill_workspace_bytes(hq, hkv, n, dt, phase_keys=phase) + \
        hq * (-(-n // 64)) * (-(-kv // 32)) * 4
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")     # no initial contents assumed
    vt, st = dev(torch.from_numpy(vi), torch.from_numpy(si))
    out, lse = msa.sparse_prefill_fused(qs, ks_, vs, vt, st, lse=True, phase_keys=phase, workspace=ws)
    ridx = oracle.build_index(vi, si, n)
    ref, rlse = oracle.attention_with_mask(q, k, v, oracle.index_mask(ridx, n))
    compare_out(out.float().cpu().numpy(), ref, fp32, "fused phases")
    compare_lse(lse.cpu().numpy(), rlse, "fused phases")
    one, one_lse = msa.sparse_prefill_fused(qs, ks_, vs, vt, st, lse=True, phase_keys=one_phase(n))
    compare_out(out.float().cpu().numpy(), one.float().cpu().numpy(), fp32, "fused phases vs one launch")
    compare_lse(lse.cpu().numpy(), one_lse.cpu().numpy(), "fused phases vs one launch")
    # the same call again on the used workspace gives the same bits
    again, again_lse = msa.sparse_prefill_fused(qs, ks_, vs, vt, st, lse=True, phase_keys=phase, workspace=ws)
    assert torch.equal(again, out) and torch.equal(again_lse, lse)
    # the list path in the same phases: the same tiles in the same order
    lo, llse, marks = list_path_phases(qs, ks_, vs, vi, si, n, phase)
    equal_where_not_walked(out, lse, lo, llse, marks, fp32, "fused vs lists, phases")


@pytest.mark.parametrize("n,kv,ks,phase", [
    (1 << 15, 500, 300, 1024),        # many phases, state carried, columns found across phases
    (1 << 15, 500, 2000, 1024),       # nearly every tile listed: the grouped walk takes most query blocks
    (1 << 15, 1024, 1 << 15, 16384),  # every diagonal, the longest phase: 256 blocks per phase
    (3 * 4096 + 700, 64, 900, 4096),  # ragged sequence, last phase partial
])
def test_fused_long_against_lists(n, kv, ks, phase):
    """Longer sequences against the list path in its own key phases and in one
    launch (the oracle's dense masks do not fit these sizes)."""
    hq, hkv = 2, 1
    q, k, v = inputs(hq, hkv, n, seed=n + 3)
    vi, si = random_sets(hq, n, kv, ks, seed=n + 4)
    qs, ks_, vs = dev(q, k, v)
    vt, st = dev(torch.from_numpy(vi), torch.from_numpy(si))
    out, lse = msa.sparse_prefill_fused(qs, ks_, vs, vt, st, lse=True, phase_keys=phase)
    ref, rlse, marks = list_path_phases(qs, ks_, vs, vi, si, n, phase)
    walked = equal_where_not_walked(out, lse, ref, rlse, marks, False, "fused vs lists, phases")
    if ks * 64 < n:                             # lists far from dense: most query blocks compared bit for bit
        assert walked < marks.size // 2
    one, one_lse = list_path(qs, ks_, vs, vi, si, n, phase_keys=one_phase(n))
    compare_out(out.float().cpu().numpy(), one.float().cpu().numpy(), False, "fused vs lists, one launch")
    compare_lse(lse.cpu().numpy(), one_lse.cpu().numpy(), "fused vs lists, one launch")
    if ks == n:                           # every diagonal: dense attention
        dense, dlse = msa.dense_prefill(qs, ks_, vs, lse=True)
        compare_out(out.float().cpu().numpy(), dense.float().cpu().numpy(), False, "fused all diagonals vs dense")
        compare_lse(lse.cpu().numpy(), dlse.cpu().numpy(), "fused all diagonals vs dense")


@pytest.mark.parametrize("phase", [0, 128])
def test_fused_empty_and_out_of_range_sets(phase):
    """Empty sets give zero rows and lse = -inf; entries outside [0, N) select
    nothing (the list path, given the same sets, agrees bit for bit in one
    launch)."""
    n, hq = 640, 2
    q, k, v = inputs(hq, 1, n, seed=11)
    qs, ks_, vs = dev(q, k, v)
    e = torch.empty((hq, 0), dtype=torch.int32, device="cuda")
    out, lse = msa.sparse_prefill_fused(qs, ks_, vs, e, e, lse=True, phase_keys=phase)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    vi = np.array([[-7, 3, 100, n, n + 5]] * hq, np.int32)
    si = np.array([[-3, -1, 0, 64, 300, n + 1]] * hq, np.int32)
    vt, st = dev(torch.from_numpy(vi), torch.from_numpy(si))
    out, lse = msa.sparse_prefill_fused(qs, ks_, vs, vt, st, lse=True, phase_keys=phase)
    keep_v = np.array([[3, 100]] * hq, np.int32)
    keep_s = np.array([[0, 64, 300]] * hq, np.int32)
    ridx = oracle.build_index(keep_v, keep_s, n)
    ref, rlse = oracle.attention_with_mask(q, k, v, oracle.index_mask(ridx, n))
    compare_out(out.float().cpu().numpy(), ref, False, "out-of-range entries")
    compare_lse(lse.cpu().numpy(), rlse, "out-of-range entries")
    if phase == 0:
        lo, llse = list_path(qs, ks_, vs, vi, si, n, phase_keys=one_phase(n))
        assert torch.equal(out, lo) and torch.equal(lse, llse)


def test_fused_layer_sets():
    """The sets the estimator writes (online, from q and k) through both paths."""
    n, hq, hkv = 4096, 4, 2
    q, k, v = inputs(hq, hkv, n, seed=21)
    qs, ks_, vs = dev(q, k, v)
    vi, si = msa.estimate_vs(qs, ks_, 200, 600)[:2]
    out, lse = msa.sparse_prefill_fused(qs, ks_, vs, vi, si, lse=True, phase_keys=one_phase(n))
    idx = msa.build_index(vi, si, n)
    ref, rlse = msa.sparse_prefill(qs, ks_, vs, idx, lse=True, phase_keys=one_phase(n))
    assert torch.equal(out, ref) and torch.equal(lse, rlse)


@pytest.mark.parametrize("hq,hkv,n,kv,ks,phase,fp32", [
    (4, 2, 640, 20, 60, 0, False),          # one launch
    (2, 1, 64 * 9 + 23, 30, 200, 0, False),  # ragged last query block
    (2, 1, 1216, 40, 300, 256, False),      # key phases, state carried
    (2, 1, 640, 9, 13, 192, True),          # fp32, phases
    (8, 2, 1024, 64, 500, 0, False),        # GQA group of 4, dense-ish diagonals
])
def test_fused_exact_union_mask(hq, hkv, n, kv, ks, phase, fp32):
    """MSA_FUSED_EXACT: attention over exactly (j <= i) and (j in V or i - j in
    S), against the oracle's exact_union_mask."""
    q, k, v = inputs(hq, hkv, n, seed=n + ks, fp32=fp32)
    vi, si = random_sets(hq, n, kv, ks, seed=n + kv)
    qs, ks_, vs = dev(q, k, v)
    vt, st = dev(torch.from_numpy(vi), torch.from_numpy(si))
    dt = torch.float32 if fp32 else torch.bfloat16
    need = msa.sparse_prefill_fused_workspace_bytes(hq, hkv, n, kv, dt, phase_keys=phase, exact=True)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    out, lse = msa.sparse_prefill_fused(qs, ks_, vs, vt, st, lse=True, phase_keys=phase, exact=True, workspace=ws)
    ref, rlse = oracle.attention_with_mask(q, k, v, oracle.exact_union_mask(vi, si, n))
    compare_out(out.float().cpu().numpy(), ref, fp32, "exact union")
    compare_lse(lse.cpu().numpy(), rlse, "exact union")
    # the exact mask is a subset of the block cover: no row keeps more mass
    _, blse = msa.sparse_prefill_fused(qs, ks_, vs, vt, st, lse=True, phase_keys=phase)
    fin = torch.isfinite(lse)
    assert torch.all(lse[fin] <= blse[fin] + 1e-5)


def test_fused_exact_special_cases():
    """Closed forms: only the main diagonal -> each row attends to itself
    (out = v of that row); every diagonal -> dense causal attention; only
    columns -> the column keys below each row."""
    n, hq = 448, 2
    q, k, v = inputs(hq, 1, n, seed=5)
    qs, ks_, vs = dev(q, k, v)
    none = torch.empty((hq, 0), dtype=torch.int32, device="cuda")
    main = torch.zeros((hq, 1), dtype=torch.int32, device="cuda")
    out = msa.sparse_prefill_fused(qs, ks_, vs, none, main, exact=True)
    assert torch.equal(out[0], vs[0]) and torch.equal(out[1], vs[0])
    every = torch.arange(n, dtype=torch.int32, device="cuda").expand(hq, -1).contiguous()
    out, lse = msa.sparse_prefill_fused(qs, ks_, vs, none, every, lse=True, exact=True)
    ref, rlse = oracle.dense_attention(q, k, v)
    compare_out(out.float().cpu().numpy(), ref, False, "exact, every diagonal")
    compare_lse(lse.cpu().numpy(), rlse, "exact, every diagonal")
    cols = np.array([[3, 70, 200, 201, 447]] * hq, np.int32)
    out, lse = msa.sparse_prefill_fused(qs, ks_, vs, dev(torch.from_numpy(cols))[0], none, lse=True, exact=True)
    ref, rlse = oracle.attention_with_mask(q, k, v, oracle.exact_union_mask(cols, np.zeros((hq, 0), np.int64), n))
    compare_out(out.float().cpu().numpy(), ref, False, "exact, columns only")
    compare_lse(lse.cpu().numpy(), rlse, "exact, columns only")
