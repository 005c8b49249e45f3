"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before touching the
device."""

import ctypes
import os
import re

import pytest

import dynamic_sparse_attention_vertical_amd as m
from dynamic_sparse_attention_vertical_amd import msa as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

OK, NULL, SHAPE, DTYPE, RANGE, CAP, WS = 0, 1, 2, 3, 4, 5, 6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return m.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 26, names
    for n in names:
        assert hasattr(lib, n), n


def P(hq=32, hkv=8, n=4096, d=128, dtype=0, scale=0.0, stride=0):
    return ctypes.byref(B.Problem(hq, hkv, n, d, dtype, scale, stride))


FAKE = ctypes.c_void_p(0x1000)       # never dereferenced: every case fails validation first


def status_of(lib, fn, *args):
    return getattr(lib, fn)(*args)


def test_problem_validation(lib):
    for prob, want in [(P(d=64), SHAPE), (P(hq=6, hkv=4), SHAPE), (P(n=0), SHAPE),
                       (P(n=1 << 31), SHAPE), (P(dtype=7), DTYPE), (P(scale=-1.0), RANGE),
                       (P(hkv=0), SHAPE), (P(stride=4095), SHAPE), (P(stride=-1), SHAPE)]:
        assert lib.msa_dense_prefill(prob, FAKE, FAKE, FAKE, FAKE, None, None) == want
        assert lib.msa_last_error()
    assert lib.msa_dense_prefill(None, FAKE, FAKE, FAKE, FAKE, None, None) == NULL
    assert lib.msa_dense_prefill(P(), None, FAKE, FAKE, FAKE, None, None) == NULL
    assert lib.msa_status_str(SHAPE) == b"MSA_ERR_SHAPE"
    # the vertical-slash estimate needs last_q = 64 rows
    assert lib.msa_estimate_vs(P(n=40), FAKE, FAKE, 64, 8, 8, FAKE, FAKE, None, None, FAKE, 1 << 30,
                               None) == SHAPE


def test_index_caps(lib):
    cb, cc = ctypes.c_int32(), ctypes.c_int32()
    assert lib.msa_index_caps(P(n=1 << 20), 1000, 6096, 64, ctypes.byref(cb), ctypes.byref(cc)) == OK
    assert (cb.value, cc.value) == (6096, 1000)
    assert lib.msa_index_caps(P(n=4096), 64, 256, 64, ctypes.byref(cb), ctypes.byref(cc)) == OK
    assert (cb.value, cc.value) == (64, 64)
    assert lib.msa_index_caps(P(n=4096), 64, 256, 32, ctypes.byref(cb), ctypes.byref(cc)) == RANGE
    assert lib.msa_index_caps(P(n=4096), 5000, 256, 64, ctypes.byref(cb), ctypes.byref(cc)) == RANGE
    # a short last query block counts as a block
    assert lib.msa_index_caps(P(n=64 * 3 + 5), 10, 150, 64, ctypes.byref(cb), ctypes.byref(cc)) == OK
    assert (cb.value, cc.value) == (4, 10)


def test_build_index_validation(lib):
    args = lambda cb, cc, blk=64: (P(n=4096), FAKE, 64, FAKE, 256, blk, FAKE, FAKE, cb, FAKE, FAKE, cc, None)
    assert lib.msa_build_index(*args(63, 64)) == CAP
    assert lib.msa_build_index(*args(64, 63)) == CAP
    assert lib.msa_build_index(*args(64, 64, blk=128)) == RANGE
    a = list(args(64, 64))
    a[6] = None
    assert lib.msa_build_index(*a) == NULL


def test_estimate_validation(lib):
    prob = P(n=4096)
    ws = lib.msa_estimate_vs_workspace(prob, 64, 64, 256)
    assert ws > 0 and lib.msa_estimate_vs_workspace(prob, 32, 64, 256) == 0
    call = lambda lq, kv, ks, wsb: lib.msa_estimate_vs(prob, FAKE, FAKE, lq, kv, ks, FAKE, FAKE, None, None,
                                                       FAKE, wsb, None)
    assert call(32, 64, 256, ws) == RANGE
    assert call(64, 0, 256, ws) == RANGE
    assert call(64, 64, 5000, ws) == RANGE
    assert call(64, 64, 256, ws - 1) == WS


def test_estimate_noalloc_validation(lib):
    """Checked on the host before any device call: the arguments as for
    msa_estimate_vs, and the scratch the problem needs against the 80 MiB the
    library holds per GPU."""
    call = lambda prob, lq=64, kv=64, ks=256: lib.msa_estimate_vs_noalloc(prob, FAKE, FAKE, lq, kv, ks, FAKE, FAKE,
                                                                           None, None, None)
    assert call(P(n=4096), lq=32) == RANGE
    assert call(P(n=4096), kv=0) == RANGE
    assert call(P(n=40)) == SHAPE
    assert lib.msa_estimate_vs_noalloc(P(n=4096), None, FAKE, 64, 64, 256, FAKE, FAKE, None, None, None) == NULL
    # 32 q heads at 1M need ~260 MiB of scratch (the workspace size of msa_estimate_vs)
    big = P(n=1 << 20)
    assert lib.msa_estimate_vs_workspace(big, 64, 1000, 6096) > 80 << 20
    assert call(big, kv=1000, ks=6096) == WS
    assert b"80" in lib.msa_last_error() or b"83886080" in lib.msa_last_error()
    # 8 q heads at 1M and 32 at 256K fit
    assert lib.msa_estimate_vs_workspace(P(hq=8, hkv=2, n=1 << 20), 64, 1000, 6096) <= 80 << 20
    assert lib.msa_estimate_vs_workspace(P(n=1 << 18), 64, 1000, 6096) <= 80 << 20


def test_estimate_bs_validation(lib):
    prob = P(n=4096)
    ws = lib.msa_estimate_bs_workspace(prob, 64)
    # pooled q and k means, then the score keys of one chunk of query blocks
    # (all 64 here)
    assert ws == 32 * 64 * 128 * 4 + 8 * 64 * 128 * 4 + 32 * 64 * 64 * 4
    call = lambda blk, k, cap, wsb: lib.msa_estimate_bs(prob, FAKE, FAKE, blk, k, FAKE, FAKE, cap, FAKE, FAKE,
                                                        wsb, None)
    assert call(32, 10, 10, ws) == RANGE
    assert call(64, 0, 10, ws) == RANGE
    assert call(64, 10, 9, ws) == CAP
    assert call(64, 10, 10, ws - 1) == WS
    # no length limit beyond seq_len < 2^31: at 1M tokens (16384 key blocks,
    # more than one query-block chunk of 1024) the workspace follows the same
    # formula and a call gets as far as the workspace check
    big = P(hq=8, hkv=2, n=1 << 20)
    nb = (1 << 20) // 64
    wsb = lib.msa_estimate_bs_workspace(big, 64)
    assert wsb == 8 * nb * 128 * 4 + 2 * nb * 128 * 4 + 8 * 1024 * nb * 4
    assert lib.msa_estimate_bs(big, FAKE, FAKE, 64, 100, FAKE, FAKE, 100, FAKE, FAKE, wsb - 1, None) == WS


def test_sparse_prefill_validation(lib):
    # n = 4096 fits one default phase: no workspace needed
    call = lambda bc, cb: lib.msa_sparse_prefill(P(), FAKE, FAKE, FAKE, bc, FAKE, cb, FAKE, FAKE, 4, 0, None, 0,
                                                 FAKE, None, None)
    assert call(None, 4) == NULL
    assert call(FAKE, -1) == CAP
    phased = lambda pk, ws, wsb: lib.msa_sparse_prefill(P(), FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 4, pk,
                                                        ws, wsb, FAKE, None, None)
    need = lib.msa_sparse_prefill_workspace(P(), 1024)
    assert phased(-64, FAKE, need) == RANGE
    assert phased(100, FAKE, need) == RANGE
    assert phased(1024, None, need) == NULL
    assert phased(1024, FAKE, need - 1) == WS
    assert phased(1024, ctypes.c_void_p(0x1004), need) == RANGE      # not 16-byte aligned


def test_sparse_prefill_fused_validation(lib):
    call = lambda prob, vi, kv, si, ks, pk=0, ws=None, wsb=0, lse=None, flags=0: lib.msa_sparse_prefill_fused(
        prob, FAKE, FAKE, FAKE, vi, kv, si, ks, pk, flags, ws, wsb, FAKE, lse, None)
    assert call(P(), None, 4, FAKE, 4) == NULL
    assert call(P(), FAKE, 4, None, 4) == NULL
    assert call(P(), FAKE, -1, FAKE, 4) == RANGE
    assert call(P(), FAKE, 4, FAKE, 4097) == RANGE                  # more than seq_len
    assert call(P(), FAKE, 1025, FAKE, 4) == RANGE                  # the kernel holds 1024 columns
    assert call(P(), ctypes.c_void_p(0x1002), 4, FAKE, 4) == RANGE  # not 4-byte aligned
    assert call(P(), FAKE, 4, FAKE, 4, pk=100) == RANGE
    assert call(P(n=1 << 17), FAKE, 4, FAKE, 4, pk=32768) == RANGE  # phases of at most 16384 keys
    assert call(P(), FAKE, 4, FAKE, 4, flags=2) == RANGE            # unknown flag
    # the exact mask needs its bitmaps even in one phase
    need_x = lib.msa_sparse_prefill_fused_workspace(P(), 4, 0, 1)
    assert need_x > 0
    assert call(P(), FAKE, 4, FAKE, 4, flags=1) == NULL
    assert call(P(), FAKE, 4, FAKE, 4, flags=1, ws=FAKE, wsb=need_x - 1) == WS
    n = 1 << 15
    need = lib.msa_sparse_prefill_fused_workspace(P(n=n), 4, 0, 0)
    assert need > 0
    assert call(P(n=n), FAKE, 4, FAKE, 4, ws=None, wsb=need) == NULL
    assert call(P(n=n), FAKE, 4, FAKE, 4, ws=FAKE, wsb=need - 1) == WS
    assert call(P(n=n), FAKE, 4, FAKE, 4, ws=ctypes.c_void_p(0x1004), wsb=need) == RANGE
    assert call(P(d=64), FAKE, 4, FAKE, 4) == SHAPE
    assert lib.msa_last_error()


def test_sparse_prefill_fused_workspace_size(lib):
    # one phase: none; phases: the list path's state, then kv bits (rounded
    # up to 32-bit words) per q head and query block
    assert lib.msa_sparse_prefill_fused_workspace(P(), 1000, 0, 0) == 0
    for kv in (0, 1, 32, 33, 1000, 1024):
        n = 1 << 17
        words = (kv + 31) // 32
        base = lib.msa_sparse_prefill_workspace(P(n=n), 0) + 32 * (n // 64) * words * 4
        assert lib.msa_sparse_prefill_fused_workspace(P(n=n), kv, 0, 0) == base
        # exact union mask: two bitmaps of n bits per q head after that
        assert lib.msa_sparse_prefill_fused_workspace(P(n=n), kv, 0, 1) == base + 2 * 32 * (n // 32) * 4
    assert lib.msa_sparse_prefill_fused_workspace(P(n=4096 + 5), 8, 0, 1) == 2 * 32 * (4096 // 32 + 1) * 4
    assert lib.msa_sparse_prefill_fused_workspace(P(n=1 << 17), 1025, 0, 0) == 0     # invalid: too many columns
    assert lib.msa_sparse_prefill_fused_workspace(P(n=1 << 17), -1, 0, 0) == 0
    assert lib.msa_sparse_prefill_fused_workspace(P(n=1 << 17), 8, 100, 0) == 0      # invalid phase length
    assert lib.msa_sparse_prefill_fused_workspace(P(n=1 << 17), 8, 0, 4) == 0        # unknown flag


def test_decode_sparse_validation(lib):
    call = lambda prob, topk=8, idx=FAKE, flags=0, ws=FAKE, wsb=1 << 30, lse=None, rec=None: lib.msa_decode_sparse(
        prob, FAKE, FAKE, FAKE, topk, idx, flags, ws, wsb, FAKE, lse, rec, None)
    need = lib.msa_decode_sparse_workspace(P())
    # scores as 32-bit keys for every (q head, cached key), top-k histograms
    assert need >= 32 * 4096 * 4 + 32 * 2048 * 4
    assert call(P(), topk=0) == RANGE
    assert call(P(), topk=4097) == RANGE
    assert call(P(), flags=2) == RANGE
    assert call(P(), idx=None) == NULL
    assert call(P(), ws=None) == NULL
    assert call(P(), wsb=need - 1) == WS
    assert call(P(), ws=ctypes.c_void_p(0x1004), wsb=need) == RANGE
    assert call(P(), idx=ctypes.c_void_p(0x1002)) == RANGE
    assert call(P(hq=6, hkv=4)) == SHAPE
    assert lib.msa_decode_sparse_workspace(P(d=64)) == 0
    # the per-cache lengths: the same checks, plus the lengths pointer itself
    vl = lambda prob, lens=FAKE, topk=8, wsb=1 << 30: lib.msa_decode_sparse_varlen(
        prob, FAKE, FAKE, FAKE, lens, topk, FAKE, 0, FAKE, wsb, FAKE, None, None, None)
    assert vl(P(), lens=None) == NULL
    assert vl(P(), lens=ctypes.c_void_p(0x1002)) == RANGE
    assert vl(P(), topk=4097) == RANGE
    assert vl(P(), wsb=need - 1) == WS
    assert vl(P(hq=6, hkv=4)) == SHAPE


def test_varlen_validation(lib):
    """The packed-batch calls check their descriptor on the host."""
    VL = lambda cu=FAKE, n=3, mx=1000: ctypes.byref(B.Varlen(cu, n, mx))
    est = lambda prob, vl, kv=8, ks=8, ws=FAKE, wsb=1 << 30: lib.msa_estimate_vs_varlen(
        prob, vl, FAKE, FAKE, 64, kv, ks, FAKE, FAKE, ws, wsb, None)
    assert est(P(), None) == NULL
    assert est(P(), VL(cu=None)) == NULL
    assert est(P(), VL(cu=ctypes.c_void_p(0x1002))) == RANGE
    assert est(P(), VL(n=0)) == SHAPE
    assert est(P(), VL(mx=0)) == SHAPE
    assert est(P(), VL(mx=4097)) == SHAPE                       # longer than the rows of a head
    assert est(P(), VL(n=1024)) == SHAPE                        # 1024 sequences x 32 heads > 32767
    assert est(P(), VL(), kv=1001) == RANGE                     # top-k above max_seqlen
    assert est(P(hq=6, hkv=4), VL()) == SHAPE
    need = lib.msa_estimate_vs_varlen_workspace(P(), VL(), 64)
    assert need > 0 and lib.msa_estimate_vs_varlen_workspace(P(), VL(), 32) == 0
    assert est(P(), VL(), wsb=need - 1) == WS
    # the work lists are sized for max_seqlen per head
    cb, cc = ctypes.c_int32(), ctypes.c_int32()
    assert lib.msa_index_caps(P(n=1000), 8, 30, 64, ctypes.byref(cb), ctypes.byref(cc)) == OK
    bi = lambda vl, cap_b=cb.value, cap_c=cc.value: lib.msa_build_index_varlen(
        P(), vl, FAKE, 8, FAKE, 30, 64, FAKE, FAKE, cap_b, FAKE, FAKE, cap_c, None)
    assert bi(None) == NULL
    assert bi(VL(), cap_b=cb.value - 1) == CAP
    assert bi(VL(mx=5000)) == SHAPE
    sp = lambda vl, wsb=1 << 30: lib.msa_sparse_prefill_varlen(
        P(n=1 << 17), vl, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 8, 0, FAKE, wsb, FAKE, None, None)
    assert sp(None) == NULL
    assert sp(VL(n=4, mx=1 << 17), wsb=1) == WS                 # phases of the longest sequence need state
    assert lib.msa_sparse_prefill_varlen_workspace(P(n=1 << 17), VL(n=4, mx=1 << 17), 0) > \
        lib.msa_sparse_prefill_varlen_workspace(P(n=1 << 17), VL(n=2, mx=1 << 17), 0) > 0
    assert lib.msa_sparse_prefill_varlen_workspace(P(n=1 << 17), VL(n=4, mx=1000), 0) == 0   # one phase
    assert lib.msa_dense_prefill_varlen(P(), VL(cu=None), FAKE, FAKE, FAKE, FAKE, None, None) == NULL
    bs = lambda vl, cap=8, wsb=1 << 30: lib.msa_estimate_bs_varlen(P(), vl, FAKE, FAKE, 64, 8, FAKE, FAKE, cap,
                                                                   FAKE, FAKE, wsb, None)
    assert bs(None) == NULL
    assert bs(VL(), cap=7) == CAP
    assert bs(VL(mx=5000)) == SHAPE
    need_bs = lib.msa_estimate_bs_varlen_workspace(P(), VL(), 64)
    assert need_bs > lib.msa_estimate_bs_varlen_workspace(P(), VL(n=2), 64) > 0
    assert bs(VL(), wsb=need_bs - 1) == WS


def test_walk_marks_query(lib):
    off, kh = ctypes.c_size_t(), ctypes.c_int32()
    # one phase covers the sequence: no workspace, no walk
    assert lib.msa_sparse_prefill_walk_marks(P(n=4096), 0, ctypes.byref(off), ctypes.byref(kh)) == OK
    assert (off.value, kh.value) == (0, 0)
    # phases: the marks follow the per-block states and records; GQA 4 -> units of 4 heads
    n = 1 << 17
    assert lib.msa_sparse_prefill_walk_marks(P(n=n), 0, ctypes.byref(off), ctypes.byref(kh)) == OK
    assert kh.value == 4 and off.value == 32 * (n // 64) * (2 * (64 * 64 + 2 * 64) * 4 + 8)
    assert off.value + 32 * (n // 64) * 4 <= lib.msa_sparse_prefill_workspace(P(n=n), 0)
    assert lib.msa_sparse_prefill_walk_marks(P(hq=6, hkv=2, n=n), 0, ctypes.byref(off), ctypes.byref(kh)) == OK
    assert kh.value == 1
    assert lib.msa_sparse_prefill_walk_marks(P(n=n), 100, ctypes.byref(off), ctypes.byref(kh)) == RANGE
    assert lib.msa_sparse_prefill_walk_marks(P(n=n), 0, None, ctypes.byref(kh)) == NULL


def test_default_phase_keys_matches_header(lib):
    text = open(HEADER).read()
    assert int(re.search(r"#define MSA_DEFAULT_PHASE_KEYS (\d+)", text).group(1)) == B.DEFAULT_PHASE_KEYS
    # the built library resolves phase_keys = 0 to the same length
    dk = B.DEFAULT_PHASE_KEYS
    assert lib.msa_sparse_prefill_workspace(P(n=dk), 0) == 0
    assert lib.msa_sparse_prefill_workspace(P(n=dk + 64), 0) > 0


def test_sparse_prefill_workspace_size(lib):
    # one phase (phase_keys >= seq_len, or the default with seq_len within it): none
    assert lib.msa_sparse_prefill_workspace(P(), 0) == 0
    assert lib.msa_sparse_prefill_workspace(P(), 4096) == 0
    assert lib.msa_sparse_prefill_workspace(P(n=1 << 17), 1 << 17) == 0
    # per q head and query block: two waves x (64 x 64 O + 64 max + 64 sum) fp32,
    # an 8-byte record (state stored, where the next phase's blocks start) and
    # a 4-byte mark of the query blocks the grouped walk takes
    per_item = 2 * (64 * 64 + 2 * 64) * 4 + 12
    assert lib.msa_sparse_prefill_workspace(P(), 1024) == 32 * 64 * per_item
    assert lib.msa_sparse_prefill_workspace(P(n=1 << 17), 0) == 32 * 2048 * per_item
    assert lib.msa_sparse_prefill_workspace(P(), 100) == 0          # invalid: not a multiple of 64
    assert lib.msa_sparse_prefill_workspace(P(d=64), 1024) == 0     # invalid problem


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros((4, 256, 128), dtype=torch.bfloat16)
    with pytest.raises(m.MsaError):
        m.dense_prefill(q, q[:1], q[:1])


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library every entry point raises; there is no
    fallback (CPU or otherwise) to compute anything."""
    import torch
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "_LIB_PATH", str(tmp_path / "libmsa.so"))
    q = torch.zeros((1, 64, 128), dtype=torch.bfloat16)
    with pytest.raises(B.MsaError, match="missing"):
        B.load()
    with pytest.raises(B.MsaError, match="missing"):
        B.dense_prefill(q, q, q)
    with pytest.raises(B.MsaError, match="missing"):
        B.sparse_prefill_workspace_bytes(1, 1, 64, phase_keys=16)


def test_alignment_validation(lib):
    odd = ctypes.c_void_p(0x1008)     # 8-byte aligned: not enough for row data or workspaces
    odd4 = ctypes.c_void_p(0x1002)    # not even 4-byte aligned
    assert lib.msa_dense_prefill(P(), odd, FAKE, FAKE, FAKE, None, None) == RANGE
    assert lib.msa_dense_prefill(P(), FAKE, FAKE, FAKE, odd, None, None) == RANGE
    assert lib.msa_dense_prefill(P(), FAKE, FAKE, FAKE, FAKE, odd4, None) == RANGE
    assert lib.msa_sparse_prefill(P(), FAKE, FAKE, odd, FAKE, FAKE, 64, FAKE, FAKE, 64, 0, FAKE, 1 << 30,
                                  FAKE, None, None) == RANGE
    assert lib.msa_sparse_prefill(P(), FAKE, FAKE, FAKE, odd4, FAKE, 64, FAKE, FAKE, 64, 0, FAKE, 1 << 30,
                                  FAKE, None, None) == RANGE
    assert lib.msa_estimate_vs(P(), FAKE, odd, 64, 8, 8, FAKE, FAKE, None, None, FAKE, 1 << 30, None) == RANGE
    assert lib.msa_estimate_vs(P(), FAKE, FAKE, 64, 8, 8, FAKE, FAKE, None, None, odd, 1 << 30, None) == RANGE
    assert lib.msa_estimate_vs(P(), FAKE, FAKE, 64, 8, 8, odd4, FAKE, None, None, FAKE, 1 << 30, None) == RANGE
    assert lib.msa_build_index(P(n=4096), FAKE, 64, FAKE, 256, 64, odd4, FAKE, 64, FAKE, FAKE, 64,
                               None) == RANGE
    assert lib.msa_estimate_bs(P(), odd, FAKE, 64, 8, FAKE, FAKE, 64, FAKE, FAKE, 1 << 30, None) == RANGE
    assert lib.msa_estimate_bs(P(), FAKE, FAKE, 64, 8, FAKE, FAKE, 64, FAKE, odd, 1 << 30, None) == RANGE
    assert b"aligned" in lib.msa_last_error()


def test_binding_rejects_mismatched_inputs(lib):
    """The binding checks shapes, dtypes and devices before any pointer reaches
    the library (CPU tensors: every case fails before the device check)."""
    import torch
    q = torch.zeros(4, 256, 128, dtype=torch.bfloat16)
    k = torch.zeros(2, 256, 128, dtype=torch.bfloat16)
    for kk, vv, what in [(k[:, :128], k, "rows per head"), (k.float(), k, "dtype"), (k, k[:1], "heads"),
                         (k, k[:, :200], "rows per head")]:
        with pytest.raises(B.MsaError, match=what):
            B.dense_prefill(q, kk, vv)
    with pytest.raises(B.MsaError, match="rows per head"):
        B.estimate_vs(q, k[:, :64], 8, 8)


def test_batch_fold_views():
    """Host logic of the batched calls: a contiguous [B, H, N, D] batch (or a
    slice of one along the sequence) folds into [B*H, N, D] views of the same
    memory in which q head b*H + h reads kv head (b*H + h) // G = b*Hkv + h // G;
    other layouts do not fold."""
    import torch
    from dynamic_sparse_attention_vertical_amd import layer as L
    Bn, H, Hkv, N, D = 3, 8, 2, 10, 128
    q = torch.arange(Bn * H * 16 * D, dtype=torch.float32).view(Bn, H, 16, D)[:, :, :N]
    k = torch.arange(Bn * Hkv * 16 * D, dtype=torch.float32).view(Bn, Hkv, 16, D)[:, :, :N]
    f = L._fold(q, k, k)
    assert f is not None
    qf, kf, _ = f
    assert qf.data_ptr() == q.data_ptr() and kf.data_ptr() == k.data_ptr()
    assert qf.stride(0) == 16 * D and kf.stride(0) == 16 * D       # head stride unchanged
    G = H // Hkv
    for b in range(Bn):
        for h in range(H):
            assert torch.equal(qf[b * H + h], q[b, h])
            assert torch.equal(kf[(b * H + h) // G], k[b, h // G])
    perm = q.transpose(0, 1).contiguous().transpose(0, 1)
    assert L._fold(perm, k, k) is None
    assert L._fold(q, k[:, :1].expand(Bn, 3, N, D), k) is None      # 8 q heads over 3 kv heads


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the refusal on a host without a GPU")
def test_graph_capture_refused_without_gpu():
    from dynamic_sparse_attention_vertical_amd.graphs import StepGraph
    with pytest.raises(m.MsaError):
        StepGraph(lambda: None)
