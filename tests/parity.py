"""Shared helpers for the GPU parity tests: tolerances and comparisons.

Tolerances (floating point):
  * bf16 path (bf16 in, fp32 accumulate, bf16 out): max |out - oracle| <= 2e-2,
    plus relative Frobenius error <= 1e-2 (near-uniform softmax over many keys
    makes |out| small, so the absolute bound alone would be weak).
  * fp32 path: max |out - oracle| <= 1e-4.
  * lse (natural log, fp32 on both paths): max abs error <= 1e-4.
  * estimator scores: |gpu - oracle| <= 1e-3 * oracle + 1e-6 (fp32 sums of fp32
    exponentials vs float64).
Index sets: exact, except entries whose oracle score lies within 1e-3
(relative) of the k-th largest score.
"""

from __future__ import annotations

import numpy as np

BF16_ATOL = 2e-2
BF16_REL_FRO = 1e-2
FP32_ATOL = 1e-4
LSE_ATOL = 1e-4
SCORE_RTOL = 1e-3
BAND = 1e-3


def compare_out(gpu, ref, fp32: bool, what: str = ""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    mx = float(err.max()) if err.size else 0.0
    if fp32:
        assert mx <= FP32_ATOL, f"{what} fp32 max abs err {mx:.3e}"
    else:
        assert mx <= BF16_ATOL, f"{what} bf16 max abs err {mx:.3e}"
        den = np.linalg.norm(ref)
        if den > 0:
            rel = float(np.linalg.norm(gpu - ref) / den)
            assert rel <= BF16_REL_FRO, f"{what} bf16 relative Frobenius err {rel:.3e}"
    return mx


def compare_lse(gpu, ref, what: str = ""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf_g, inf_r = np.isneginf(gpu), np.isneginf(ref)
    assert np.array_equal(inf_g, inf_r), f"{what} empty rows differ"
    fin = ~inf_r
    if fin.any():
        mx = float(np.abs(gpu[fin] - ref[fin]).max())
        assert mx <= LSE_ATOL, f"{what} lse max abs err {mx:.3e}"


def check_band(gpu_set, scores, k: int, what: str = ""):
    """GPU top-k set vs float64 oracle scores, with the 1e-3 tie band."""
    g = np.asarray(gpu_set, dtype=np.int64)
    x = np.asarray(scores, dtype=np.float64)
    assert len(g) == k and len(np.unique(g)) == k, f"{what}: size/distinctness"
    assert np.all(np.diff(g) > 0), f"{what}: not ascending"
    assert g.min() >= 0 and g.max() < len(x)
    xk = np.sort(x)[::-1][k - 1]
    must = np.nonzero(x > xk * (1 + BAND))[0]
    forbid = set(np.nonzero(x < xk * (1 - BAND))[0].tolist())
    gs = set(g.tolist())
    missing = [j for j in must.tolist() if j not in gs]
    assert not missing, f"{what}: {len(missing)} entries clearly above the k-th score missing"
    bad = gs & forbid
    assert not bad, f"{what}: {len(bad)} entries clearly below the k-th score selected"


def compare_index(gpu_idx, ref_idx, what: str = ""):
    """Work lists must match exactly up to each count."""
    bc = gpu_idx.block_count.cpu().numpy()
    cc = gpu_idx.column_count.cpu().numpy()
    assert np.array_equal(bc, ref_idx.block_count), f"{what}: block counts differ"
    assert np.array_equal(cc, ref_idx.column_count), f"{what}: column counts differ"
    # the two sides may use different capacities; counts fit in both
    wb = int(bc.max()) if bc.size else 0
    wc = int(cc.max()) if cc.size else 0
    bo = gpu_idx.block_offset[:, :, :wb].cpu().numpy()
    ci = gpu_idx.column_index[:, :, :wc].cpu().numpy()
    mb = np.arange(wb)[None, None, :] < bc[:, :, None]
    mc = np.arange(wc)[None, None, :] < cc[:, :, None]
    assert np.array_equal(bo[mb], ref_idx.block_offset[:, :, :wb][mb]), f"{what}: block offsets differ"
    assert np.array_equal(ci[mc], ref_idx.column_index[:, :, :wc][mc]), f"{what}: columns differ"


def to_oracle_index(gpu_idx):
    import oracle
    return oracle.IndexArrays(gpu_idx.block_count.cpu().numpy(), gpu_idx.block_offset.cpu().numpy(),
                              gpu_idx.column_count.cpu().numpy(), gpu_idx.column_index.cpu().numpy())
