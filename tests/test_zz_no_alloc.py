"""msa_estimate_vs_noalloc (the estimate with the library's own per-GPU
scratch instead of a workspace) against msa_estimate_vs (caller workspace):
same index sets and scores, on two calls in a row, the second smaller than the
first, so that the scratch holds the first call's contents when the second
starts.  Also: a problem whose scratch would exceed the array is refused."""

import pytest
import torch

import dynamic_sparse_attention_vertical_amd as msa
from synth import make_inputs, small_workload

pytestmark = pytest.mark.gpu


def _inputs(hq, hkv, n, seed):
    w = small_workload(n_q_heads=hq, n_kv_heads=hkv, seq_len=n, seed=seed, n_planted=4)
    x = make_inputs(w, device="cuda")
    return x["q"], x["k"]


def _both(q, k, kv, ks):
    hq, n = q.shape[0], q.shape[1]
    f32 = dict(dtype=torch.float32, device="cuda")
    vs_a, ss_a = torch.empty((hq, n), **f32), torch.empty((hq, n), **f32)
    va, sa = msa.estimate_vs(q, k, kv, ks, v_score=vs_a, s_score=ss_a)
    vs_b, ss_b = torch.full((hq, n), -1.0, **f32), torch.full((hq, n), -1.0, **f32)
    vb, sb = msa.estimate_vs_noalloc(q, k, kv, ks, v_score=vs_b, s_score=ss_b)
    torch.cuda.synchronize()
    return (va, sa, vs_a, ss_a), (vb, sb, vs_b, ss_b)


def test_noalloc_matches_workspace_call_twice():
    cases = [(32, 8, 131072, 1000, 6096, 1), (4, 1, 4096 + 37, 64, 256, 2)]   # the second is smaller
    for hq, hkv, n, kv, ks, seed in cases:
        print(f"[no-alloc] hq={hq} hkv={hkv} n={n} kv={kv} ks={ks}", flush=True)
        q, k = _inputs(hq, hkv, n, seed)
        ref, got = _both(q, k, kv, ks)
        for r, g, name in zip(ref, got, ("v_idx", "s_idx", "v_score", "s_score")):
            # same kernels, same inputs, deterministic (no float atomics): bit for bit
            assert torch.equal(r, g), f"{name} differs at n={n}"


def test_noalloc_refuses_problems_above_its_scratch():
    q = torch.empty((32, 1 << 20, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((8, 1 << 20, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(msa.MsaError, match="MSA_ERR_WORKSPACE"):
        msa.estimate_vs_noalloc(q, k, 1000, 6096)
