"""Input generator: determinism, shapes, rounding, planted structure."""

import torch

from synth import WORKLOADS, make_inputs, small_workload


def test_named_workloads_shapes():
    w = WORKLOADS["llama3_8b_1m"]
    assert (w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim) == (32, 8, 1 << 20, 128)
    assert (w.vertical_topk, w.slash_topk, w.last_q, w.block) == (1000, 6096, 64, 64)
    m = WORKLOADS["mixed_256k"]
    assert m.heads_with("a") == list(range(8)) and m.heads_with("bs") == list(range(24, 32))
    s = WORKLOADS["single_head_4k"]
    assert s.dtypes == ("fp32", "bf16") and (s.vertical_topk, s.slash_topk) == (64, 256)


def test_deterministic_and_rounded():
    w = small_workload(seq_len=512, dtypes=("fp32", "bf16"))
    a = make_inputs(w)
    b = make_inputs(w)
    for name in ("q", "k", "v", "q32", "k32", "v32"):
        assert torch.equal(a[name], b[name])
    # bf16 copy is the round-to-nearest-even of the float32 copy
    assert torch.equal(a["q"], a["q32"].to(torch.bfloat16))
    assert a["q"].shape == (4, 512, 128) and a["k"].shape == (1, 512, 128)
    c = make_inputs(w, seed=w.seed + 1)
    assert not torch.equal(a["q"], c["q"])


def test_planted_columns_present():
    w = small_workload(seq_len=1024, n_planted=5)
    x = make_inputs(w)
    assert x["planted"].shape == (1, 5) and int(x["planted"][0, 0]) == 0
    assert len(set(x["planted"][0].tolist())) == 5


def test_periodic_boost_biases_offsets():
    """Keys at offset multiples of the period get pulled toward the queries that
    sit one period later."""
    w = small_workload(seq_len=2048, slash_period=256, n_planted=0, n_q_heads=1, seed=3)
    x = make_inputs(w)
    w0 = small_workload(seq_len=2048, slash_period=0, n_planted=0, n_q_heads=1, seed=3)
    y = make_inputs(w0)
    q = x["q32"] if "q32" in x else x["q"].float()
    dk = x["k"].float() - y["k"].float()
    # boost of key j is 3 * mean of later same-residue queries: for j = N-1-256 it is 3 q[N-1]
    j = 2048 - 1 - 256
    assert torch.allclose(dk[0, j], 3 * q[0, 2047], atol=0.1)
