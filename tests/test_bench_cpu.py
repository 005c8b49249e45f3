"""bench.py logic that needs no GPU: the phase-launch count, the counter
traffic records' source-hash guards (prefill and decode), the refusal of more than one GPU, and the
band workload's shape."""

import json
import os
import subprocess
import sys

import bench
from synth import WORKLOADS, make_inputs, small_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_phase_launches():
    from dynamic_sparse_attention_vertical_amd.msa import DEFAULT_PHASE_KEYS as R
    # one launch when one phase covers the sequence; else the grouped walk
    # and one launch per phase
    assert bench.phase_launches(R) == 1
    assert bench.phase_launches(R + 64) == 3
    assert bench.phase_launches(1 << 17) == 1 + -(-(1 << 17) // R)     # a short last phase counts
    assert bench.phase_launches(1 << 20) == 1 + -(-(1 << 20) // R)
    assert bench.phase_launches(3 * R) == 4


def test_traffic_record_follows_the_kernel_source(tmp_path, monkeypatch):
    rec = {"workloads": {"w": {"fetch_kib_per_step": 10.0, "write_kib_per_step": 2.0}},
           "attention_src_sha": bench.attn_src_sha(), "fetch_calib": 2.0, "write_calib": 1.0}
    f = tmp_path / "t.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("w") == 10.0 * 1024 * 2.0 + 2.0 * 1024 * 1.0
    assert bench.measured_traffic("other") is None
    rec["attention_src_sha"] = "0" * 16                     # taken on another kernel source
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic("w") is None


def test_decode_traffic_record_follows_the_sources(tmp_path, monkeypatch):
    import hashlib
    csrc = os.path.join(ROOT, "dynamic_sparse_attention_vertical_amd", "csrc")
    sha = {n: hashlib.sha256(open(os.path.join(csrc, n), "rb").read()).hexdigest()[:16]
           for n in ("decode.hip", "topk.hip", "msa_api.hip")}
    rec = {"workloads": {"d": {"fetch_kib_per_step": 4.0, "write_kib_per_step": 1.0}},
           "src_sha": sha, "fetch_calib": 2.0, "write_calib": 1.0}
    f = tmp_path / "d.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "DECODE_TRAFFIC_FILE", str(f))
    assert bench.measured_decode_traffic("d") == 4.0 * 1024 * 2.0 + 1.0 * 1024
    assert bench.measured_decode_traffic("other") is None
    rec["src_sha"]["topk.hip"] = "0" * 16                   # taken on another top-k source
    f.write_text(json.dumps(rec))
    assert bench.measured_decode_traffic("d") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_band_workload_gathers_slashes():
    w = WORKLOADS["llama3_8b_1m_band"]
    assert (w.band, w.band_pairs, w.slash_period) == (12.0, 48, 512)
    # the shared direction raises <q_i, k_j> near the diagonal: small case, no RoPE
    sw = small_workload(seq_len=256, n_q_heads=1, n_kv_heads=1, n_planted=0, band=12.0, band_pairs=48,
                        rope_base=1e30)
    x = make_inputs(sw)
    z = (x["q"][0].double() @ x["k"][0].double().T).diagonal().mean()
    y = make_inputs(small_workload(seq_len=256, n_q_heads=1, n_kv_heads=1, n_planted=0, rope_base=1e30))
    z0 = (y["q"][0].double() @ y["k"][0].double().T).diagonal().mean()
    assert z > z0 + 100


def test_listed_and_executed_tiles():
    """Listed tiles count blocks and 64-column chunks; a query block the
    grouped walk took counts all aligned tiles 0..b instead."""
    import torch
    from dynamic_sparse_attention_vertical_amd.msa import IndexTensors
    bc = torch.tensor([[1, 2, 1], [0, 1, 3]], dtype=torch.int32)
    cc = torch.tensor([[0, 65, 3], [1, 0, 64]], dtype=torch.int32)
    idx = IndexTensors(bc, torch.zeros((2, 3, 3), dtype=torch.int32), cc, torch.zeros((2, 3, 65), dtype=torch.int32))
    assert bench.listed_tiles(idx) == (1 + 2 + 1 + 0 + 1 + 3) + (0 + 2 + 1 + 1 + 0 + 1)
    assert bench.executed_tiles(idx, None) == (bench.listed_tiles(idx), 0)
    marks = torch.tensor([[0, 0, 1], [1, 0, 1]], dtype=torch.int32)
    # walked: (h0, b2) -> 3 tiles, (h1, b0) -> 1, (h1, b2) -> 3; the rest as listed
    assert bench.executed_tiles(idx, marks) == ((1) + (2 + 2) + 3 + 1 + (1 + 0) + 3, 3)
