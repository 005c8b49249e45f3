"""Synthetic long-context attention inputs.

The five named workloads are stand-ins for the long-context LLM prefill
workloads the MInference pages measure on (LLaMA-3-8B-1M-style layers, 128K to
1M tokens; "MInference 1.0 README", section "TL;DR"; talk slides
"System-Algorithm Co-design", slide "Dynamic sparsity in attention").  No
model weights or datasets are used: Q, K and V are Gaussian, rotated with
rotary position embedding (base 500000, rotate-half form) and given planted
structure so that vertical lines (attention sinks, heavy columns) and slash
lines (equidistant diagonals) exist for the estimator to find.

Everything here is input shaping; none of it is the method's arithmetic.

Generation:
  * CPU (small cases, tests): Q/K/V drawn in float64, rotated and planted in
    float64, then rounded to float32 (round-to-nearest-even) and from there to
    bfloat16, so the float32 and bfloat16 copies share one draw.
  * GPU (the 128K-1M workloads): same recipe in float32 on the device, with the
    rotary angles computed in float64 and chunked over positions.
Each (workload, seed, device) triple is deterministic.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    name: str
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    head_dim: int = HEAD_DIM
    dtypes: tuple = ("bf16",)
    vertical_topk: int = 1000
    slash_topk: int = 6096
    last_q: int = 64
    block: int = 64
    rope_base: float = 500000.0
    n_planted: int = 16          # planted vertical columns per kv head, key 0 included
    plant_gain: float = 3.0      # K[col] += gain * mean(q)
    slash_period: int = 0        # >0: keys at offset multiples of this are biased toward q
    band: float = 0.0            # >0: a content direction shared by all q and k of a kv group
    band_pairs: int = 64         # rotary pairs (fastest first) the shared direction occupies
    head_patterns: tuple = field(default_factory=tuple)  # per q head: "vs" | "a" | "bs"
    sink: int = 128              # A-shape: leading columns kept
    window: int = 4096           # A-shape: local diagonals kept
    bs_topk: int = 100           # block-sparse: key blocks kept per query block
    seed: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_blocks(self) -> int:
        return self.seq_len // self.block

    def pattern(self, h: int) -> str:
        return self.head_patterns[h] if self.head_patterns else "vs"

    def heads_with(self, pat: str) -> list:
        return [h for h in range(self.n_q_heads) if self.pattern(h) == pat]


def _mixed_patterns(n: int = 32) -> tuple:
    return tuple("a" if h < 8 else ("vs" if h < 24 else "bs") for h in range(n))


WORKLOADS = {
    # single head, 4K tokens, float32 and bfloat16 copies of one draw
    "single_head_4k": Workload("single_head_4k", 1, 1, 4096, dtypes=("fp32", "bf16"),
                               vertical_topk=64, slash_topk=256, n_planted=9, seed=1001),
    # LLaMA-3-8B attention layer shape (32 q / 8 kv heads, GQA 4:1)
    "llama3_8b_128k": Workload("llama3_8b_128k", 32, 8, 131072, seed=1002),
    "llama3_8b_512k": Workload("llama3_8b_512k", 32, 8, 524288, slash_period=512, seed=1003),
    "llama3_8b_1m": Workload("llama3_8b_1m", 32, 8, 1048576, slash_period=512, seed=1004),
    # heads 0-7 A-shape, 8-23 vertical-slash, 24-31 block-sparse
    "mixed_256k": Workload("mixed_256k", 32, 8, 262144, head_patterns=_mixed_patterns(), seed=1005),
    # clustered slashes ("local band"): the 1M layer plus a shared content
    # direction on the 48 fastest rotary pairs, so that the selected diagonals
    # gather near the main diagonal (a labelled extra workload, not one of the
    # five above)
    "llama3_8b_1m_band": Workload("llama3_8b_1m_band", 32, 8, 1048576, slash_period=512, band=12.0,
                                  band_pairs=48, seed=1006),
}


@dataclass(frozen=True)
class DecodeWorkload:
    """One decode step over a batch of key caches: batch sequences of
    cache_len cached tokens, each with the layer's q / kv heads; the decode
    query of a sequence is the last query row of its synthetic prefill.  With
    lengths, sequence b holds lengths[b] tokens in a cache of capacity
    cache_len."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    cache_len: int
    topk: int
    seed: int = 0
    lengths: tuple = ()

    def length(self, b: int) -> int:
        return self.lengths[b] if self.lengths else self.cache_len

    def prefill(self, b: int) -> Workload:
        return Workload(f"{self.name}_{b}", self.n_q_heads, self.n_kv_heads, self.length(b), seed=self.seed + b)


DECODE_WORKLOADS = {
    # LLaMA-3-8B attention shape decoding over 100K cached tokens, top-1000
    # keys per head (the talk slides' decoding panel), 8 sequences at once
    "llama3_8b_decode_100k": DecodeWorkload("llama3_8b_decode_100k", 8, 32, 8, 100000, 1000, seed=2001),
    # the same shape with the sequences at different positions: caches of
    # capacity 128K holding 4K to 128K tokens (485,584 in all)
    "llama3_8b_decode_varlen": DecodeWorkload("llama3_8b_decode_varlen", 8, 32, 8, 131072, 1000, seed=2101,
                                              lengths=(131072, 98304, 65536, 40000, 24576, 12000, 110000, 4096)),
}


def make_decode_inputs(dw: DecodeWorkload, device: str = "cpu") -> dict:
    """q [batch * Hq, D] (each sequence's last query row), k and v caches
    [batch * Hkv, cache_len, D], bfloat16; sequences folded into the heads.
    With lengths, sequence b's keys fill the first lengths[b] rows of its
    caches (the rest zero) and cache_lens [batch] int32 is returned too."""
    qs, ks, vs = [], [], []
    for b in range(dw.batch):
        x = make_inputs(dw.prefill(b), device=device)
        qs.append(x["q"][:, -1].clone())
        L = dw.length(b)
        if L == dw.cache_len:
            ks.append(x["k"])
            vs.append(x["v"])
        else:
            for src, dst in ((x["k"], ks), (x["v"], vs)):
                buf = torch.zeros((src.shape[0], dw.cache_len, src.shape[2]), dtype=src.dtype, device=device)
                buf[:, :L] = src
                dst.append(buf)
        del x
    res = {"q": torch.cat(qs).contiguous(), "k": torch.cat(ks), "v": torch.cat(vs)}
    if dw.lengths:
        res["cache_lens"] = torch.tensor([dw.length(b) for b in range(dw.batch)], dtype=torch.int32, device=device)
    return res


@dataclass(frozen=True)
class PackedWorkload:
    """A prefill batch of sequences of different lengths packed along the
    rows ([heads, total, D], sequence i at rows cu[i] .. cu[i+1]-1), each of
    the single-sequence recipe with its own seed."""
    name: str
    n_q_heads: int
    n_kv_heads: int
    lengths: tuple
    vertical_topk: int = 1000
    slash_topk: int = 6096
    seed: int = 0

    def sequence(self, i: int) -> Workload:
        return Workload(f"{self.name}_{i}", self.n_q_heads, self.n_kv_heads, self.lengths[i],
                        vertical_topk=self.vertical_topk, slash_topk=self.slash_topk, seed=self.seed + i)


PACKED_WORKLOADS = {
    # LLaMA-3-8B attention shape, 64 prompts of 1,062 to 32,444 tokens
    # (516,245 in all; lengths drawn once, log-uniform over 1K..32K, seed 2201)
    "llama3_8b_packed_64": PackedWorkload("llama3_8b_packed_64", 32, 8, (
        13039, 1674, 12436, 11505, 11600, 22901, 1363, 17329, 22318, 5504, 3218, 16594, 3164, 1512, 3054, 32444,
        6841, 8179, 2492, 2748, 4455, 5982, 3093, 9549, 1461, 3920, 2841, 3023, 4602, 2838, 20765, 15880, 4435,
        2140, 8080, 3913, 3511, 2809, 1974, 9432, 4318, 10344, 6202, 1717, 1454, 2281, 5094, 14056, 1165, 1561,
        9677, 1679, 21155, 12621, 1858, 27981, 14001, 1481, 1062, 2025, 19360, 25824, 4118, 10593), seed=2301),
}


def make_packed_inputs(pw: PackedWorkload, device: str = "cpu") -> dict:
    """q [Hq, total, D], k and v [Hkv, total, D] (bfloat16) with the
    sequences one after another, and cu_seqlens (a list)."""
    qs, ks, vs = [], [], []
    for i in range(len(pw.lengths)):
        x = make_inputs(pw.sequence(i), device=device)
        qs.append(x["q"])
        ks.append(x["k"])
        vs.append(x["v"])
        del x
    cu = [0]
    for n in pw.lengths:
        cu.append(cu[-1] + n)
    return {"q": torch.cat(qs, dim=1), "k": torch.cat(ks, dim=1), "v": torch.cat(vs, dim=1), "cu_seqlens": cu}


def small_workload(name: str = "small", **kw) -> Workload:
    """A test-sized workload (same recipe, smaller shapes)."""
    base = dict(n_q_heads=4, n_kv_heads=1, seq_len=1024, vertical_topk=64, slash_topk=128,
                n_planted=5, seed=7)
    base.update(kw)
    return Workload(name, **base)


def rope_tables(positions: torch.Tensor, head_dim: int, base: float, dtype: torch.dtype):
    """cos/sin tables [len(positions), head_dim/2] for rotate-half rotary embedding.

    Angles are formed in float64 (position * base^(-2i/head_dim)) and cast once.
    """
    half = head_dim // 2
    inv_freq = base ** (-(torch.arange(half, dtype=torch.float64, device=positions.device) * 2.0)
                        / head_dim)
    ang = positions.to(torch.float64)[:, None] * inv_freq[None, :]
    return torch.cos(ang).to(dtype), torch.sin(ang).to(dtype)


def _rotate_(x: torch.Tensor, base: float, chunk: int) -> None:
    """In-place rotate-half rotary embedding over positions 0..N-1 of x [H, N, D]."""
    H, N, D = x.shape
    half = D // 2
    for p0 in range(0, N, chunk):
        p1 = min(N, p0 + chunk)
        cos, sin = rope_tables(torch.arange(p0, p1, device=x.device), D, base, x.dtype)
        x1 = x[:, p0:p1, :half].clone()
        x2 = x[:, p0:p1, half:].clone()
        x[:, p0:p1, :half] = x1 * cos - x2 * sin
        x[:, p0:p1, half:] = x2 * cos + x1 * sin


def _planted_columns(w: Workload, seed: int) -> torch.Tensor:
    """Per kv head: key 0 plus (n_planted-1) distinct random keys in [1, N)."""
    g = torch.Generator(device="cpu").manual_seed(seed * 7919 + 17)
    cols = []
    for _ in range(w.n_kv_heads):
        extra = torch.randperm(w.seq_len - 1, generator=g)[: w.n_planted - 1] + 1
        cols.append(torch.cat([torch.zeros(1, dtype=torch.long), torch.sort(extra).values]))
    return torch.stack(cols)


def _plant_(w: Workload, q: torch.Tensor, k: torch.Tensor, planted: torch.Tensor) -> None:
    G, N, D = w.group, w.seq_len, w.head_dim
    for g in range(w.n_kv_heads):
        qg = q[g * G:(g + 1) * G]
        if w.n_planted > 0:
            qbar = qg.mean(dim=(0, 1))                       # mean over positions and group heads
            cols = planted[g].to(k.device)
            k[g, cols] += w.plant_gain * qbar
        if w.slash_period > 0:
            P = w.slash_period
            assert N % P == 0
            qpos = qg.mean(dim=0).reshape(N // P, P, D)      # per-position group mean
            incl = torch.flip(torch.cumsum(torch.flip(qpos, [0]), 0), [0])
            excl = incl - qpos                               # sum over later positions j+P*m, m>=1
            cnt = (N // P - 1 - torch.arange(N // P, device=q.device, dtype=q.dtype))
            boost = torch.where(cnt[:, None, None] > 0,
                                excl / cnt.clamp(min=1)[:, None, None],
                                torch.zeros((), dtype=q.dtype, device=q.device))
            k[g] += w.plant_gain * boost.reshape(N, D)


def make_inputs(w: Workload, seed: int | None = None, device: str = "cpu") -> dict:
    """Draw Q [Hq,N,D], K and V [Hkv,N,D] for workload w.

    Returns a dict with 'q','k','v' in bfloat16 (when "bf16" is in w.dtypes),
    'q32','k32','v32' in float32 (when "fp32" is in w.dtypes), and 'planted'
    (the planted vertical columns, [Hkv, n_planted]).
    """
    seed = w.seed if seed is None else seed
    dev = torch.device(device)
    work = torch.float64 if dev.type == "cpu" else torch.float32
    gen = torch.Generator(device=dev).manual_seed(int(seed))
    Hq, Hkv, N, D = w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim
    q = torch.randn((Hq, N, D), generator=gen, dtype=work, device=dev)
    k = torch.randn((Hkv, N, D), generator=gen, dtype=work, device=dev)
    v = torch.randn((Hkv, N, D), generator=gen, dtype=work, device=dev)
    if w.band > 0:
        # local band: every query and key of kv group g gets band * u_g (a
        # random unit vector) before the rotation, so q_i . k_j carries
        # band^2 * sum_f |u_g,f|^2 cos((i - j) theta_f): largest near the
        # diagonal and decaying with the offset, as rotary embeddings do
        # (faster the fewer and faster the rotary pairs u occupies)
        u = torch.randn((Hkv, D), generator=gen, dtype=work, device=dev)
        keep = (torch.arange(D, device=dev) % (D // 2)) < w.band_pairs
        u = torch.where(keep, u, torch.zeros((), dtype=work, device=dev))
        u = u / u.norm(dim=1, keepdim=True)
        G = Hq // Hkv
        q += w.band * u.repeat_interleave(G, dim=0)[:, None, :]
        k += w.band * u[:, None, :]
    chunk = 1 << 16
    _rotate_(q, w.rope_base, chunk)
    _rotate_(k, w.rope_base, chunk)
    planted = _planted_columns(w, seed) if w.n_planted > 0 else torch.zeros((Hkv, 0), dtype=torch.long)
    _plant_(w, q, k, planted)
    out = {"planted": planted}
    for name, t in (("q", q), ("k", k), ("v", v)):
        t32 = t.to(torch.float32)
        del t
        if "fp32" in w.dtypes:
            out[name + "32"] = t32.contiguous()
        if "bf16" in w.dtypes:
            out[name] = t32.to(torch.bfloat16).contiguous()
        del t32
    return out


def with_seq_len(w: Workload, n: int) -> Workload:
    return replace(w, seq_len=n)
