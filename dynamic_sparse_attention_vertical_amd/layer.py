"""One attention layer's sparse prefill, composed from the C-ABI steps.

vertical_slash_layer is the composition the MInference README exposes as one
kernel-only call, vertical_slash_sparse_attention(q, k, v, vertical_topk,
slash) ("MInference 1.0 README", section "How to use MInference", kernel-only
usage): estimate the index online, build the work lists, run the sparse
kernel.  mixed_layer runs heads with different patterns in one layer (A-shape,
vertical-slash and block-sparse heads, the three patterns of talk slides
"System-Algorithm Co-design", patterns slide), sharing one sparse-attention
launch.  Buffers can be preallocated once (LayerPlan) so repeated calls
allocate nothing.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import msa


@dataclass
class LayerPlan:
    """Preallocated device buffers for one layer shape."""
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    vertical_topk: int
    slash_topk: int
    device: str = "cuda"
    dtype: torch.dtype = torch.bfloat16
    index: msa.IndexTensors = field(init=False)
    workspace: torch.Tensor = field(init=False)
    attn_workspace: torch.Tensor | None = field(init=False)
    v_idx: torch.Tensor = field(init=False)
    s_idx: torch.Tensor = field(init=False)

    def __post_init__(self):
        cb, cc = msa.index_caps(self.seq_len, self.vertical_topk, self.slash_topk, self.n_q_heads)
        self.index = msa.alloc_index(self.n_q_heads, self.seq_len, cb, cc, self.device)
        ws = msa.estimate_vs_workspace_bytes(self.n_q_heads, self.n_kv_heads, self.seq_len, self.dtype)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.device)
        aws = msa.sparse_prefill_workspace_bytes(self.n_q_heads, self.n_kv_heads, self.seq_len, self.dtype)
        self.attn_workspace = torch.empty(aws, dtype=torch.uint8, device=self.device) if aws else None
        i32 = dict(dtype=torch.int32, device=self.device)
        self.v_idx = torch.empty((self.n_q_heads, self.vertical_topk), **i32)
        self.s_idx = torch.empty((self.n_q_heads, self.slash_topk), **i32)


@msa.on_stream
def vertical_slash_layer(q, k, v, vertical_topk: int, slash_topk: int, *, plan: LayerPlan | None = None,
                         out: torch.Tensor | None = None, lse=None, stream=None):
    """Estimate + build index + sparse prefill for every head of q.

    Returns (out, plan); plan.v_idx / plan.s_idx / plan.index hold the index."""
    hq, n = q.shape[0], q.shape[1]
    if plan is None:
        plan = LayerPlan(hq, k.shape[0], n, vertical_topk, slash_topk, str(q.device), q.dtype)
    msa.estimate_vs(q, k, vertical_topk, slash_topk, workspace=plan.workspace, v_idx=plan.v_idx,
                    s_idx=plan.s_idx, stream=stream)
    msa.build_index(plan.v_idx, plan.s_idx, n, out=plan.index, stream=stream)
    res = msa.sparse_prefill(q, k, v, plan.index, out=out, lse=lse, workspace=plan.attn_workspace,
                             stream=stream)
    return res, plan


def _slice_index(idx: msa.IndexTensors, h0: int, h1: int) -> msa.IndexTensors:
    return msa.IndexTensors(idx.block_count[h0:h1], idx.block_offset[h0:h1],
                            idx.column_count[h0:h1], idx.column_index[h0:h1])


def _runs(patterns, pat):
    """Contiguous head ranges [h0, h1) with pattern pat."""
    out, h = [], 0
    while h < len(patterns):
        if patterns[h] == pat:
            h1 = h
            while h1 < len(patterns) and patterns[h1] == pat:
                h1 += 1
            out.append((h, h1))
            h = h1
        else:
            h += 1
    return out


@dataclass
class MixedPlan:
    patterns: tuple
    n_kv_heads: int
    seq_len: int
    vertical_topk: int
    slash_topk: int
    sink: int
    window: int
    bs_topk: int
    device: str = "cuda"
    dtype: torch.dtype = torch.bfloat16
    index: msa.IndexTensors = field(init=False)

    def __post_init__(self):
        n, hq = self.seq_len, len(self.patterns)
        nqb = (n + msa.BLOCK - 1) // msa.BLOCK
        caps = [(0, 0)]
        if "vs" in self.patterns:
            caps.append(msa.index_caps(n, self.vertical_topk, self.slash_topk, 1))
        if "a" in self.patterns:
            caps.append(msa.index_caps(n, min(self.sink, n), min(self.window, n), 1))
        if "bs" in self.patterns:
            caps.append((min(self.bs_topk, nqb), 0))
        cb = max(c[0] for c in caps)
        cc = max(c[1] for c in caps)
        self.index = msa.alloc_index(hq, n, cb, cc, self.device)
        i32 = dict(dtype=torch.int32, device=self.device)
        na = max(sum(p == "a" for p in self.patterns), 1)
        self.a_v = torch.arange(min(self.sink, n), **i32).expand(na, -1).contiguous()
        self.a_s = torch.arange(min(self.window, n), **i32).expand(na, -1).contiguous()
        nvs = sum(p == "vs" for p in self.patterns)
        self.v_idx = torch.empty((max(nvs, 1), self.vertical_topk), **i32)
        self.s_idx = torch.empty((max(nvs, 1), self.slash_topk), **i32)
        G = hq // self.n_kv_heads
        ws_vs = max([msa.estimate_vs_workspace_bytes(h1 - h0, (h1 - h0) // G, n, self.dtype)
                     for h0, h1 in _runs(self.patterns, "vs")] or [0])
        self.workspace = torch.empty(max(ws_vs, 1), dtype=torch.uint8, device=self.device)
        ws_bs = max([msa.estimate_bs_workspace_bytes(h1 - h0, (h1 - h0) // G, n, self.dtype)
                     for h0, h1 in _runs(self.patterns, "bs")] or [0])
        self.bs_workspace = torch.empty(max(ws_bs, 1), dtype=torch.uint8, device=self.device)
        aws = msa.sparse_prefill_workspace_bytes(hq, self.n_kv_heads, n, self.dtype)
        self.attn_workspace = torch.empty(aws, dtype=torch.uint8, device=self.device) if aws else None


@msa.on_stream
def mixed_index(q, k, plan: MixedPlan, *, stream=None) -> msa.IndexTensors:
    """Work lists of every head of a mixed layer: 'a' (static sink + window
    index), 'vs' (online vertical-slash estimate) and 'bs' (online
    block-sparse estimate), written into plan.index.  Head runs must align
    with kv groups."""
    hq, n = q.shape[0], q.shape[1]
    G = hq // k.shape[0]
    vs_row = 0
    for pat in ("a", "vs", "bs"):
        for h0, h1 in _runs(plan.patterns, pat):
            if h0 % G or h1 % G:
                raise msa.MsaError("pattern runs must align with kv-head groups")
            qs, ks_ = q[h0:h1], k[h0 // G: h1 // G]
            sub = _slice_index(plan.index, h0, h1)
            if pat == "a":
                nh = h1 - h0
                msa.build_index(plan.a_v[:nh], plan.a_s[:nh], n, out=sub, stream=stream)
            elif pat == "vs":
                nh = h1 - h0
                vi, si = plan.v_idx[vs_row: vs_row + nh], plan.s_idx[vs_row: vs_row + nh]
                vs_row += nh
                msa.estimate_vs(qs, ks_, plan.vertical_topk, plan.slash_topk, workspace=plan.workspace,
                                v_idx=vi, s_idx=si, stream=stream)
                msa.build_index(vi, si, n, out=sub, stream=stream)
            else:
                msa.estimate_bs(qs, ks_, plan.bs_topk, out=sub, workspace=plan.bs_workspace, stream=stream)
    return plan.index


@msa.on_stream
def mixed_layer(q, k, v, plan: MixedPlan, *, out: torch.Tensor | None = None, lse=None, stream=None):
    """Per-head patterns in one layer (see mixed_index), then a single sparse
    prefill over all heads."""
    mixed_index(q, k, plan, stream=stream)
    return msa.sparse_prefill(q, k, v, plan.index, out=out, lse=lse, workspace=plan.attn_workspace,
                              stream=stream)


# ---------------------------------------------------------------------------
# The README's kernel-only calls ("MInference 1.0 README", section "How to use
# MInference", kernel-only usage: vertical_slash_sparse_attention,
# block_sparse_attention, streaming_forward), on [batch, heads, seq, dim] or
# [heads, seq, dim] tensors, or on a packed batch of sequences of different
# lengths ([heads, total, dim] with cu_seqlens, sequence i being rows
# cu_seqlens[i] .. cu_seqlens[i+1]-1).  A batch whose batch stride is heads x
# the head stride (a contiguous [B, H, N, D] tensor, or a slice of one along
# the sequence) runs as one problem of B*H heads: one launch chain for the
# whole batch.  A packed batch runs as one problem too, through the C ABI's
# variable-length calls (one launch chain for all sequences).  Other batch
# layouts run one element after another on the stream through the same C-ABI
# steps.


def _cu_list(q, k, v, cu_seqlens):
    """cu_seqlens checked on the host: a list rising strictly from 0 to the
    packed length."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise msa.MsaError("packed q, k, v must be [heads, total, dim]")
    cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    if len(cu) < 2 or cu[0] != 0 or cu[-1] != q.shape[1] or any(b <= a for a, b in zip(cu, cu[1:])):
        raise msa.MsaError("cu_seqlens must rise strictly from 0 to the packed length")
    return cu


def _packed_varlen(q, k, v, cu_seqlens, sets, stream):
    """Attention of a packed batch over the cover of per-head index sets in
    one launch chain: sets(cu_dev, max_len) gives v_idx, s_idx for the
    n_seqs * heads heads."""
    cu = _cu_list(q, k, v, cu_seqlens)
    max_len = max(b - a for a, b in zip(cu, cu[1:]))
    cu_dev = torch.tensor(cu, dtype=torch.int32, device=q.device)
    v_idx, s_idx = sets(cu_dev, max_len)
    idx = msa.build_index_varlen(v_idx, s_idx, cu_dev, max_len, q.shape[0], rows=q.shape[1], stream=stream)
    return msa.sparse_prefill_varlen(q, k, v, idx, cu_dev, max_len, stream=stream)

def _batched(q, k, v):
    if q.dim() == 3:
        return q[None], k[None], v[None], True
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape[0] != q.shape[0] or v.shape[0] != q.shape[0]:
        raise msa.MsaError("q, k, v must all be [batch, heads, seq, dim] (or all [heads, seq, dim])")
    return q, k, v, False


def _fold(q4, k4, v4):
    """[B, H, N, D] inputs as [B*H, N, D] views of the same memory, or None
    when a tensor's batch stride is not H head strides.  Head h of batch
    element b becomes head b*H + h; with H = G*Hkv its kv head under the C
    ABI's mapping (q head // G) is b*Hkv + h // G, the same element's."""
    if any(t.shape[1] > 1 and t.stride(0) != t.shape[1] * t.stride(1) for t in (q4, k4, v4)):
        return None
    if q4.shape[1] % k4.shape[1]:
        return None                     # leave the head-count error to the per-element call
    try:
        return tuple(t.view(t.shape[0] * t.shape[1], t.shape[2], t.shape[3]) for t in (q4, k4, v4))
    except RuntimeError:
        return None


def _rows(t):
    """Rows between heads of a [heads, seq, dim] view."""
    return t.stride(0) // t.shape[2] if t.shape[0] > 1 else t.shape[1]


def _unfold(out, q4):
    return out.view(q4.shape[0], q4.shape[1], out.shape[1], out.shape[2])


@msa.on_stream
def vertical_slash_sparse_attention(q, k, v, vertical_topk: int, slash_topk: int, *, cu_seqlens=None,
                                    stream=None):
    """Vertical-slash sparse attention: per head, the vertical_topk key columns
    and slash_topk diagonals the online estimate selects, then causal
    attention over their 64-wide block cover.  Returns the attention output."""
    if cu_seqlens is not None:
        # each sequence estimated, indexed and attended as on its own (a
        # sequence of at most k tokens selects all of them); one launch chain
        def sets(cu_dev, max_len):
            return msa.estimate_vs_varlen(q, k, cu_dev, max_len, min(vertical_topk, max_len),
                                          min(slash_topk, max_len), stream=stream)
        return _packed_varlen(q, k, v, cu_seqlens, sets, stream)
    q4, k4, v4, squeeze = _batched(q, k, v)
    f = _fold(q4, k4, v4)
    if f is not None:
        out, _ = vertical_slash_layer(*f, vertical_topk, slash_topk, stream=stream)
        out = _unfold(out, q4)
        return out[0] if squeeze else out
    out = torch.empty_like(q4)
    plan = LayerPlan(q4.shape[1], k4.shape[1], q4.shape[2], vertical_topk, slash_topk, str(q4.device), q4.dtype)
    for bi in range(q4.shape[0]):
        vertical_slash_layer(q4[bi], k4[bi], v4[bi], vertical_topk, slash_topk, plan=plan, out=out[bi],
                             stream=stream)
    return out[0] if squeeze else out


@msa.on_stream
def block_sparse_attention(q, k, v, topk: int, *, cu_seqlens=None, stream=None):
    """Block-sparse attention: each 64-row query block attends to its topk
    highest-scoring 64-key blocks (mean-pooled q and k block scores), causally."""
    if cu_seqlens is not None:
        cu = _cu_list(q, k, v, cu_seqlens)
        max_len = max(b - a for a, b in zip(cu, cu[1:]))
        cu_dev = torch.tensor(cu, dtype=torch.int32, device=q.device)
        idx = msa.estimate_bs_varlen(q, k, cu_dev, max_len, topk, stream=stream)
        return msa.sparse_prefill_varlen(q, k, v, idx, cu_dev, max_len, stream=stream)
    q4, k4, v4, squeeze = _batched(q, k, v)
    f = _fold(q4, k4, v4)
    if f is not None:
        idx = msa.estimate_bs(f[0], f[1], topk, stream=stream)
        out = _unfold(msa.sparse_prefill(*f, idx, stream=stream), q4)
        return out[0] if squeeze else out
    out = torch.empty_like(q4)
    hq, hkv, n = q4.shape[1], k4.shape[1], q4.shape[2]
    idx = msa.alloc_index(hq, n, min(topk, (n + msa.BLOCK - 1) // msa.BLOCK), 0, q4.device)
    ws = torch.empty(max(msa.estimate_bs_workspace_bytes(hq, hkv, n, q4.dtype), 1), dtype=torch.uint8,
                     device=q4.device)
    aws_bytes = msa.sparse_prefill_workspace_bytes(hq, hkv, n, q4.dtype)
    aws = torch.empty(aws_bytes, dtype=torch.uint8, device=q4.device) if aws_bytes else None
    for bi in range(q4.shape[0]):
        msa.estimate_bs(q4[bi], k4[bi], topk, out=idx, workspace=ws, stream=stream)
        msa.sparse_prefill(q4[bi], k4[bi], v4[bi], idx, out=out[bi], workspace=aws, stream=stream)
    return out[0] if squeeze else out


@msa.on_stream
def streaming_forward(q, k, v, init_num: int, local_window_num: int, *, cu_seqlens=None, stream=None):
    """A-shape (streaming) attention: every row attends to the first init_num
    keys and to the local_window_num keys ending at itself (diagonal offsets
    0 .. local_window_num - 1), causally, over their 64-wide block cover."""
    if cu_seqlens is not None:
        if init_num < 1 or local_window_num < 1:
            raise msa.MsaError("init_num and local_window_num must be at least 1")

        def sets(cu_dev, max_len):
            # the same sets for every head; entries past a sequence's end select nothing
            heads = (cu_dev.shape[0] - 1) * q.shape[0]
            i32 = dict(dtype=torch.int32, device=q.device)
            return (torch.arange(min(init_num, max_len), **i32).expand(heads, -1).contiguous(),
                    torch.arange(min(local_window_num, max_len), **i32).expand(heads, -1).contiguous())
        return _packed_varlen(q, k, v, cu_seqlens, sets, stream)
    q4, k4, v4, squeeze = _batched(q, k, v)
    hq, hkv, n = q4.shape[1], k4.shape[1], q4.shape[2]
    if not (1 <= init_num <= n and 1 <= local_window_num <= n):
        raise msa.MsaError("init_num and local_window_num must be in [1, seq_len]")
    f = _fold(q4, k4, v4)
    if f is not None:
        out = torch.empty((f[0].shape[0], _rows(f[0]), f[0].shape[2]), dtype=q4.dtype,
                          device=q4.device)[:, :n]
        _streaming_into(*f, init_num, local_window_num, out, stream)
        out = _unfold(out, q4)
        return out[0] if squeeze else out
    i32 = dict(dtype=torch.int32, device=q4.device)
    vi = torch.arange(init_num, **i32).expand(hq, -1).contiguous()
    si = torch.arange(local_window_num, **i32).expand(hq, -1).contiguous()
    idx = msa.build_index(vi, si, n, stream=stream)       # the same for every batch element
    out = torch.empty_like(q4)
    aws_bytes = msa.sparse_prefill_workspace_bytes(hq, hkv, n, q4.dtype)
    aws = torch.empty(aws_bytes, dtype=torch.uint8, device=q4.device) if aws_bytes else None
    for bi in range(q4.shape[0]):
        msa.sparse_prefill(q4[bi], k4[bi], v4[bi], idx, out=out[bi], workspace=aws, stream=stream)
    return out[0] if squeeze else out


def _streaming_into(q, k, v, init_num, local_window_num, out, stream):
    """streaming_forward for one [heads, seq, dim] sequence, written into out."""
    hq, n = q.shape[0], q.shape[1]
    i32 = dict(dtype=torch.int32, device=q.device)
    vi = torch.arange(init_num, **i32).expand(hq, -1).contiguous()
    si = torch.arange(local_window_num, **i32).expand(hq, -1).contiguous()
    idx = msa.build_index(vi, si, n, stream=stream)
    msa.sparse_prefill(q, k, v, idx, out=out, stream=stream)
