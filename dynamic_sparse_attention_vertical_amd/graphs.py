"""A whole call chain replayed as one HIP graph.

Small problems (a decode step, a short prefill) are bound by launches and by
the Python marshalling around them rather than by their kernels: one
vertical-slash layer issues about a dozen launches through the C ABI, each
prepared from Python.  No entry point of the library allocates, frees,
synchronises or clears memory with a memset: workspaces come from the caller
and every kernel writes what a later one reads.  So a chain called with
preallocated buffers can be captured once into a HIP graph (torch's CUDAGraph,
a hipGraph on ROCm) and then replayed with one launch from the host.

A replay reads the same input buffers and writes the same output buffers as
the captured call: copy new inputs into the buffers before a replay.  Sizes
and pointers are fixed at capture; a different shape needs another capture.
Calls that read host-side lengths from device data (cu_seqlens lists turned
into Python ints) cannot be captured; the packed entry points called with a
host max_seqlen and device cu_seqlens can.
"""

from __future__ import annotations

import warnings
from typing import Callable

import torch

from . import msa
from .layer import LayerPlan, vertical_slash_layer


class StepGraph:
    """Capture fn() (launches on torch's current stream only) and replay it.

    fn runs `warmup` times eagerly on a side stream first (library load,
    allocator pools), then once under capture; outputs is what the captured
    call returned, the tensors every replay rewrites."""

    def __init__(self, fn: Callable[[], object], *, warmup: int = 1):
        if not torch.cuda.is_available():
            raise msa.MsaError("graph capture needs a GPU")
        self.fn = fn
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with warnings.catch_warnings(record=True) as caught:
            warnings.simplefilter("always")
            with torch.cuda.graph(self.graph):
                self.outputs = fn()
        if any("empty" in str(w.message).lower() for w in caught):
            raise msa.MsaError("the capture recorded no launch: fn must launch on torch's current stream "
                               "(pass no stream, or torch.cuda.current_stream() read inside fn)")
        for w in caught:
            warnings.warn_explicit(w.message, w.category, w.filename, w.lineno)

    def replay(self):
        """Launch the captured chain on torch's current stream; returns outputs."""
        self.graph.replay()
        return self.outputs


def layer_graph(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, vertical_topk: int, slash_topk: int, *,
                plan: LayerPlan | None = None, lse: bool = True) -> tuple[StepGraph, LayerPlan]:
    """One vertical-slash layer (estimate, index, sparse prefill) over the
    buffers q, k, v as a graph.  Returns the graph, whose outputs are (out,
    lse) or out, and the plan holding the index sets and work lists."""
    if plan is None:
        plan = LayerPlan(q.shape[0], k.shape[0], q.shape[1], vertical_topk, slash_topk, str(q.device), q.dtype)
    out = torch.empty_like(q)
    lse_t = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device) if lse else None

    def step():
        vertical_slash_layer(q, k, v, vertical_topk, slash_topk, plan=plan, out=out,
                             lse=lse_t if lse else None)
        return (out, lse_t) if lse else out

    return StepGraph(step), plan


def decode_graph(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, topk: int, *,
                 cache_lens: torch.Tensor | None = None, lse: bool = False,
                 recovery: bool = False) -> StepGraph:
    """One decode step (scores, top-k, attention over the selected keys) over
    the buffers q, k, v (and cache_lens, read on the device at every replay)
    as a graph.  Outputs: (out, idx) plus lse and recovery when asked for."""
    hq = q.shape[0]
    ws = torch.empty(msa.decode_sparse_workspace_bytes(hq, k.shape[0], k.shape[1], q.dtype), dtype=torch.uint8,
                     device=q.device)
    idx = torch.empty((hq, topk), dtype=torch.int32, device=q.device)
    out = torch.empty_like(q)
    f32 = dict(dtype=torch.float32, device=q.device)
    lse_t = torch.empty(hq, **f32) if lse else None
    rec_t = torch.empty(hq, **f32) if recovery else None

    def step():
        return msa.decode_sparse(q, k, v, topk, idx=idx, out=out, lse=lse_t, recovery=rec_t,
                                 cache_lens=cache_lens, workspace=ws)

    return StepGraph(step)
