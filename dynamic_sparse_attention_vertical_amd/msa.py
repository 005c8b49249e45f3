"""ctypes binding for libmsa.so.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers and the current HIP stream are handed to the C
entry points, and a non-zero status raises MsaError with the library's message.
Every step of the computation runs in the HIP kernels; there is no fallback.
"""

from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")
_lib = None

MSA_BF16, MSA_F32 = 0, 1
HEAD_DIM = 128
BLOCK = 64
DEFAULT_PHASE_KEYS = 12288    # MSA_DEFAULT_PHASE_KEYS: keys per sparse-prefill phase when phase_keys is 0
LAST_Q = 64


class MsaError(RuntimeError):
    pass


class Problem(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("seq_len", ctypes.c_int64), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("sm_scale", ctypes.c_float), ("seq_stride", ctypes.c_int64)]


_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "msa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "msa_last_error": (ctypes.c_char_p, []),
    "msa_index_caps": (ctypes.c_int, [_VP, _I32, _I32, _I32, _VP, _VP]),
    "msa_estimate_vs_workspace": (ctypes.c_size_t, [_VP, _I32, _I32, _I32]),
    "msa_estimate_vs": (ctypes.c_int, [_VP, _VP, _VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP,
                                       ctypes.c_size_t, _VP]),
    "msa_estimate_vs_noalloc": (ctypes.c_int, [_VP, _VP, _VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP]),
    "msa_build_index": (ctypes.c_int, [_VP, _VP, _I32, _VP, _I32, _I32, _VP, _VP, _I32, _VP, _VP,
                                       _I32, _VP]),
    "msa_sparse_prefill": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32,
                                          _VP, ctypes.c_size_t, _VP, _VP, _VP]),
    "msa_sparse_prefill_workspace": (ctypes.c_size_t, [_VP, _I32]),
    "msa_sparse_prefill_fused_workspace": (ctypes.c_size_t, [_VP, _I32, _I32, _I32]),
    "msa_decode_sparse_workspace": (ctypes.c_size_t, [_VP]),
    "msa_decode_sparse": (ctypes.c_int, [_VP, _VP, _VP, _VP, _I32, _VP, _I32, _VP, ctypes.c_size_t, _VP, _VP, _VP,
                                         _VP]),
    "msa_decode_sparse_varlen": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I32, _VP, _I32, _VP, ctypes.c_size_t, _VP,
                                                _VP, _VP, _VP]),
    "msa_sparse_prefill_walk_marks": (ctypes.c_int, [_VP, _I32, _VP, _VP]),
    "msa_sparse_prefill_fused": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I32, _VP, _I32, _I32, _I32, _VP,
                                                ctypes.c_size_t, _VP, _VP, _VP]),
    "msa_dense_prefill": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "msa_estimate_bs_workspace": (ctypes.c_size_t, [_VP, _I32]),
    "msa_estimate_vs_varlen_workspace": (ctypes.c_size_t, [_VP, _VP, _I32]),
    "msa_estimate_vs_varlen": (ctypes.c_int, [_VP, _VP, _VP, _VP, _I32, _I32, _I32, _VP, _VP, _VP, ctypes.c_size_t,
                                              _VP]),
    "msa_build_index_varlen": (ctypes.c_int, [_VP, _VP, _VP, _I32, _VP, _I32, _I32, _VP, _VP, _I32, _VP, _VP, _I32,
                                              _VP]),
    "msa_sparse_prefill_varlen_workspace": (ctypes.c_size_t, [_VP, _VP, _I32]),
    "msa_sparse_prefill_varlen": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32, _VP,
                                                 ctypes.c_size_t, _VP, _VP, _VP]),
    "msa_dense_prefill_varlen": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "msa_estimate_bs_varlen_workspace": (ctypes.c_size_t, [_VP, _VP, _I32]),
    "msa_estimate_bs_varlen": (ctypes.c_int, [_VP, _VP, _VP, _VP, _I32, _I32, _VP, _VP, _I32, _VP, _VP,
                                              ctypes.c_size_t, _VP]),
    "msa_estimate_bs": (ctypes.c_int, [_VP, _VP, _VP, _I32, _I32, _VP, _VP, _I32, _VP, _VP,
                                       ctypes.c_size_t, _VP]),
}


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libmsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise MsaError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m dynamic_sparse_attention_vertical_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        lib = load()
        raise MsaError(f"{what}: {lib.msa_status_str(status).decode()}: "
                       f"{lib.msa_last_error().decode()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MSA_BF16
    if t.dtype == torch.float32:
        return MSA_F32
    raise MsaError(f"unsupported dtype {t.dtype}")


def problem(n_q_heads: int, n_kv_heads: int, seq_len: int, dtype: int, sm_scale: float = 0.0,
            seq_stride: int = 0) -> Problem:
    return Problem(n_q_heads, n_kv_heads, seq_len, HEAD_DIM, dtype, sm_scale, seq_stride)


def _head_stride(t: torch.Tensor, name: str) -> int:
    """Rows from one head's start to the next for a [heads, seq, 128] tensor
    whose rows are contiguous (a whole tensor, or a slice of a packed one)."""
    if t.dim() != 3 or t.shape[2] != HEAD_DIM or t.stride(2) != 1 or t.stride(1) != HEAD_DIM or \
            t.stride(0) % HEAD_DIM != 0:
        raise MsaError(f"{name} must be [heads, seq_len, {HEAD_DIM}] with contiguous rows")
    return t.stride(0) // HEAD_DIM if t.shape[0] > 1 else t.shape[1]


def _problem_of(q: torch.Tensor, k: torch.Tensor, sm_scale: float, v: torch.Tensor | None = None) -> Problem:
    if q.dim() != 3 or k.dim() != 3 or (v is not None and v.dim() != 3):
        raise MsaError("q, k and v must be [heads, seq_len, head_dim]")
    n = q.shape[1]
    for t, name in ((k, "k"), (v, "v")):
        if t is None:
            continue
        if t.dtype != q.dtype or t.device != q.device:
            raise MsaError(f"{name} must have q's dtype and device")
        if t.shape[1] != n:
            raise MsaError(f"{name} has {t.shape[1]} rows per head, q has {n}")
    if v is not None and v.shape[0] != k.shape[0]:
        raise MsaError("k and v must have the same number of heads")
    sq = _head_stride(q, "q")
    rows = {sq} | ({_head_stride(k, "k")} if k.shape[0] > 1 else set()) | \
        ({_head_stride(v, "v")} if v is not None and v.shape[0] > 1 else set())
    if len(rows) != 1:
        raise MsaError("q, k and v must have the same head stride")
    return problem(q.shape[0], k.shape[0], n, _dtype_code(q), sm_scale, 0 if sq == n else sq)


def _stride_rows(p: Problem) -> int:
    return p.seq_stride or p.seq_len


def _out_like(q: torch.Tensor, p: Problem) -> torch.Tensor:
    """An output laid out like q (head stride included)."""
    if p.seq_stride == 0:
        return torch.empty_like(q)
    return torch.empty((q.shape[0], p.seq_stride, HEAD_DIM), dtype=q.dtype, device=q.device)[:, : p.seq_len]


def _lse_like(q: torch.Tensor, p: Problem) -> torch.Tensor:
    return torch.empty((q.shape[0], _stride_rows(p)), dtype=torch.float32, device=q.device)[:, : p.seq_len]


def _rows_dev(t: torch.Tensor, name: str, p: Problem, like: torch.Tensor, lse: bool = False) -> int:
    """Pointer of an output that must follow the problem's head stride."""
    if not t.is_cuda or t.device != like.device:
        raise MsaError(f"{name} must be a GPU tensor on q's device")
    shape = (p.n_q_heads, p.seq_len) if lse else (p.n_q_heads, p.seq_len, HEAD_DIM)
    if tuple(t.shape) != shape or t.dtype != (torch.float32 if lse else like.dtype):
        raise MsaError(f"{name} must be {'float32' if lse else like.dtype} {list(shape)}")
    r = _stride_rows(p)
    ok = (t.dim() == 2 and t.stride(1) == 1 and (t.shape[0] == 1 or t.stride(0) == r)) if lse else \
        (t.dim() == 3 and t.stride(2) == 1 and t.stride(1) == HEAD_DIM and
         (t.shape[0] == 1 or t.stride(0) == r * HEAD_DIM))
    if not ok:
        raise MsaError(f"{name} must have the inputs' head stride ({r} rows)")
    return t.data_ptr()


def _in_dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise MsaError(f"{name} must be a GPU tensor")
    return t.data_ptr()


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise MsaError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise MsaError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def on_stream(fn):
    """Run a call with its `stream` (if given) as torch's current stream, so
    that every buffer it allocates belongs to that stream (the caching
    allocator reuses its memory only after the stream's work on it) and every
    torch op it issues is ordered with the library's launches."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, stream=None, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return wrapper


@dataclass
class IndexTensors:
    """Per-query-block work lists on the GPU (int32)."""
    block_count: torch.Tensor      # [H, nQB]
    block_offset: torch.Tensor     # [H, nQB, cap_blocks]
    column_count: torch.Tensor     # [H, nQB]
    column_index: torch.Tensor     # [H, nQB, cap_cols]

    @property
    def cap_blocks(self) -> int:
        return self.block_offset.shape[2]

    @property
    def cap_cols(self) -> int:
        return self.column_index.shape[2]


def index_caps(seq_len: int, vertical_topk: int, slash_topk: int, n_q_heads: int = 1):
    cb, cc = ctypes.c_int32(), ctypes.c_int32()
    p = problem(n_q_heads, 1, seq_len, MSA_BF16)
    _check(load().msa_index_caps(ctypes.byref(p), vertical_topk, slash_topk, BLOCK,
                                 ctypes.byref(cb), ctypes.byref(cc)), "msa_index_caps")
    return cb.value, cc.value


def alloc_index(n_q_heads: int, seq_len: int, cap_blocks: int, cap_cols: int, device="cuda") -> IndexTensors:
    nqb = (seq_len + BLOCK - 1) // BLOCK
    i32 = dict(dtype=torch.int32, device=device)
    return IndexTensors(torch.empty((n_q_heads, nqb), **i32),
                        torch.empty((n_q_heads, nqb, max(cap_blocks, 1)), **i32)[:, :, :cap_blocks],
                        torch.empty((n_q_heads, nqb), **i32),
                        torch.empty((n_q_heads, nqb, max(cap_cols, 1)), **i32)[:, :, :cap_cols])


def estimate_vs_workspace_bytes(n_q_heads: int, n_kv_heads: int, seq_len: int, dtype=torch.bfloat16) -> int:
    p = problem(n_q_heads, n_kv_heads, seq_len, MSA_BF16 if dtype == torch.bfloat16 else MSA_F32)
    return int(load().msa_estimate_vs_workspace(ctypes.byref(p), LAST_Q, 1, 1))


def estimate_bs_workspace_bytes(n_q_heads: int, n_kv_heads: int, seq_len: int, dtype=torch.bfloat16) -> int:
    p = problem(n_q_heads, n_kv_heads, seq_len, MSA_BF16 if dtype == torch.bfloat16 else MSA_F32)
    return int(load().msa_estimate_bs_workspace(ctypes.byref(p), BLOCK))


@on_stream
def estimate_vs(q: torch.Tensor, k: torch.Tensor, vertical_topk: int, slash_topk: int, *,
                last_q: int = LAST_Q, v_score: torch.Tensor | None = None,
                s_score: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                v_idx: torch.Tensor | None = None, s_idx: torch.Tensor | None = None,
                sm_scale: float = 0.0, stream=None):
    """Vertical and slash index sets, each [Hq, k] int32 ascending."""
    lib = load()
    p = _problem_of(q, k, sm_scale)
    hq, n = q.shape[0], q.shape[1]
    ws_bytes = int(lib.msa_estimate_vs_workspace(ctypes.byref(p), last_q, vertical_topk, slash_topk))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    if v_idx is None:
        v_idx = torch.empty((hq, vertical_topk), dtype=torch.int32, device=q.device)
    if s_idx is None:
        s_idx = torch.empty((hq, slash_topk), dtype=torch.int32, device=q.device)
    for t, name in ((v_score, "v_score"), (s_score, "s_score")):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (hq, n)):
            raise MsaError(f"{name} must be float32 [{hq}, {n}]")
    for t, name, kk in ((v_idx, "v_idx", vertical_topk), (s_idx, "s_idx", slash_topk)):
        if t.dtype != torch.int32 or tuple(t.shape) != (hq, kk):
            raise MsaError(f"{name} must be int32 [{hq}, {kk}]")
    _check(lib.msa_estimate_vs(ctypes.byref(p), _in_dev(q, "q"), _in_dev(k, "k"), last_q, vertical_topk,
                               slash_topk, _dev(v_idx, "v_idx"), _dev(s_idx, "s_idx"),
                               _dev(v_score, "v_score") if v_score is not None else None,
                               _dev(s_score, "s_score") if s_score is not None else None,
                               _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                               _stream(stream)), "msa_estimate_vs")
    return v_idx, s_idx


@on_stream
def estimate_vs_noalloc(q: torch.Tensor, k: torch.Tensor, vertical_topk: int, slash_topk: int, *,
                        last_q: int = LAST_Q, v_score: torch.Tensor | None = None,
                        s_score: torch.Tensor | None = None, v_idx: torch.Tensor | None = None,
                        s_idx: torch.Tensor | None = None, sm_scale: float = 0.0, stream=None):
    """estimate_vs through msa_estimate_vs_noalloc: the library's own
    per-GPU scratch instead of a workspace (the C call allocates nothing;
    pass v_idx and s_idx to keep this wrapper from allocating them)."""
    lib = load()
    p = _problem_of(q, k, sm_scale)
    hq, n = q.shape[0], q.shape[1]
    if v_idx is None:
        v_idx = torch.empty((hq, vertical_topk), dtype=torch.int32, device=q.device)
    if s_idx is None:
        s_idx = torch.empty((hq, slash_topk), dtype=torch.int32, device=q.device)
    for t, name in ((v_score, "v_score"), (s_score, "s_score")):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (hq, n)):
            raise MsaError(f"{name} must be float32 [{hq}, {n}]")
    for t, name, kk in ((v_idx, "v_idx", vertical_topk), (s_idx, "s_idx", slash_topk)):
        if t.dtype != torch.int32 or tuple(t.shape) != (hq, kk):
            raise MsaError(f"{name} must be int32 [{hq}, {kk}]")
    with torch.cuda.device(q.device):
        _check(lib.msa_estimate_vs_noalloc(ctypes.byref(p), _in_dev(q, "q"), _in_dev(k, "k"), last_q,
                                           vertical_topk, slash_topk, _dev(v_idx, "v_idx"), _dev(s_idx, "s_idx"),
                                           _dev(v_score, "v_score") if v_score is not None else None,
                                           _dev(s_score, "s_score") if s_score is not None else None,
                                           _stream(stream)), "msa_estimate_vs_noalloc")
    return v_idx, s_idx


@on_stream
def build_index(v_idx: torch.Tensor, s_idx: torch.Tensor, seq_len: int, *,
                out: IndexTensors | None = None, stream=None) -> IndexTensors:
    lib = load()
    hq, kv = v_idx.shape
    ks = s_idx.shape[1]
    p = problem(hq, 1, seq_len, MSA_BF16)
    if out is None:
        cb, cc = index_caps(seq_len, kv, ks, hq)
        out = alloc_index(hq, seq_len, cb, cc, v_idx.device)
    for t in (v_idx, s_idx):
        if t.dtype != torch.int32 or t.dim() != 2 or t.shape[0] != hq:
            raise MsaError(f"index sets must be int32 [{hq}, k]")
    bc, bo, cb, cc, ci, ccap = _index_ptrs(out, hq, seq_len)
    _check(lib.msa_build_index(ctypes.byref(p), _dev(v_idx, "v_idx") if kv else None, kv,
                               _dev(s_idx, "s_idx") if ks else None, ks, BLOCK, bc, bo, cb, cc, ci, ccap,
                               _stream(stream)),
           "msa_build_index")
    return out


def _index_ptrs(idx: IndexTensors, hq: int, n: int):
    """Pointers and capacities of work lists shaped for hq heads of n tokens."""
    nqb = (n + BLOCK - 1) // BLOCK
    for name in ("block_count", "block_offset", "column_count", "column_index"):
        if not getattr(idx, name).is_cuda:
            raise MsaError(f"{name} must be a GPU tensor")
    for name in ("block_count", "column_count"):
        t = getattr(idx, name)
        if t.dtype != torch.int32 or tuple(t.shape) != (hq, nqb) or not t.is_contiguous():
            raise MsaError(f"{name} must be contiguous int32 [{hq}, {nqb}]")
    for name in ("block_offset", "column_index"):
        t = getattr(idx, name)
        if t.dtype != torch.int32 or t.shape[0] != hq or t.shape[1] != nqb or \
                t.stride(2) != 1 or t.stride(1) != t.shape[2] or t.stride(0) != nqb * t.shape[2]:
            if t.shape[2] > 0:
                raise MsaError(f"{name} must be a dense int32 [{hq}, {nqb}, cap] array")
    return (idx.block_count.data_ptr(), idx.block_offset.data_ptr(), idx.cap_blocks,
            idx.column_count.data_ptr(), idx.column_index.data_ptr(), idx.cap_cols)


def sparse_prefill_workspace_bytes(n_q_heads: int, n_kv_heads: int, seq_len: int, dtype=torch.bfloat16,
                                   phase_keys: int = 0) -> int:
    """Workspace bytes of sparse_prefill (0: one key phase, none needed)."""
    p = problem(n_q_heads, n_kv_heads, seq_len, MSA_BF16 if dtype == torch.bfloat16 else MSA_F32)
    return int(load().msa_sparse_prefill_workspace(ctypes.byref(p), phase_keys))


FUSED_EXACT = 1


def sparse_prefill_fused_workspace_bytes(n_q_heads: int, n_kv_heads: int, seq_len: int, vertical_topk: int,
                                         dtype=torch.bfloat16, phase_keys: int = 0, exact: bool = False) -> int:
    """Workspace bytes of sparse_prefill_fused (0: none needed)."""
    p = problem(n_q_heads, n_kv_heads, seq_len, MSA_BF16 if dtype == torch.bfloat16 else MSA_F32)
    return int(load().msa_sparse_prefill_fused_workspace(ctypes.byref(p), vertical_topk, phase_keys,
                                                         FUSED_EXACT if exact else 0))


def sparse_walk_marks(workspace: torch.Tensor, n_q_heads: int, n_kv_heads: int, seq_len: int,
                      dtype=torch.bfloat16, phase_keys: int = 0) -> torch.Tensor | None:
    """The grouped walk's marks from a sparse_prefill workspace, expanded to
    one int32 per (q head, query block): 1 where the walk ran the block (all
    aligned tiles 0..b, masked), else 0.  None when the call used no
    workspace.  Reads the workspace as the last call on it left it."""
    p = problem(n_q_heads, n_kv_heads, seq_len, MSA_BF16 if dtype == torch.bfloat16 else MSA_F32)
    off, kh = ctypes.c_size_t(), ctypes.c_int32()
    _check(load().msa_sparse_prefill_walk_marks(ctypes.byref(p), phase_keys, ctypes.byref(off),
                                                 ctypes.byref(kh)), "msa_sparse_prefill_walk_marks")
    if kh.value == 0:
        return None
    nqb = (seq_len + BLOCK - 1) // BLOCK
    units = n_q_heads // kh.value
    m = workspace[off.value: off.value + units * nqb * 4].view(torch.int32).reshape(units, nqb)
    return m.repeat_interleave(kh.value, dim=0)


@on_stream
def sparse_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, index: IndexTensors, *,
                   out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = None,
                   sm_scale: float = 0.0, phase_keys: int = 0, workspace: torch.Tensor | None = None,
                   stream=None):
    """Causal attention restricted to the work lists.  Returns out (and lse if requested).

    phase_keys: keys per phase (0: the library default); workspace: a device
    uint8 buffer of sparse_prefill_workspace_bytes(...) bytes, allocated here
    when None and needed."""
    lib = load()
    p = _problem_of(q, k, sm_scale, v)
    hq, n = q.shape[0], q.shape[1]
    if out is None:
        out = _out_like(q, p)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = _lse_like(q, p)
    bc, bo, cb, cc, ci, ccap = _index_ptrs(index, hq, n)
    need = int(lib.msa_sparse_prefill_workspace(ctypes.byref(p), phase_keys))
    ws_ptr, ws_bytes = None, 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    _check(lib.msa_sparse_prefill(ctypes.byref(p), _in_dev(q, "q"), _in_dev(k, "k"), _in_dev(v, "v"),
                                  bc, bo, cb, cc, ci, ccap, phase_keys, ws_ptr, ws_bytes,
                                  _rows_dev(out, "out", p, q), _rows_dev(lse, "lse", p, q, True) if want_lse else None,
                                  _stream(stream)),
           "msa_sparse_prefill")
    return (out, lse) if want_lse else out


@on_stream
def sparse_prefill_fused(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, v_idx: torch.Tensor,
                         s_idx: torch.Tensor, *, out: torch.Tensor | None = None,
                         lse: torch.Tensor | bool | None = None, sm_scale: float = 0.0, phase_keys: int = 0,
                         exact: bool = False, workspace: torch.Tensor | None = None, stream=None):
    """Causal attention over the greedy block cover of s_idx plus the leftover
    columns of v_idx, the work lists walked inside the kernel (no index
    arrays).  The same tiles in the same order as sparse_prefill(q, k, v,
    build_index(v_idx, s_idx, seq_len)) without its grouped walk; exact: attend
    only to the selected columns and diagonals themselves (the same tiles,
    masked); workspace: sparse_prefill_fused_workspace_bytes(...) bytes,
    allocated here when None and needed."""
    lib = load()
    p = _problem_of(q, k, sm_scale, v)
    hq, n = q.shape[0], q.shape[1]
    for t, name in ((v_idx, "v_idx"), (s_idx, "s_idx")):
        if t.dtype != torch.int32 or t.dim() != 2 or t.shape[0] != hq:
            raise MsaError(f"{name} must be int32 [{hq}, k]")
    if out is None:
        out = _out_like(q, p)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = _lse_like(q, p)
    kv, ks = v_idx.shape[1], s_idx.shape[1]
    flags = FUSED_EXACT if exact else 0
    need = int(lib.msa_sparse_prefill_fused_workspace(ctypes.byref(p), kv, phase_keys, flags))
    ws_ptr, ws_bytes = None, 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    _check(lib.msa_sparse_prefill_fused(ctypes.byref(p), _in_dev(q, "q"), _in_dev(k, "k"), _in_dev(v, "v"),
                                        _dev(v_idx, "v_idx") if kv else None, kv,
                                        _dev(s_idx, "s_idx") if ks else None, ks, phase_keys, flags, ws_ptr, ws_bytes,
                                        _rows_dev(out, "out", p, q),
                                        _rows_dev(lse, "lse", p, q, True) if want_lse else None, _stream(stream)),
           "msa_sparse_prefill_fused")
    return (out, lse) if want_lse else out


class Varlen(ctypes.Structure):
    """msa_varlen: a packed batch of sequences of different lengths."""
    _fields_ = [("cu_seqlens", ctypes.c_void_p), ("n_seqs", ctypes.c_int32), ("max_seqlen", ctypes.c_int32)]


def varlen(cu_seqlens: torch.Tensor, max_seqlen: int) -> Varlen:
    """The descriptor of a packed batch: cu_seqlens int32 [n_seqs + 1] on the
    GPU (rows cu[s] .. cu[s+1]-1 of every head are sequence s), max_seqlen
    at least every length."""
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 2:
        raise MsaError("cu_seqlens must be int32 [n_seqs + 1]")
    return Varlen(_dev(cu_seqlens, "cu_seqlens"), cu_seqlens.shape[0] - 1, int(max_seqlen))


def estimate_vs_varlen_workspace_bytes(n_q_heads: int, n_kv_heads: int, rows: int, cu_seqlens: torch.Tensor,
                                       max_seqlen: int, dtype=torch.bfloat16) -> int:
    p = problem(n_q_heads, n_kv_heads, rows, MSA_BF16 if dtype == torch.bfloat16 else MSA_F32)
    vl = varlen(cu_seqlens, max_seqlen)
    return int(load().msa_estimate_vs_varlen_workspace(ctypes.byref(p), ctypes.byref(vl), LAST_Q))


@on_stream
def estimate_vs_varlen(q: torch.Tensor, k: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                       vertical_topk: int, slash_topk: int, *, workspace: torch.Tensor | None = None,
                       v_idx: torch.Tensor | None = None, s_idx: torch.Tensor | None = None,
                       sm_scale: float = 0.0, stream=None):
    """estimate_vs of every sequence of a packed batch (q [Hq, total, 128], k
    [Hkv, total, 128]) in one launch chain: v_idx [n_seqs * Hq, vertical_topk]
    and s_idx [n_seqs * Hq, slash_topk], head h of sequence s at row
    s * Hq + h."""
    lib = load()
    p = _problem_of(q, k, sm_scale)
    vl = varlen(cu_seqlens, max_seqlen)
    heads = vl.n_seqs * q.shape[0]
    need = int(lib.msa_estimate_vs_varlen_workspace(ctypes.byref(p), ctypes.byref(vl), LAST_Q))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if v_idx is None:
        v_idx = torch.empty((heads, vertical_topk), dtype=torch.int32, device=q.device)
    if s_idx is None:
        s_idx = torch.empty((heads, slash_topk), dtype=torch.int32, device=q.device)
    for t, name, kk in ((v_idx, "v_idx", vertical_topk), (s_idx, "s_idx", slash_topk)):
        if t.dtype != torch.int32 or tuple(t.shape) != (heads, kk):
            raise MsaError(f"{name} must be int32 [{heads}, {kk}]")
    _check(lib.msa_estimate_vs_varlen(ctypes.byref(p), ctypes.byref(vl), _in_dev(q, "q"), _in_dev(k, "k"), LAST_Q,
                                      vertical_topk, slash_topk, _dev(v_idx, "v_idx"), _dev(s_idx, "s_idx"),
                                      _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "msa_estimate_vs_varlen")
    return v_idx, s_idx


@on_stream
def build_index_varlen(v_idx: torch.Tensor, s_idx: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                       n_q_heads: int, *, rows: int | None = None, out: IndexTensors | None = None,
                       stream=None) -> IndexTensors:
    """build_index of every sequence of a packed batch: work lists of
    n_seqs * n_q_heads heads, each for max_seqlen tokens (rows: the packed
    length, which bounds cu_seqlens; default max_seqlen * n_seqs)."""
    lib = load()
    vl = varlen(cu_seqlens, max_seqlen)
    heads, kv = v_idx.shape
    ks = s_idx.shape[1]
    if heads != vl.n_seqs * n_q_heads:
        raise MsaError(f"index sets must have n_seqs * n_q_heads = {vl.n_seqs * n_q_heads} rows")
    p = problem(n_q_heads, 1, rows if rows is not None else max_seqlen * vl.n_seqs, MSA_BF16)
    if out is None:
        cb, cc = index_caps(max_seqlen, kv, ks, heads)
        out = alloc_index(heads, max_seqlen, cb, cc, v_idx.device)
    for t in (v_idx, s_idx):
        if t.dtype != torch.int32 or t.dim() != 2 or t.shape[0] != heads:
            raise MsaError(f"index sets must be int32 [{heads}, k]")
    bc, bo, cb, cc, ci, ccap = _index_ptrs(out, heads, max_seqlen)
    _check(lib.msa_build_index_varlen(ctypes.byref(p), ctypes.byref(vl), _dev(v_idx, "v_idx") if kv else None, kv,
                                      _dev(s_idx, "s_idx") if ks else None, ks, BLOCK, bc, bo, cb, cc, ci, ccap,
                                      _stream(stream)), "msa_build_index_varlen")
    return out


def sparse_prefill_varlen_workspace_bytes(n_q_heads: int, n_kv_heads: int, rows: int, cu_seqlens: torch.Tensor,
                                          max_seqlen: int, dtype=torch.bfloat16, phase_keys: int = 0) -> int:
    p = problem(n_q_heads, n_kv_heads, rows, MSA_BF16 if dtype == torch.bfloat16 else MSA_F32)
    vl = varlen(cu_seqlens, max_seqlen)
    return int(load().msa_sparse_prefill_varlen_workspace(ctypes.byref(p), ctypes.byref(vl), phase_keys))


@on_stream
def sparse_prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, index: IndexTensors,
                          cu_seqlens: torch.Tensor, max_seqlen: int, *, out: torch.Tensor | None = None,
                          lse: torch.Tensor | bool | None = None, sm_scale: float = 0.0, phase_keys: int = 0,
                          workspace: torch.Tensor | None = None, stream=None):
    """sparse_prefill of every sequence of a packed batch over the work lists
    of build_index_varlen; out (and lse) packed like q."""
    lib = load()
    p = _problem_of(q, k, sm_scale, v)
    vl = varlen(cu_seqlens, max_seqlen)
    if out is None:
        out = _out_like(q, p)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = _lse_like(q, p)
    bc, bo, cb, cc, ci, ccap = _index_ptrs(index, vl.n_seqs * q.shape[0], max_seqlen)
    need = int(lib.msa_sparse_prefill_varlen_workspace(ctypes.byref(p), ctypes.byref(vl), phase_keys))
    ws_ptr, ws_bytes = None, 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    _check(lib.msa_sparse_prefill_varlen(ctypes.byref(p), ctypes.byref(vl), _in_dev(q, "q"), _in_dev(k, "k"),
                                         _in_dev(v, "v"), bc, bo, cb, cc, ci, ccap, phase_keys, ws_ptr, ws_bytes,
                                         _rows_dev(out, "out", p, q),
                                         _rows_dev(lse, "lse", p, q, True) if want_lse else None, _stream(stream)),
           "msa_sparse_prefill_varlen")
    return (out, lse) if want_lse else out


@on_stream
def dense_prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                         max_seqlen: int, *, out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = None,
                         sm_scale: float = 0.0, stream=None):
    """Dense causal attention of every sequence of a packed batch."""
    lib = load()
    p = _problem_of(q, k, sm_scale, v)
    vl = varlen(cu_seqlens, max_seqlen)
    if out is None:
        out = _out_like(q, p)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = _lse_like(q, p)
    _check(lib.msa_dense_prefill_varlen(ctypes.byref(p), ctypes.byref(vl), _in_dev(q, "q"), _in_dev(k, "k"),
                                        _in_dev(v, "v"), _rows_dev(out, "out", p, q),
                                        _rows_dev(lse, "lse", p, q, True) if want_lse else None, _stream(stream)),
           "msa_dense_prefill_varlen")
    return (out, lse) if want_lse else out


DECODE_GIVEN_KEYS = 1


def decode_sparse_workspace_bytes(n_q_heads: int, n_kv_heads: int, cache_len: int, dtype=torch.bfloat16) -> int:
    """Workspace bytes of decode_sparse."""
    p = problem(n_q_heads, n_kv_heads, cache_len, MSA_BF16 if dtype == torch.bfloat16 else MSA_F32)
    return int(load().msa_decode_sparse_workspace(ctypes.byref(p)))


@on_stream
def decode_sparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, topk: int, *, idx: torch.Tensor | None = None,
                  given: bool = False, out: torch.Tensor | None = None, lse: torch.Tensor | bool | None = None,
                  recovery: torch.Tensor | bool | None = None, sm_scale: float = 0.0,
                  cache_lens: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """One decode step: q [Hq, 128] (one row per head) against the caches k, v
    [Hkv, N, 128] (rows may be strided), attending only to the top-k keys of
    each head by score (idx receives them, ascending) or, with given=True, to
    the keys in idx.  Returns out [Hq, 128] and idx, plus lse and recovery (the
    selected share of the dense attention mass) when asked for (True or a
    tensor).

    cache_lens: int32 on q's device, [Hkv] (keys in each kv head's cache) or
    [B] for a batch of B sequences folded into the heads (each length then
    serves the sequence's Hkv / B kv heads); N is then the capacity and the
    rows past a length are never read (msa_decode_sparse_varlen)."""
    lib = load()
    if q.dim() != 2 or q.shape[1] != HEAD_DIM or not q.is_contiguous():
        raise MsaError(f"q must be contiguous [heads, {HEAD_DIM}]")
    if k.dim() != 3 or v.dim() != 3 or k.shape != v.shape:
        raise MsaError("k and v must be caches of the same shape [kv heads, cache_len, head_dim]")
    for t, name in ((k, "k"), (v, "v")):
        if t.dtype != q.dtype or t.device != q.device:
            raise MsaError(f"{name} must have q's dtype and device")
    hq, hk, n = q.shape[0], k.shape[0], k.shape[1]
    sk, sv = _head_stride(k, "k"), _head_stride(v, "v")
    if hk > 1 and sk != sv:
        raise MsaError("k and v must have the same head stride")
    p = problem(hq, hk, n, _dtype_code(q), sm_scale, 0 if sk == n else sk)
    if idx is None:
        if given:
            raise MsaError("given=True needs idx")
        idx = torch.empty((hq, topk), dtype=torch.int32, device=q.device)
    if idx.dtype != torch.int32 or tuple(idx.shape) != (hq, topk) or not idx.is_contiguous():
        raise MsaError(f"idx must be contiguous int32 [{hq}, {topk}]")
    if out is None:
        out = torch.empty((hq, HEAD_DIM), dtype=q.dtype, device=q.device)
    if tuple(out.shape) != (hq, HEAD_DIM) or out.dtype != q.dtype or not out.is_contiguous():
        raise MsaError(f"out must be contiguous {q.dtype} [{hq}, {HEAD_DIM}]")
    extra = []
    for t, name in ((lse, "lse"), (recovery, "recovery")):
        if t is True:
            t = torch.empty(hq, dtype=torch.float32, device=q.device)
        if t is not None and t is not False:
            if t.dtype != torch.float32 or tuple(t.shape) != (hq,) or not t.is_contiguous():
                raise MsaError(f"{name} must be contiguous float32 [{hq}]")
            extra.append(t)
        else:
            extra.append(None)
    need = int(lib.msa_decode_sparse_workspace(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    tail = (topk, _dev(idx, "idx"), DECODE_GIVEN_KEYS if given else 0, _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _dev(out, "out"),
            _dev(extra[0], "lse") if extra[0] is not None else None,
            _dev(extra[1], "recovery") if extra[1] is not None else None, _stream(stream))
    if cache_lens is None:
        _check(lib.msa_decode_sparse(ctypes.byref(p), _dev(q, "q"), _in_dev(k, "k"), _in_dev(v, "v"), *tail),
               "msa_decode_sparse")
    else:
        if cache_lens.dtype != torch.int32 or cache_lens.dim() != 1 or cache_lens.device != q.device:
            raise MsaError("cache_lens must be int32 [kv heads] or [batch] on q's device")
        nb = cache_lens.shape[0]
        if nb == 0 or hk % nb != 0:
            raise MsaError(f"cache_lens has {nb} entries; it needs one per kv head ({hk}) or per sequence")
        lens = cache_lens.repeat_interleave(hk // nb) if nb != hk else cache_lens.contiguous()
        _check(lib.msa_decode_sparse_varlen(ctypes.byref(p), _dev(q, "q"), _in_dev(k, "k"), _in_dev(v, "v"),
                                            _dev(lens, "cache_lens"), *tail), "msa_decode_sparse_varlen")
    res = [out, idx]
    res += [t for t, want in zip(extra, (lse, recovery)) if want is not None and want is not False]
    return tuple(res)


@on_stream
def dense_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, out: torch.Tensor | None = None,
                  lse: torch.Tensor | bool | None = None, sm_scale: float = 0.0, stream=None):
    """Dense causal attention.  Returns out (and lse if requested)."""
    lib = load()
    p = _problem_of(q, k, sm_scale, v)
    hq, n = q.shape[0], q.shape[1]
    if out is None:
        out = _out_like(q, p)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = _lse_like(q, p)
    _check(lib.msa_dense_prefill(ctypes.byref(p), _in_dev(q, "q"), _in_dev(k, "k"), _in_dev(v, "v"),
                                 _rows_dev(out, "out", p, q), _rows_dev(lse, "lse", p, q, True) if want_lse else None,
                                 _stream(stream)), "msa_dense_prefill")
    return (out, lse) if want_lse else out


@on_stream
def estimate_bs(q: torch.Tensor, k: torch.Tensor, topk_blocks: int, *, cap_blocks: int | None = None,
                out: IndexTensors | None = None, workspace: torch.Tensor | None = None,
                sm_scale: float = 0.0, stream=None) -> IndexTensors:
    """Block-sparse work lists (no columns)."""
    lib = load()
    p = _problem_of(q, k, sm_scale)
    hq, n = q.shape[0], q.shape[1]
    nqb = (n + BLOCK - 1) // BLOCK
    if out is None:
        cap = cap_blocks if cap_blocks is not None else min(topk_blocks, nqb)
        out = alloc_index(hq, n, cap, 0, q.device)
    ws_bytes = int(lib.msa_estimate_bs_workspace(ctypes.byref(p), BLOCK))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    bc, bo, cb, cc, _, _ = _index_ptrs(out, hq, n)
    _check(lib.msa_estimate_bs(ctypes.byref(p), _in_dev(q, "q"), _in_dev(k, "k"), BLOCK, topk_blocks,
                               bc, bo, cb, cc,
                               _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                               _stream(stream)), "msa_estimate_bs")
    return out


@on_stream
def estimate_bs_varlen(q: torch.Tensor, k: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                       topk_blocks: int, *, out: IndexTensors | None = None, workspace: torch.Tensor | None = None,
                       sm_scale: float = 0.0, stream=None) -> IndexTensors:
    """estimate_bs of every sequence of a packed batch: work lists of
    n_seqs * Hq heads, each for max_seqlen tokens."""
    lib = load()
    p = _problem_of(q, k, sm_scale)
    vl = varlen(cu_seqlens, max_seqlen)
    heads = vl.n_seqs * q.shape[0]
    nqb = (max_seqlen + BLOCK - 1) // BLOCK
    if out is None:
        out = alloc_index(heads, max_seqlen, min(topk_blocks, nqb), 0, q.device)
    ws_bytes = int(lib.msa_estimate_bs_varlen_workspace(ctypes.byref(p), ctypes.byref(vl), BLOCK))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    bc, bo, cb, cc, _, _ = _index_ptrs(out, heads, max_seqlen)
    _check(lib.msa_estimate_bs_varlen(ctypes.byref(p), ctypes.byref(vl), _in_dev(q, "q"), _in_dev(k, "k"), BLOCK,
                                      topk_blocks, bc, bo, cb, cc, _dev(workspace, "workspace"),
                                      workspace.numel() * workspace.element_size(), _stream(stream)),
           "msa_estimate_bs_varlen")
    return out
