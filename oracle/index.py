"""Oracle: sparse index construction and the attention masks it defines.

Test infrastructure only (see the package docstring).

build_index runs the plain C greedy builder in csrc/index_ref.c (the covering
rule is stated there).  The mask helpers turn index arrays into the explicit
boolean mask the attention oracle applies:

  M[i, j] = (j <= i) and (j in a block of b(i) or j in the columns of b(i)),

and exact_union_mask gives the union of the selected columns and diagonals
themselves, M_x[i, j] = (j <= i) and (j in V or i - j in S), which M contains.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "index_ref.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def compile_oracle(force: bool = False) -> str:
    """Build liboracle.so from the plain C sources with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(compile_oracle())
        P = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_build_index.restype = ctypes.c_int
        lib.oracle_build_index.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                           P, ctypes.c_int, P, ctypes.c_int,
                                           P, P, ctypes.c_int, P, P, ctypes.c_int]
        _lib = lib
    return _lib


@dataclass
class IndexArrays:
    """Per-query-block work lists.  Entries past each count are -1."""
    block_count: np.ndarray      # int32 [H, nQB]
    block_offset: np.ndarray     # int32 [H, nQB, cap_b], key start of each 64-wide block
    column_count: np.ndarray     # int32 [H, nQB]
    column_index: np.ndarray     # int32 [H, nQB, cap_c], ascending key ids

    @property
    def n_heads(self) -> int:
        return self.block_count.shape[0]


def index_caps(n: int, kv: int, ks: int, block: int = 64):
    nqb = (n + block - 1) // block
    return min(ks, nqb), min(kv, n)


def build_index(v_idx, s_idx, n: int, block: int = 64, cap_b: int | None = None,
                cap_c: int | None = None) -> IndexArrays:
    """v_idx [H, kv] ascending column ids, s_idx [H, ks] ascending offsets o = i - j."""
    v_idx = np.ascontiguousarray(np.asarray(v_idx, dtype=np.int32))
    s_idx = np.ascontiguousarray(np.asarray(s_idx, dtype=np.int32))
    H, kv = v_idx.shape
    ks = s_idx.shape[1]
    cb, cc = index_caps(n, kv, ks, block)
    cap_b = cb if cap_b is None else cap_b
    cap_c = cc if cap_c is None else cap_c
    nqb = (n + block - 1) // block
    bc = np.zeros((H, nqb), np.int32)
    bo = np.full((H, nqb, cap_b), -1, np.int32)
    ccnt = np.zeros((H, nqb), np.int32)
    ci = np.full((H, nqb, max(cap_c, 0)), -1, np.int32)
    P = ctypes.POINTER(ctypes.c_int32)
    rc = _load().oracle_build_index(H, n, block, v_idx.ctypes.data_as(P), kv,
                                    s_idx.ctypes.data_as(P), ks,
                                    bc.ctypes.data_as(P), bo.ctypes.data_as(P), cap_b,
                                    ccnt.ctypes.data_as(P), ci.ctypes.data_as(P), cap_c)
    if rc != 0:
        raise ValueError("index capacity too small")
    return IndexArrays(bc, bo, ccnt, ci)


def a_shape_sets(n: int, sink: int = 128, window: int = 4096):
    """A-shape (attention sink + local window) as a fixed vertical-slash index:
    columns 0..sink-1 and diagonals 0..window-1 (talk slides "System-Algorithm
    Co-design", patterns A-shape / local windows / sink tokens; "MInference 1.0
    README", kernel-only usage streaming_forward(q, k, v, init_num,
    local_window_num))."""
    return np.arange(min(sink, n), dtype=np.int32), np.arange(min(window, n), dtype=np.int32)


def block_key_sets(idx: IndexArrays, h: int, b: int, n: int, block: int = 64) -> np.ndarray:
    """Boolean [r1+1]: keys listed for query block b of head h (before the causal cut)."""
    r1 = min(b * block + block - 1, n - 1)
    keys = np.zeros(r1 + 1, dtype=bool)
    for t in range(int(idx.block_count[h, b])):
        st = int(idx.block_offset[h, b, t])
        keys[st: min(st + block, r1 + 1)] = True
    for t in range(int(idx.column_count[h, b])):
        j = int(idx.column_index[h, b, t])
        if j <= r1:
            keys[j] = True
    return keys


def exact_union_rows(v_set, s_set, r0: int, r1: int, n: int) -> np.ndarray:
    """Rows r0..r1 of one head's M_x over keys 0..r1: (j <= i) and (j in V or
    i - j in S), V and S that head's column and diagonal sets (entries outside
    [0, n) select nothing)."""
    col = np.zeros(n, dtype=bool)
    diag = np.zeros(n, dtype=bool)
    v_set = np.asarray(v_set, dtype=np.int64)
    s_set = np.asarray(s_set, dtype=np.int64)
    col[v_set[(v_set >= 0) & (v_set < n)]] = True
    diag[s_set[(s_set >= 0) & (s_set < n)]] = True
    i = np.arange(r0, r1 + 1)[:, None]
    j = np.arange(r1 + 1)[None, :]
    return (j <= i) & (col[None, : r1 + 1] | diag[np.clip(i - j, 0, n - 1)])


def index_mask(idx: IndexArrays, n: int, block: int = 64) -> np.ndarray:
    """Explicit boolean mask M [H, N, N] of the index (causal cut applied)."""
    H = idx.n_heads
    M = np.zeros((H, n, n), dtype=bool)
    causal = np.tril(np.ones((n, n), dtype=bool))
    nqb = (n + block - 1) // block
    for h in range(H):
        for b in range(nqb):
            r0, r1 = b * block, min(b * block + block - 1, n - 1)
            keys = block_key_sets(idx, h, b, n, block)
            M[h, r0: r1 + 1, : r1 + 1] = keys[None, :]
        M[h] &= causal
    return M


def exact_union_mask(v_idx, s_idx, n: int) -> np.ndarray:
    """M_x [H, N, N]: (j <= i) and (j in V or i - j in S)."""
    v_idx = np.asarray(v_idx)
    s_idx = np.asarray(s_idx)
    H = v_idx.shape[0]
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    M = np.zeros((H, n, n), dtype=bool)
    for h in range(H):
        col = np.zeros(n, dtype=bool)
        col[v_idx[h]] = True
        diag = np.zeros(n, dtype=bool)
        diag[s_idx[h]] = True
        off = np.clip(i - j, 0, n - 1)
        M[h] = (j <= i) & (col[None, :] | diag[off])
    return M
