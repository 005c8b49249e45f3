"""Decode-side dynamic sparsity, in float64 (test infrastructure only; see the
package header).

One new query row per q head attends to the cached keys of its kv head; the
dynamic sparse step keeps only the top-k keys by attention score, chosen anew
for every query (talk slides "System-Algorithm Co-design", slide "Dynamic
sparsity in attention", decoding panel: the top-1000 keys chosen dynamically
keep more of the attention mass than a static choice).  The quality measure
the slide reports is the kept share of the dense attention mass ("recovery").
"""

from __future__ import annotations

import numpy as np

from .estimate import as_f64, top_k_indices


def decode_scores(q, k, scale: float | None = None) -> np.ndarray:
    """s[h, j] = scale * <q_h, k_{g(h), j}> for q [Hq, D] and k [Hkv, N, D]
    (q head h reads kv head h // (Hq / Hkv))."""
    q = as_f64(q)
    k = as_f64(k)
    Hq, D = q.shape
    G = Hq // k.shape[0]
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    return np.stack([scale * (k[h // G] @ q[h]) for h in range(Hq)])


def _logsumexp(x: np.ndarray) -> float:
    m = x.max()
    return float(m + np.log(np.exp(x - m).sum()))


def decode_sparse_attention(q, k, v, topk: int, idx=None, scale: float | None = None):
    """Attention of each query row over a subset of the cache: the exact
    top-k keys by score (ties to the lower index, ascending), or the given
    idx [Hq, k].  Returns out [Hq, D], lse [Hq] (natural log over the chosen
    keys), recovery [Hq] = sum over chosen e^s / sum over all e^s, and the
    chosen indices."""
    s = decode_scores(q, k, scale)
    v = as_f64(v)
    Hq = s.shape[0]
    G = Hq // v.shape[0]
    if idx is None:
        idx = np.stack([top_k_indices(s[h], topk) for h in range(Hq)])
    idx = np.asarray(idx, dtype=np.int64)
    out = np.zeros((Hq, v.shape[2]))
    lse = np.zeros(Hq)
    rec = np.zeros(Hq)
    for h in range(Hq):
        sel = s[h, idx[h]]
        m = sel.max()
        p = np.exp(sel - m)
        out[h] = (p[:, None] * v[h // G][idx[h]]).sum(axis=0) / p.sum()
        lse[h] = m + np.log(p.sum())
        rec[h] = np.exp(lse[h] - _logsumexp(s[h]))
    return out, lse, rec, idx
