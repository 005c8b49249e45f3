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


def decode_sparse_attention(q, k, v, topk: int, idx=None, scale: float | None = None, cache_len=None):
    """Attention of each query row over a subset of the cache: the exact
    top-k keys by score (ties to the lower index, ascending), or the given
    idx [Hq, k].  Returns out [Hq, D], lse [Hq] (natural log over the chosen
    keys), recovery [Hq] = sum over chosen e^s / sum over all e^s, and the
    chosen indices.

    cache_len [Hkv] (optional): kv head g holds keys 0 .. cache_len[g] - 1
    only; the rows past them are capacity, not keys.  Reading: a key that is
    not in the cache takes no part in the attention, so it scores -inf: it
    gets no weight and is outside the dense sum.  The top-k is then taken over
    those scores as before, so a head whose cache holds fewer than topk keys
    selects all of them and, by the tie rule, the lowest positions past its
    end (with no weight).  A head with no key at all: out 0, lse -inf,
    recovery 0."""
    s = decode_scores(q, k, scale)
    v = as_f64(v)
    Hq, N = s.shape
    G = Hq // v.shape[0]
    if cache_len is not None:
        for h in range(Hq):
            s[h, int(cache_len[h // G]):] = -np.inf
    if idx is None:
        idx = np.stack([top_k_indices(s[h], topk) for h in range(Hq)])
    idx = np.asarray(idx, dtype=np.int64)
    out = np.zeros((Hq, v.shape[2]))
    lse = np.full(Hq, -np.inf)
    rec = np.zeros(Hq)
    for h in range(Hq):
        sel = s[h, idx[h]]
        keep = sel > -np.inf
        if not keep.any():
            continue
        m = sel[keep].max()
        p = np.where(keep, np.exp(sel - m), 0.0)
        rows = np.where(keep[:, None], v[h // G][idx[h]], 0.0)
        out[h] = (p[:, None] * rows).sum(axis=0) / p.sum()
        lse[h] = m + np.log(p.sum())
        rec[h] = np.exp(lse[h] - _logsumexp(s[h][s[h] > -np.inf]))
    return out, lse, rec, idx
