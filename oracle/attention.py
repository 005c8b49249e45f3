"""Oracle: softmax attention under an explicit boolean mask, float64.

Test infrastructure only (see the package docstring).

The method computes causal attention only over the selected entries ("MInference
1.0 README", section "TL;DR"; talk slides "System-Algorithm Co-design", slide
"MInference": dynamic sparse attention calculation).  Given the mask, that is
exact softmax attention restricted to it:

    O[i] = sum_{j : M[i,j]} softmax_j(scale * <q_i, k_j>) v_j,
    lse[i] = log sum_{j : M[i,j]} exp(scale * <q_i, k_j>),

with O[i] = 0 and lse[i] = -inf for a row whose mask is empty.  Dense causal
attention is the case M[i, j] = (j <= i).
"""

from __future__ import annotations

import numpy as np

from .estimate import as_f64
from .index import IndexArrays, block_key_sets


def _masked_softmax_rows(qrows: np.ndarray, keys: np.ndarray, vals: np.ndarray,
                         mask: np.ndarray, scale: float):
    z = scale * (qrows @ keys.T)
    z = np.where(mask, z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    safe = np.where(l > 0, l, 1.0)
    o = (e / safe) @ vals
    o[empty] = 0.0
    lse = np.where(empty, -np.inf, m[:, 0] + np.log(safe[:, 0]))
    return o, lse, e / safe


def attention_with_mask(q, k, v, mask, scale: float | None = None, heads=None,
                        return_probs: bool = False):
    """O [H, N, D], lse [H, N] for an explicit mask [H, N, N] (or [N, N] shared)."""
    Hq, N, D = q.shape
    G = Hq // k.shape[0]
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    heads = list(range(Hq)) if heads is None else list(heads)
    O = np.zeros((len(heads), N, D))
    LSE = np.zeros((len(heads), N))
    probs = []
    for n, h in enumerate(heads):
        g = h // G
        mk = mask if mask.ndim == 2 else mask[n]
        o, lse, p = _masked_softmax_rows(as_f64(q[h]), as_f64(k[g]), as_f64(v[g]), mk, scale)
        O[n], LSE[n] = o, lse
        if return_probs:
            probs.append(p)
    if return_probs:
        return O, LSE, probs
    return O, LSE


def dense_attention(q, k, v, scale: float | None = None, heads=None):
    N = q.shape[1]
    return attention_with_mask(q, k, v, np.tril(np.ones((N, N), dtype=bool)), scale, heads)


def _grouped(items, G):
    by_g = {}
    for (h, b) in items:
        by_g.setdefault(h // G, []).append((h, b))
    return by_g


def masked_attention_blocks(q, k, v, idx: IndexArrays, items, head_rows=None, block: int = 64,
                            scale: float | None = None):
    """Masked attention for sampled (head, query block) pairs.

    idx holds the index of the heads listed in head_rows (head id -> row of idx;
    default: row h).  Returns {(h, b): (O [rows, D], lse [rows])}.  The mask is
    the row-by-row evaluation of the same M as index_mask."""
    Hq, N, D = q.shape
    G = Hq // k.shape[0]
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    out = {}
    for g, its in _grouped(items, G).items():
        kg = as_f64(k[g])
        vg = as_f64(v[g])
        for (h, b) in its:
            r0, r1 = b * block, min(b * block + block - 1, N - 1)
            row = h if head_rows is None else head_rows[h]
            keys = block_key_sets(idx, row, b, N, block)
            causal = np.arange(r1 + 1)[None, :] <= np.arange(r0, r1 + 1)[:, None]
            mask = keys[None, :] & causal
            o, lse, _ = _masked_softmax_rows(as_f64(q[h, r0: r1 + 1]), kg[: r1 + 1], vg[: r1 + 1],
                                             mask, scale)
            out[(h, b)] = (o, lse)
    return out


def exact_attention_blocks(q, k, v, v_idx, s_idx, items, block: int = 64, scale: float | None = None):
    """Attention under the exact union mask M_x for sampled (head, query
    block) pairs: {(h, b): (O [rows, D], lse [rows])}, row by row as
    exact_union_mask defines it."""
    from .index import exact_union_rows
    Hq, N, D = q.shape
    G = Hq // k.shape[0]
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    out = {}
    for g, its in _grouped(items, G).items():
        kg = as_f64(k[g])
        vg = as_f64(v[g])
        for (h, b) in its:
            r0, r1 = b * block, min(b * block + block - 1, N - 1)
            mask = exact_union_rows(v_idx[h], s_idx[h], r0, r1, N)
            o, lse, _ = _masked_softmax_rows(as_f64(q[h, r0: r1 + 1]), kg[: r1 + 1], vg[: r1 + 1],
                                             mask, scale)
            out[(h, b)] = (o, lse)
    return out


def dense_attention_blocks(q, k, v, items, block: int = 64, scale: float | None = None):
    """Dense causal attention for sampled (head, query block) pairs."""
    Hq, N, D = q.shape
    G = Hq // k.shape[0]
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    out = {}
    for g, its in _grouped(items, G).items():
        kg = as_f64(k[g])
        vg = as_f64(v[g])
        for (h, b) in its:
            r0, r1 = b * block, min(b * block + block - 1, N - 1)
            mask = np.arange(r1 + 1)[None, :] <= np.arange(r0, r1 + 1)[:, None]
            o, lse, _ = _masked_softmax_rows(as_f64(q[h, r0: r1 + 1]), kg[: r1 + 1], vg[: r1 + 1],
                                             mask, scale)
            out[(h, b)] = (o, lse)
    return out


def attention_recall(q, k, mask, scale: float | None = None, heads=None):
    """Share of each row's dense causal attention that the mask keeps, [H, N].

    The pages judge a sparse selection by how much of the attention scores it
    recovers (talk slides "System-Algorithm Co-design", slide "Dynamic
    sparsity in attention", figure panels (a)-(c): coverage and recovery of
    top-k selections).  Written as that definition:
        p[i, :] = softmax_j(scale * <q_i, k_j>) over j <= i
        recall[i] = sum_{j <= i, M[i, j]} p[i, j]
    mask: [H, N, N] (or [N, N] shared), as in attention_with_mask."""
    Hq, N, D = q.shape
    G = Hq // k.shape[0]
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    heads = list(range(Hq)) if heads is None else list(heads)
    causal = np.tril(np.ones((N, N), dtype=bool))
    out = np.zeros((len(heads), N))
    for n, h in enumerate(heads):
        g = h // G
        mk = mask if mask.ndim == 2 else mask[n]
        _, _, p = _masked_softmax_rows(as_f64(q[h]), as_f64(k[g]), np.zeros((N, 1)), causal, scale)
        out[n] = np.where(mk & causal, p, 0.0).sum(axis=1)
    return out
