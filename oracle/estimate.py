"""Oracle: online sparse-index estimation (vertical-slash and block-sparse).

Test infrastructure only (see the package docstring).  float64 throughout.

Vertical-slash estimate.  The pages say the index is approximated online per
head at inference time ("MInference 1.0 README", section "TL;DR"; talk slides
"System-Algorithm Co-design", slide "MInference": step 2, online estimation of
sparsity indices) and that the dynamic elements are a column index and a slash
index (same slides, slide "Dynamic sparsity in attention").  They do not write
the estimator out.  Reading taken here: the last L queries of the head are
scored against every key under the causal mask, each query row is softmax
normalised, and the normalised scores are summed per key column (vertical
score) and per diagonal offset o = i - j (slash score).  The Inf-MLLM article
("Inf-MLLM: 4M-token long-sequence QA on a single 4090D", section 3.2, KV
cache eviction and update) describes the same construction for its columns: a
window of recent queries scored against all keys, averaged over the window,
then top-t; the vertical score here is that window average times L.
"""

from __future__ import annotations

import numpy as np


def as_f64(x) -> np.ndarray:
    """Exact float64 copy of a numpy array or a CPU/GPU torch tensor."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def estimate_vs(q, k, last_q: int = 64, heads=None, scale: float | None = None):
    """Vertical and slash scores of the last `last_q` queries.

    q: [Hq, N, D], k: [Hkv, N, D]; q head h reads kv head h // (Hq // Hkv).
    Returns (v, s), each float64 [len(heads), N]:
        z[r, j] = scale * <q[h, p_r], k[g, j]>,  p_r = N - L + r,  j <= p_r
        P[r, :] = softmax_j z[r, :]
        v[j]    = sum_r P[r, j]
        s[o]    = sum_r P[r, p_r - o]      (terms with p_r - o >= 0 only)
    """
    Hq, N, D = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    L = last_q
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    heads = list(range(Hq)) if heads is None else list(heads)
    pos = np.arange(N - L, N)                       # query positions p_r
    keys = np.arange(N)
    allowed = keys[None, :] <= pos[:, None]          # causal mask, [L, N]
    v_out = np.zeros((len(heads), N))
    s_out = np.zeros((len(heads), N))
    kg_cache = {}
    for n, h in enumerate(heads):
        g = h // G
        if g not in kg_cache:
            kg_cache.clear()
            kg_cache[g] = as_f64(k[g])
        kg = kg_cache[g]
        qh = as_f64(q[h, N - L:])
        z = scale * (qh @ kg.T)
        z = np.where(allowed, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p = p / p.sum(axis=1, keepdims=True)
        v_out[n] = p.sum(axis=0)
        for r in range(L):
            pr = int(pos[r])
            # o = pr - j runs 0..pr as j runs pr..0
            s_out[n, : pr + 1] += p[r, pr::-1]
    return v_out, s_out


def top_k_indices(x, k: int) -> np.ndarray:
    """Indices of the k largest entries of x, ties broken toward the lower index,
    returned in ascending index order (the order of the set is not significant)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    k = min(k, n)
    order = np.lexsort((np.arange(n), -x))          # by score descending, then index ascending
    return np.sort(order[:k]).astype(np.int64)


def block_scores(q, k, h: int, block: int = 64, scale: float | None = None) -> np.ndarray:
    """Mean-pooled block scores of q head h: u[b, c] = scale * <mean q-block b,
    mean k-block c>, for c <= b; -inf above the block diagonal.  A last block
    shorter than `block` rows (N not a multiple of it) is the mean of the rows
    it has."""
    Hq, N, D = q.shape
    G = Hq // k.shape[0]
    g = h // G
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    nb = (N + block - 1) // block
    qh, kh = as_f64(q[h]), as_f64(k[g])
    qb = np.stack([qh[b * block: (b + 1) * block].mean(axis=0) for b in range(nb)])
    kb = np.stack([kh[c * block: (c + 1) * block].mean(axis=0) for c in range(nb)])
    u = scale * (qb @ kb.T)
    u[np.triu_indices(nb, 1)] = -np.inf
    return u


def block_sparse_select(q, k, heads, topk: int = 100, block: int = 64, scale: float | None = None):
    """Block-sparse index: per (head, query block b), the top min(topk, b+1)
    key blocks c <= b by mean-pooled score (ties -> lower c), as ascending key
    starts 64*c.  Returns (block_count [H, nb], block_offset [H, nb, topk] with -1
    past the count, scores [H, nb, nb])."""
    Hq, N, D = q.shape
    nb = (N + block - 1) // block
    heads = list(heads)
    counts = np.zeros((len(heads), nb), dtype=np.int32)
    offs = np.full((len(heads), nb, topk), -1, dtype=np.int32)
    scores = np.zeros((len(heads), nb, nb))
    for n, h in enumerate(heads):
        u = block_scores(q, k, h, block, scale)
        scores[n] = u
        for b in range(nb):
            sel = top_k_indices(u[b, : b + 1], min(topk, b + 1))
            counts[n, b] = len(sel)
            offs[n, b, : len(sel)] = sel * block
    return counts, offs, scores
