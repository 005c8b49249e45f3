"""Pins for the CPU oracle: each check ties an oracle function to something other
than itself (a closed form, an invariant, a library routine, or a brute-force
evaluation of the definition on tiny inputs)."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.index import index_caps

RNG = np.random.default_rng(12345)


def rand_qkv(hq, hkv, n, d, seed=0, scale=1.0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((hq, n, d)) * scale, r.standard_normal((hkv, n, d)) * scale,
            r.standard_normal((hkv, n, d)))


def random_sets(h, n, kv, ks, seed=0):
    r = np.random.default_rng(seed)
    v = np.stack([np.sort(r.choice(n, size=kv, replace=False)) for _ in range(h)]).astype(np.int32)
    s = np.stack([np.sort(r.choice(n, size=ks, replace=False)) for _ in range(h)]).astype(np.int32)
    return v, s


# ---------------------------------------------------------------- estimator

def brute_estimate(q, k, L, G, scale):
    """Per-entry loops straight from the definition (pure Python, tiny sizes)."""
    Hq, N, D = q.shape
    v = [[0.0] * N for _ in range(Hq)]
    s = [[0.0] * N for _ in range(Hq)]
    for h in range(Hq):
        g = h // G
        for r in range(L):
            p = N - L + r
            z = [scale * sum(q[h, p, d] * k[g, j, d] for d in range(D)) for j in range(p + 1)]
            m = max(z)
            w = [math.exp(x - m) for x in z]
            tot = math.fsum(w)
            for j in range(p + 1):
                v[h][j] += w[j] / tot
                s[h][p - j] += w[j] / tot
    return np.array(v), np.array(s)


@pytest.mark.parametrize("hq,hkv,n,d,L", [(4, 2, 24, 3, 4), (2, 1, 40, 5, 7), (1, 1, 9, 2, 9)])
def test_estimate_matches_brute_force(hq, hkv, n, d, L):
    q, k, _ = rand_qkv(hq, hkv, n, d, seed=n)
    scale = 1.0 / math.sqrt(d)
    v, s = oracle.estimate_vs(q, k, last_q=L)
    bv, bs = brute_estimate(q, k, L, hq // hkv, scale)
    np.testing.assert_allclose(v, bv, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s, bs, rtol=0, atol=1e-12)


def test_estimate_geometric_closed_form():
    """q = (c, 0, ...), k_j = (j, 0, ...), scale 1: row p has weights
    x^j / sum_{t<=p} x^t with x = e^c, so v and s have closed forms that fix the
    direction of the diagonal index (o = i - j)."""
    N, L, D, c = 12, 3, 4, 0.3
    q = np.zeros((1, N, D))
    q[0, :, 0] = c
    k = np.zeros((1, N, D))
    k[0, :, 0] = np.arange(N)
    v, s = oracle.estimate_vs(q, k, last_q=L, scale=1.0)
    x = math.exp(c)
    ev = np.zeros(N)
    es = np.zeros(N)
    for r in range(L):
        p = N - L + r
        S = (x ** (p + 1) - 1) / (x - 1)
        for j in range(p + 1):
            ev[j] += x ** j / S
            es[p - j] += x ** j / S
    np.testing.assert_allclose(v[0], ev, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(s[0], es, rtol=1e-13, atol=1e-15)
    # every row puts its largest weight on its own diagonal, so s falls with o
    assert np.all(np.diff(s[0]) < 0)


def test_estimate_zero_query_uniform():
    """q = 0: every allowed key of row p has weight 1/(p+1)."""
    N, L, D = 50, 6, 8
    q = np.zeros((2, N, D))
    k = RNG.standard_normal((1, N, D))
    v, s = oracle.estimate_vs(q, k, last_q=L)
    for j in range(N):
        want = sum(1.0 / (p + 1) for p in range(N - L, N) if p >= j)
        assert abs(v[0, j] - want) < 1e-13 and abs(s[1, j] - want) < 1e-13


def test_estimate_mass_and_last_row_symmetry():
    """Each softmax row sums to one: sum v = sum s = L.  With L = 1 the only row
    is p = N-1, so s[o] = v[N-1-o] exactly."""
    q, k, _ = rand_qkv(4, 1, 300, 16, seed=3)
    v, s = oracle.estimate_vs(q, k, last_q=64)
    np.testing.assert_allclose(v.sum(1), 64.0, rtol=1e-12)
    np.testing.assert_allclose(s.sum(1), 64.0, rtol=1e-12)
    v1, s1 = oracle.estimate_vs(q, k, last_q=1)
    np.testing.assert_array_equal(s1, v1[:, ::-1])


def test_estimate_gqa_mapping():
    """q head h reads kv head h // G: duplicating a kv head changes nothing."""
    q, k, _ = rand_qkv(4, 2, 80, 8, seed=5)
    v, s = oracle.estimate_vs(q, k, last_q=8)
    k4 = np.repeat(k, 2, axis=0)
    v4, s4 = oracle.estimate_vs(q, k4, last_q=8)
    np.testing.assert_array_equal(v, v4)
    np.testing.assert_array_equal(s, s4)


# ---------------------------------------------------------------- top-k

@pytest.mark.parametrize("seed", range(5))
def test_top_k_definition(seed):
    """Every chosen score beats every unchosen one, ties go to the lower index,
    output ascending -- checked pairwise."""
    r = np.random.default_rng(seed)
    x = r.integers(0, 6, size=40).astype(float)      # many exact ties
    k = 13
    sel = oracle.top_k_indices(x, k)
    assert len(sel) == k and np.all(np.diff(sel) > 0)
    chosen = set(sel.tolist())
    for i in chosen:
        for j in range(len(x)):
            if j not in chosen:
                assert x[i] > x[j] or (x[i] == x[j] and i < j)


# ---------------------------------------------------------------- index builder

def union_points(s_set, r0, r1):
    U = set()
    for o in s_set:
        if o <= r1:
            U.update(range(max(0, r0 - o), r1 - o + 1))
    return U


def leftmost_cover(U, w=64):
    """Blocks placed at the leftmost point of U not yet covered (set form)."""
    pts = sorted(U)
    out, cov = [], -1
    for u in pts:
        if u > cov:
            out.append(u)
            cov = u + w - 1
    return out


def min_cover_dp(U, w=64):
    """Minimum number of width-w integer intervals covering U, by exhaustive DP
    over every start that covers the leftmost remaining point."""
    pts = sorted(U)
    f = [0] * (len(pts) + 1)            # f[i]: blocks needed for pts[i:]
    for i in range(len(pts) - 1, -1, -1):
        best = None
        for st in range(pts[i] - w + 1, pts[i] + 1):
            j = i
            while j < len(pts) and pts[j] <= st + w - 1:
                j += 1
            c = 1 + f[j]
            best = c if best is None else min(best, c)
        f[i] = best
    return f[0]


@pytest.mark.parametrize("n,kv,ks,seed", [(320, 7, 9, 0), (256, 3, 40, 1), (640, 20, 30, 2),
                                          (100, 5, 17, 3), (192, 1, 1, 4)])
def test_index_characterisation(n, kv, ks, seed):
    v_idx, s_idx = random_sets(2, n, kv, ks, seed)
    idx = oracle.build_index(v_idx, s_idx, n)
    nqb = (n + 63) // 64
    for h in range(2):
        for b in range(nqb):
            r0, r1 = 64 * b, min(64 * b + 63, n - 1)
            cnt = idx.block_count[h, b]
            blocks = idx.block_offset[h, b, :cnt].tolist()
            U = union_points(s_idx[h].tolist(), r0, r1)
            assert blocks == leftmost_cover(U)
            assert cnt == min_cover_dp(U)
            assert cnt <= min(ks, b + 1)
            assert all(blocks[i] + 64 <= blocks[i + 1] for i in range(len(blocks) - 1))
            covered = set()
            for st in blocks:
                covered.update(range(st, st + 64))
            assert U <= covered
            cols = idx.column_index[h, b, : idx.column_count[h, b]].tolist()
            want = [j for j in v_idx[h].tolist() if j <= r1 and j not in covered]
            assert cols == want


def test_index_mask_contains_exact_union():
    n = 384
    v_idx, s_idx = random_sets(3, n, 11, 23, seed=9)
    idx = oracle.build_index(v_idx, s_idx, n)
    M = oracle.index_mask(idx, n)
    Mx = oracle.exact_union_mask(v_idx, s_idx, n)
    assert np.all(M >= Mx)
    assert np.all(~np.triu(np.ones((n, n), bool), 1)[None] | ~M)   # causal


def brute_exact_union(v_idx, s_idx, n):
    """M_x straight from the lists, one entry at a time: row i sees key j iff
    j <= i and (j is a selected column or i - j a selected diagonal)."""
    H = len(v_idx)
    M = np.zeros((H, n, n), dtype=bool)
    for h in range(H):
        cols = set(int(x) for x in v_idx[h])
        diags = set(int(x) for x in s_idx[h])
        for i in range(n):
            for j in range(i + 1):
                M[h, i, j] = (j in cols) or ((i - j) in diags)
    return M


@pytest.mark.parametrize("n,kv,ks,seed", [(40, 3, 5, 1), (97, 7, 11, 2), (130, 1, 30, 3), (64, 20, 1, 4)])
def test_exact_union_mask_brute_force(n, kv, ks, seed):
    v_idx, s_idx = random_sets(3, n, kv, ks, seed=seed)
    np.testing.assert_array_equal(oracle.exact_union_mask(v_idx, s_idx, n), brute_exact_union(v_idx, s_idx, n))


def test_exact_union_mask_closed_forms():
    """Each term alone, by its closed form: the main diagonal only is the
    identity; one column c is the column below row c; diagonal o alone is the
    sub-diagonal i - j = o; every diagonal is the causal mask."""
    n = 50
    none = np.zeros((1, 0), np.int32)
    np.testing.assert_array_equal(oracle.exact_union_mask(none, np.array([[0]]), n)[0], np.eye(n, dtype=bool))
    c = 17
    want = np.zeros((n, n), bool)
    want[c:, c] = True
    np.testing.assert_array_equal(oracle.exact_union_mask(np.array([[c]]), none, n)[0], want)
    o = 9
    np.testing.assert_array_equal(oracle.exact_union_mask(none, np.array([[o]]), n)[0],
                                  np.eye(n, k=-o, dtype=bool))
    np.testing.assert_array_equal(oracle.exact_union_mask(none, np.arange(n)[None], n)[0],
                                  np.tril(np.ones((n, n), bool)))


@pytest.mark.parametrize("n,kv,ks,seed", [(200, 7, 30, 0), (130, 0, 50, 1), (257, 20, 0, 2)])
def test_exact_union_rows_and_blocks(n, kv, ks, seed):
    """Row slices of exact_union_mask (brute-force pinned above) from
    exact_union_rows, ragged last block included, plus entries outside [0, n)
    selecting nothing; exact_attention_blocks against attention_with_mask
    under the full mask on the same rows."""
    rng = np.random.default_rng(seed)
    vi = np.sort(rng.choice(n, kv, replace=False))[None].astype(np.int64)
    si = np.sort(rng.choice(n, ks, replace=False))[None].astype(np.int64)
    full = oracle.exact_union_mask(vi, si, n)[0]
    for b in range((n + 63) // 64):
        r0, r1 = 64 * b, min(64 * b + 63, n - 1)
        np.testing.assert_array_equal(oracle.exact_union_rows(vi[0], si[0], r0, r1, n), full[r0:r1 + 1, :r1 + 1])
        padded_v = np.r_[-5, vi[0], n, n + 7]
        padded_s = np.r_[-1, si[0], n + 2]
        np.testing.assert_array_equal(oracle.exact_union_rows(padded_v, padded_s, r0, r1, n),
                                      full[r0:r1 + 1, :r1 + 1])
    q = rng.standard_normal((1, n, 32))
    k = rng.standard_normal((1, n, 32))
    v = rng.standard_normal((1, n, 32))
    ref, rlse = oracle.attention_with_mask(q, k, v, full[None])
    items = [(0, b) for b in range((n + 63) // 64)]
    got = oracle.exact_attention_blocks(q, k, v, vi, si, items)
    for (h, b), (o, l) in got.items():
        r0, r1 = 64 * b, min(64 * b + 63, n - 1)
        np.testing.assert_allclose(o, ref[0, r0:r1 + 1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, rlse[0, r0:r1 + 1], rtol=0, atol=1e-12)


def test_index_all_selected_is_causal():
    n = 320
    all_ = np.arange(n, dtype=np.int32)[None]
    idx = oracle.build_index(all_, all_, n)
    for b in range((n + 63) // 64):
        assert idx.block_offset[0, b, : idx.block_count[0, b]].tolist() == list(range(0, 64 * b + 1, 64))
        assert idx.column_count[0, b] == 0
    M = oracle.index_mask(idx, n)
    np.testing.assert_array_equal(M[0], np.tril(np.ones((n, n), bool)))


def test_index_a_shape_closed_form():
    """Sink 128 + window 4096: for r0 >= 4095 + 128 the blocks start at
    r0 - 4095 + 64 t, t < 65, and all 128 sink columns are leftovers."""
    n = 64 * 80
    v, s = oracle.a_shape_sets(n, 128, 4096)
    idx = oracle.build_index(v[None], s[None], n)
    for b in range(66, 80):
        r0 = 64 * b
        assert idx.block_offset[0, b, : idx.block_count[0, b]].tolist() == \
            [r0 - 4095 + 64 * t for t in range(65)]
        assert idx.column_index[0, b, : idx.column_count[0, b]].tolist() == list(range(128))
    # early blocks: the window reaches key 0, so it tiles [0, r1] and no column is left over
    for b in range(0, 60):
        assert idx.block_offset[0, b, : idx.block_count[0, b]].tolist() == list(range(0, 64 * b + 1, 64))
        assert idx.column_count[0, b] == 0


def test_index_capacity_error():
    v_idx, s_idx = random_sets(1, 256, 4, 40, seed=1)
    with pytest.raises(ValueError):
        oracle.build_index(v_idx, s_idx, 256, cap_b=1)


# ---------------------------------------------------------------- attention

def brute_masked_attention(q, k, v, idx, n, G, scale):
    """Per-entry membership straight from the index lists, pure Python."""
    Hq, N, D = q.shape
    O = np.zeros((Hq, N, D))
    for h in range(Hq):
        g = h // G
        for i in range(N):
            b = i // 64
            blocks = idx.block_offset[h, b, : idx.block_count[h, b]].tolist()
            cols = set(idx.column_index[h, b, : idx.column_count[h, b]].tolist())
            allowed = [j for j in range(i + 1)
                       if any(st <= j <= st + 63 for st in blocks) or j in cols]
            if not allowed:
                continue
            z = [scale * sum(q[h, i, d] * k[g, j, d] for d in range(D)) for j in allowed]
            m = max(z)
            w = [math.exp(t - m) for t in z]
            tot = math.fsum(w)
            for d in range(D):
                O[h, i, d] = math.fsum(w[t] * v[g, allowed[t], d] for t in range(len(allowed))) / tot
    return O


@pytest.mark.parametrize("n,kv,ks", [(64, 3, 5), (128, 4, 9), (320, 6, 11)])
def test_masked_attention_brute_force(n, kv, ks):
    hq, hkv, d = 4, 2, 6
    q, k, v = rand_qkv(hq, hkv, n, d, seed=n)
    v_idx, s_idx = random_sets(hq, n, kv, ks, seed=n + 1)
    idx = oracle.build_index(v_idx, s_idx, n)
    M = oracle.index_mask(idx, n)
    O, lse, probs = oracle.attention_with_mask(q, k, v, M, return_probs=True)
    B = brute_masked_attention(q, k, v, idx, n, hq // hkv, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(O, B, rtol=0, atol=1e-12)
    # softmax rows sum to one on non-empty rows, and empty rows give 0 / -inf
    for h in range(hq):
        rows = M[h].any(axis=1)
        np.testing.assert_allclose(probs[h][rows].sum(1), 1.0, atol=1e-12)
        assert np.all(O[h][~rows] == 0) and np.all(np.isneginf(lse[h][~rows]))
    # the row-sampled evaluation is the same mask
    items = [(h, b) for h in range(hq) for b in range(n // 64)]
    blk = oracle.masked_attention_blocks(q, k, v, idx, items)
    for (h, b), (o, l) in blk.items():
        np.testing.assert_allclose(o, O[h, 64 * b: 64 * b + 64], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, lse[h, 64 * b: 64 * b + 64], rtol=0, atol=1e-13)


def test_all_selected_equals_dense_and_sdpa():
    n, d = 256, 32
    q, k, v = rand_qkv(4, 2, n, d, seed=11)
    all_ = np.tile(np.arange(n, dtype=np.int32), (4, 1))
    idx = oracle.build_index(all_, all_, n)
    O, lse = oracle.attention_with_mask(q, k, v, oracle.index_mask(idx, n))
    Od, lsed = oracle.dense_attention(q, k, v)
    np.testing.assert_allclose(O, Od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lsed, rtol=0, atol=1e-12)
    tq = torch.from_numpy(q)[None]
    tk = torch.from_numpy(np.repeat(k, 2, axis=0))[None]
    tv = torch.from_numpy(np.repeat(v, 2, axis=0))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].numpy()
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    blk = oracle.dense_attention_blocks(q, k, v, [(1, 2), (3, 0)])
    np.testing.assert_allclose(blk[(1, 2)][0], ref[1, 128:192], atol=1e-12)
    np.testing.assert_allclose(blk[(3, 0)][0], ref[3, 0:64], atol=1e-12)


def test_single_allowed_key_returns_value_row():
    n, d = 128, 8
    q, k, v = rand_qkv(1, 1, n, d, seed=2)
    v_idx = np.array([[5]], np.int32)
    s_idx = np.array([[n - 1]], np.int32)       # diagonal offset only reachable from the last row
    idx = oracle.build_index(v_idx, s_idx, n)
    M = oracle.index_mask(idx, n)
    O, lse = oracle.attention_with_mask(q, k, v, M)
    rows = [i for i in range(5, 64) if M[0, i].sum() == 1]
    assert rows, "expected rows whose only key is column 5"
    for i in rows:
        np.testing.assert_array_equal(O[0, i], v[0, 5])


def test_linearity_and_zero_query():
    n, d = 192, 16
    q, k, v = rand_qkv(2, 1, n, d, seed=4)
    v_idx, s_idx = random_sets(2, n, 5, 12, seed=6)
    idx = oracle.build_index(v_idx, s_idx, n)
    M = oracle.index_mask(idx, n)
    O, _ = oracle.attention_with_mask(q, k, v, M)
    O3, _ = oracle.attention_with_mask(q, k, -2.5 * v, M)
    np.testing.assert_allclose(O3, -2.5 * O, atol=1e-12)
    Oz, lz = oracle.attention_with_mask(np.zeros_like(q), k, v, M)
    for h in range(2):
        for i in range(n):
            allowed = np.nonzero(M[h, i])[0]
            if len(allowed):
                np.testing.assert_allclose(Oz[h, i], v[0, allowed].mean(0), atol=1e-12)
                assert abs(lz[h, i] - math.log(len(allowed))) < 1e-12


# ---------------------------------------------------------------- attention recall

@pytest.mark.parametrize("n,kv,ks", [(64, 3, 5), (192, 5, 9)])
def test_recall_brute_force(n, kv, ks):
    """Per-entry loop: share of the causal softmax mass on the masked keys."""
    hq, hkv, d = 2, 1, 6
    q, k, v = rand_qkv(hq, hkv, n, d, seed=n + 5)
    v_idx, s_idx = random_sets(hq, n, kv, ks, seed=n + 6)
    idx = oracle.build_index(v_idx, s_idx, n)
    M = oracle.index_mask(idx, n)
    R = oracle.attention_recall(q, k, M)
    scale = 1.0 / math.sqrt(d)
    for h in range(hq):
        for i in range(0, n, 7):
            z = [scale * sum(q[h, i, t] * k[0, j, t] for t in range(d)) for j in range(i + 1)]
            m = max(z)
            w = [math.exp(x - m) for x in z]
            want = math.fsum(w[j] for j in range(i + 1) if M[h, i, j]) / math.fsum(w)
            assert abs(R[h, i] - want) < 1e-12


def test_recall_closed_forms_and_lse_identity():
    n, d = 256, 16
    q, k, v = rand_qkv(2, 1, n, d, seed=21)
    v_idx, s_idx = random_sets(2, n, 6, 20, seed=22)
    idx = oracle.build_index(v_idx, s_idx, n)
    M = oracle.index_mask(idx, n)
    causal = np.tril(np.ones((n, n), dtype=bool))
    # the causal mask keeps everything
    np.testing.assert_allclose(oracle.attention_recall(q, k, causal), 1.0, atol=1e-12)
    # disjoint masks add up
    R = oracle.attention_recall(q, k, M)
    Rc = oracle.attention_recall(q, k, causal[None] & ~M)
    np.testing.assert_allclose(R + Rc, 1.0, atol=1e-12)
    # zero queries: uniform attention, recall = allowed keys / (i + 1)
    Rz = oracle.attention_recall(np.zeros_like(q), k, M)
    np.testing.assert_allclose(Rz, (M & causal[None]).sum(-1) / np.arange(1, n + 1)[None], atol=1e-12)
    # the same quantity through the log-sum-exps of masked and dense attention
    _, lse = oracle.attention_with_mask(q, k, v, M)
    _, lsed = oracle.dense_attention(q, k, v)
    np.testing.assert_allclose(R, np.exp(lse - lsed), atol=1e-12)


# ---------------------------------------------------------------- block-sparse

def test_block_scores_brute_force():
    n, d = 256, 5
    q, k, _ = rand_qkv(2, 1, n, d, seed=8)
    u = oracle.block_scores(q, k, 1, block=64)
    for b in range(4):
        for c in range(4):
            if c > b:
                assert u[b, c] == -np.inf
                continue
            qm = [sum(q[1, 64 * b + t, e] for t in range(64)) / 64 for e in range(d)]
            km = [sum(k[0, 64 * c + t, e] for t in range(64)) / 64 for e in range(d)]
            want = sum(qm[e] * km[e] for e in range(d)) / math.sqrt(d)
            assert abs(u[b, c] - want) < 1e-12


def test_block_scores_ragged_last_block():
    """N not a multiple of 64: the last block is the mean of its rows."""
    n, d = 64 * 3 + 17, 4
    q, k, _ = rand_qkv(1, 1, n, d, seed=9)
    u = oracle.block_scores(q, k, 0, block=64)
    assert u.shape == (4, 4)
    qm = [sum(q[0, 192 + t, e] for t in range(17)) / 17 for e in range(d)]
    for c in range(4):
        rows = range(64 * c, min(64 * c + 64, n))
        km = [sum(k[0, t, e] for t in rows) / len(rows) for e in range(d)]
        want = sum(qm[e] * km[e] for e in range(d)) / math.sqrt(d)
        assert abs(u[3, c] - want) < 1e-12


def test_index_ragged_last_block():
    """N not a multiple of 64: the last query block ends at row N-1, and its
    blocks and columns stop there too."""
    n = 64 * 5 + 23
    v_idx, s_idx = random_sets(2, n, 9, 30, seed=12)
    idx = oracle.build_index(v_idx, s_idx, n)
    assert idx.block_count.shape == (2, 6)
    M = oracle.index_mask(idx, n)
    Mx = oracle.exact_union_mask(v_idx, s_idx, n)
    assert np.all(M[Mx])                          # every selected entry is covered
    for h in range(2):
        for t in range(int(idx.column_count[h, 5])):
            assert idx.column_index[h, 5, t] <= n - 1
        # rows of the last block see no key past themselves
        assert not np.any(np.triu(M[h], 1))


def test_block_sparse_full_topk_is_dense():
    n, d = 320, 16
    q, k, v = rand_qkv(2, 1, n, d, seed=10)
    cnt, offs, _ = oracle.block_sparse_select(q, k, [0, 1], topk=100)
    nb = n // 64
    for b in range(nb):
        assert cnt[0, b] == b + 1 and offs[0, b, : b + 1].tolist() == [64 * c for c in range(b + 1)]
    idx = oracle.IndexArrays(cnt, offs, np.zeros_like(cnt), np.zeros((2, nb, 0), np.int32))
    O, _ = oracle.attention_with_mask(q, k, v, oracle.index_mask(idx, n))
    Od, _ = oracle.dense_attention(q, k, v)
    np.testing.assert_allclose(O, Od, atol=1e-13)


def test_block_sparse_topk_picks_best_blocks():
    n, d = 64 * 12, 8
    q, k, _ = rand_qkv(1, 1, n, d, seed=12)
    cnt, offs, scores = oracle.block_sparse_select(q, k, [0], topk=3)
    for b in range(12):
        chosen = set((offs[0, b, : cnt[0, b]] // 64).tolist())
        assert len(chosen) == min(3, b + 1)
        for c in range(b + 1):
            if c not in chosen:
                assert all(scores[0, b, x] >= scores[0, b, c] for x in chosen)


def test_index_caps():
    assert index_caps(1 << 20, 1000, 6096) == (6096, 1000)
    assert index_caps(4096, 64, 256) == (64, 64)


def _brute_decode(q, k, v, topk, scale):
    """Plain loops: scores, the top-k by score (ties to the lower index),
    softmax over them, the weighted V sum and the kept share of e^s."""
    Hq, D = q.shape
    G = Hq // k.shape[0]
    N = k.shape[1]
    outs, lses, recs, idxs = [], [], [], []
    for h in range(Hq):
        g = h // G
        s = [scale * sum(float(q[h, d]) * float(k[g, j, d]) for d in range(D)) for j in range(N)]
        order = sorted(range(N), key=lambda j: (-s[j], j))[:topk]
        sel = sorted(order)
        m = max(s[j] for j in sel)
        w = [math.exp(s[j] - m) for j in sel]
        tot = sum(w)
        outs.append([sum(w[t] * float(v[g, sel[t], d]) for t in range(len(sel))) / tot for d in range(D)])
        lses.append(m + math.log(tot))
        m_all = max(s)
        recs.append(tot * math.exp(m - m_all) / sum(math.exp(x - m_all) for x in s))
        idxs.append(sel)
    return np.array(outs), np.array(lses), np.array(recs), np.array(idxs)


@pytest.mark.parametrize("hq,hkv,n,d,topk,seed", [(2, 1, 9, 4, 3, 0), (4, 2, 13, 3, 5, 1), (3, 3, 7, 5, 7, 2)])
def test_decode_sparse_brute_force(hq, hkv, n, d, topk, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    k[:, 2] = k[:, 5]                                  # equal scores: the tie goes to the lower index
    out, lse, rec, idx = oracle.decode_sparse_attention(q, k, v, topk, scale=0.7)
    bo, bl, br, bi = _brute_decode(q, k, v, topk, 0.7)
    np.testing.assert_array_equal(idx, bi)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rec, br, rtol=1e-12, atol=1e-12)


def test_decode_sparse_closed_forms():
    """All keys: the dense attention of the last row of a causal prefill whose
    last query is q, recovery 1.  One key: V at the highest score, lse = that
    score, recovery = its softmax weight.  A zero query: every score 0, so the
    first k keys (ties to the lower index), their mean V, recovery k / N."""
    rng = np.random.default_rng(3)
    hq, hkv, n, d = 4, 2, 40, 16
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    out, lse, rec, idx = oracle.decode_sparse_attention(q, k, v, n)
    qf = np.zeros((hq, n, d))
    qf[:, -1] = q
    dense, dlse = oracle.dense_attention(qf, k, v)
    np.testing.assert_allclose(out, dense[:, -1], atol=1e-12)
    np.testing.assert_allclose(lse, dlse[:, -1], atol=1e-12)
    np.testing.assert_allclose(rec, 1.0, atol=1e-12)
    s = oracle.decode_scores(q, k)
    out, lse, rec, idx = oracle.decode_sparse_attention(q, k, v, 1)
    G = hq // hkv
    for h in range(hq):
        j = int(np.argmax(s[h]))
        assert idx[h, 0] == j
        np.testing.assert_allclose(out[h], v[h // G, j], atol=1e-12)
        np.testing.assert_allclose(lse[h], s[h, j], atol=1e-12)
        np.testing.assert_allclose(rec[h], np.exp(s[h, j]) / np.exp(s[h]).sum(), atol=1e-12)
    out, lse, rec, idx = oracle.decode_sparse_attention(np.zeros((hq, d)), k, v, 7)
    np.testing.assert_array_equal(idx, np.tile(np.arange(7), (hq, 1)))
    for h in range(hq):
        np.testing.assert_allclose(out[h], v[h // G, :7].mean(axis=0), atol=1e-12)
    np.testing.assert_allclose(rec, 7 / n, atol=1e-12)


def _brute_decode_varlen(q, k, v, topk, scale, lens):
    """Plain loops over caches of different lengths: kv head g has the keys
    j < lens[g] only.  The top-k of those by score (ties to the lower index);
    when fewer than topk exist, the selection is filled with the positions
    lens[g], lens[g] + 1, ... (no weight).  Softmax, V sum and kept share over
    the keys that exist; no key: out 0, lse -inf, kept share 0."""
    Hq, D = q.shape
    G = Hq // k.shape[0]
    outs, lses, recs, idxs = [], [], [], []
    for h in range(Hq):
        g = h // G
        L = int(lens[g])
        s = [scale * sum(float(q[h, d]) * float(k[g, j, d]) for d in range(D)) for j in range(L)]
        sel = sorted(sorted(range(L), key=lambda j: (-s[j], j))[:topk])
        idxs.append(sel + list(range(L, L + topk - len(sel))))
        if not sel:
            outs.append([0.0] * D)
            lses.append(-math.inf)
            recs.append(0.0)
            continue
        m = max(s[j] for j in sel)
        w = [math.exp(s[j] - m) for j in sel]
        tot = sum(w)
        outs.append([sum(w[t] * float(v[g, sel[t], d]) for t in range(len(sel))) / tot for d in range(D)])
        lses.append(m + math.log(tot))
        m_all = max(s)
        recs.append(tot * math.exp(m - m_all) / sum(math.exp(x - m_all) for x in s))
    return np.array(outs), np.array(lses), np.array(recs), np.array(idxs)


@pytest.mark.parametrize("hq,hkv,n,d,topk,lens,seed", [
    (4, 2, 12, 4, 5, (7, 12), 0),        # one short cache, one full
    (6, 3, 10, 3, 4, (0, 3, 4), 1),      # empty, shorter than topk, exactly topk
    (2, 2, 9, 5, 9, (9, 1), 2),          # topk = capacity; a single key
])
def test_decode_varlen_brute_force(hq, hkv, n, d, topk, lens, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    for g, L in enumerate(lens):                       # rows past a cache's end are not keys
        k[g, L:] = np.nan
        v[g, L:] = np.nan
    if lens[0] > 5:
        k[0, 2] = k[0, 5]                              # equal scores inside the cache
    out, lse, rec, idx = oracle.decode_sparse_attention(q, k, v, topk, scale=0.6, cache_len=np.array(lens))
    bo, bl, br, bi = _brute_decode_varlen(q, k, v, topk, 0.6, lens)
    np.testing.assert_array_equal(idx, bi)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rec, br, rtol=1e-12, atol=1e-12)


def test_decode_varlen_reduces_to_shorter_caches():
    """A cache of length L inside a larger capacity gives what a cache of
    exactly L keys gives (L >= topk); with L < topk, the dense attention of
    the last row of a causal prefill over those L keys, recovery 1."""
    rng = np.random.default_rng(5)
    hq, hkv, n, d = 6, 3, 50, 16
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    lens = np.array([31, 50, 12])
    out, lse, rec, idx = oracle.decode_sparse_attention(q, k, v, 20, cache_len=lens)
    for g in range(hkv):
        L = int(lens[g])
        hs = slice(2 * g, 2 * g + 2)
        if L >= 20:
            o2, l2, r2, i2 = oracle.decode_sparse_attention(q[hs], k[g:g + 1, :L], v[g:g + 1, :L], 20)
            np.testing.assert_array_equal(idx[hs], i2)
            np.testing.assert_allclose(out[hs], o2, atol=1e-12)
            np.testing.assert_allclose(lse[hs], l2, atol=1e-12)
            np.testing.assert_allclose(rec[hs], r2, atol=1e-12)
        else:
            qf = np.zeros((2, L, d))
            qf[:, -1] = q[hs]
            dense, dlse = oracle.dense_attention(qf, k[g:g + 1, :L], v[g:g + 1, :L])
            np.testing.assert_allclose(out[hs], dense[:, -1], atol=1e-12)
            np.testing.assert_allclose(lse[hs], dlse[:, -1], atol=1e-12)
            np.testing.assert_allclose(rec[hs], 1.0, atol=1e-12)
            np.testing.assert_array_equal(idx[hs], np.tile(np.arange(20), (2, 1)))


def test_decode_scores_gqa_and_given_keys():
    """q head h reads kv head h // (Hq / Hkv): swapping the two kv heads swaps
    the scores of their q heads.  A given key set is used as is."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 8))
    k = rng.standard_normal((2, 30, 8))
    v = rng.standard_normal((2, 30, 8))
    s = oracle.decode_scores(q, k)
    s2 = oracle.decode_scores(q, k[::-1].copy())
    scale = 1 / np.sqrt(8)
    for h in range(4):
        np.testing.assert_allclose(s[h], scale * k[h // 2] @ q[h], atol=1e-12)
        np.testing.assert_allclose(s2[h], scale * k[1 - h // 2] @ q[h], atol=1e-12)
    given = np.array([[0, 5, 29]] * 4)
    out, lse, rec, idx = oracle.decode_sparse_attention(q, k, v, 3, idx=given)
    np.testing.assert_array_equal(idx, given)
    for h in range(4):
        w = np.exp(s[h, given[h]] - s[h, given[h]].max())
        np.testing.assert_allclose(out[h], (w[:, None] * v[h // 2, given[h]]).sum(0) / w.sum(), atol=1e-12)
