/*
 * Oracle index builder (plain C, test infrastructure only).
 *
 * Turns a head's selected slash diagonals and vertical columns into, for every
 * 64-row query block, a list of 64-wide key blocks plus the selected columns
 * that those blocks leave uncovered.  The pages fix the inputs (a column index
 * and a slash index per head: talk slides "System-Algorithm Co-design", slide
 * "Dynamic sparsity in attention") and ask that the sparse work come in large
 * blocks for the matrix units and be built online with little overhead ("How to
 * optimise the TTFT of an 8B LLM with 1M tokens to 20 seconds", section "How to
 * co-design the algorithm and the system", principles 1 and 2).  They leave the
 * covering rule open; the reading implemented here is:
 *
 *   query block b covers rows r0 = 64b .. r1 = min(64b+63, N-1).
 *   Each selected offset o <= r1 needs keys [a, e] = [max(0, r0-o), r1-o].
 *   Visit those ranges by descending o (ascending a) with cov = 0:
 *     if e < cov the range is already covered, skip it;
 *     else emit a block starting at st = max(a, cov) and set cov = st + 64.
 *   Columns: every selected j <= r1 that no emitted block contains, ascending.
 *
 * Blocks are not aligned to multiples of 64.  Entries past each count are left
 * untouched.  Returns 0, or -1 if a capacity is too small.
 */
#include <stdint.h>

int oracle_build_index(int n_heads, int64_t n, int block,
                       const int32_t *v_idx, int kv, const int32_t *s_idx, int ks,
                       int32_t *block_count, int32_t *block_offset, int cap_b,
                       int32_t *column_count, int32_t *column_index, int cap_c)
{
    int64_t nqb = (n + block - 1) / block;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int64_t t = 0; t < (int64_t)n_heads * nqb; ++t) {
        int64_t h = t / nqb, b = t % nqb;
        int64_t r0 = b * block;
        int64_t r1 = r0 + block - 1;
        if (r1 > n - 1) r1 = n - 1;
        const int32_t *S = s_idx + h * ks;
        const int32_t *V = v_idx + h * kv;
        int32_t *blk = block_offset + t * (int64_t)cap_b;
        int32_t *col = column_index + t * (int64_t)cap_c;
        int64_t cov = 0;
        int cnt = 0;
        for (int i = ks - 1; i >= 0; --i) {
            int64_t o = S[i];
            if (o > r1) continue;
            int64_t a = r0 - o > 0 ? r0 - o : 0;
            int64_t e = r1 - o;
            if (e < cov) continue;
            int64_t st = a > cov ? a : cov;
            if (cnt >= cap_b) { bad = 1; break; }
            blk[cnt++] = (int32_t)st;
            cov = st + block;
        }
        block_count[t] = cnt;
        int p = 0, cc = 0;
        for (int i = 0; i < kv; ++i) {
            int64_t j = V[i];
            if (j > r1) break;
            while (p < cnt && (int64_t)blk[p] + block - 1 < j) ++p;
            int inside = (p < cnt && blk[p] <= j);
            if (inside) continue;
            if (cc >= cap_c) { bad = 1; break; }
            col[cc++] = (int32_t)j;
        }
        column_count[t] = cc;
    }
    return bad ? -1 : 0;
}
