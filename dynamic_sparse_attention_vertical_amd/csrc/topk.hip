// Exact top-k of the vertical and slash scores, per head, for gfx950.
//
// The pages warn that per-query top-k on a GPU is not kernel friendly ("How to
// optimise the TTFT of an 8B LLM with 1M tokens to 20 seconds", section on
// co-designing algorithm and system); here it is one selection per head over
// N scores, done as a radix select on the scores' bit patterns.  Scores are
// non-negative floats, so their IEEE bit patterns order like unsigned
// integers.  Three histogram passes (11 + 11 + 10 bits) find the k-th largest
// pattern T and how many entries equal to T are needed; a count / scan / write
// sequence then emits, in ascending index order, every entry above T and the
// lowest-index entries equal to T.  Ties therefore go to the lower index and
// the result is exact and deterministic (integer atomics only).
//
// Rows: 2*hq of them -- rows [0, hq) select vertical columns (k0 each),
// rows [hq, 2hq) select slash diagonals (k1 each).
#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = kTopkSlice / kThreads;     // 16 consecutive elements per thread

struct RowView {
    const float *src;
    int32_t *dst;
    int32_t k;
};

__device__ __forceinline__ RowView row_view(const TopkArgs &a, int row) {
    RowView r;
    if (row < a.hq) {
        r.src = a.src0 + (int64_t)row * a.n;
        r.dst = a.dst0 + (int64_t)row * a.k0;
        r.k = a.k0;
    } else {
        r.src = a.src1 + (int64_t)(row - a.hq) * a.n;
        r.dst = a.dst1 + (int64_t)(row - a.hq) * a.k1;
        r.k = a.k1;
    }
    return r;
}

// entries of a row: n, or the row's own length (clamped into [0, n])
__device__ __forceinline__ int64_t row_n(const TopkArgs &a, int row) {
    if (a.row_len == nullptr) return a.n;
    const int64_t len = a.row_len[(row % a.hq) / a.row_len_div];   // the two sets of a row share it
    return len < 0 ? 0 : (len > a.n ? a.n : len);
}

// pass p: bucket bits and the prefix the element must match
__device__ __forceinline__ int pass_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__device__ __forceinline__ int pass_bits(int p) { return p == 2 ? 10 : 11; }

__global__ __launch_bounds__(kThreads) void topk_init_kernel(TopkArgs a) {
    const int row = blockIdx.x;
    for (int i = threadIdx.x; i < 2048; i += kThreads) a.hist[(int64_t)row * 2048 + i] = 0u;
    if (threadIdx.x == 0) {
        RowView r = row_view(a, row);
        a.state[row * 4 + 0] = 0u;                 // prefix of the threshold found so far
        a.state[row * 4 + 1] = (uint32_t)r.k;      // entries still to take at or below it
    }
}

__device__ __forceinline__ void load_slice(const float *src, int64_t n, int64_t e0, uint32_t (&x)[kPer],
                                           bool (&valid)[kPer]) {
    if (e0 + kPer <= n) {
#pragma unroll
        for (int c = 0; c < kPer / 4; ++c) {
            u32x4 w = *reinterpret_cast<const u32x4 *>(src + e0 + 4 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i) { x[4 * c + i] = w[i]; valid[4 * c + i] = true; }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            valid[i] = e0 + i < n;
            x[i] = valid[i] ? __float_as_uint(src[e0 + i]) : 0u;
        }
    }
}

template <int P>
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(TopkArgs a) {
    __shared__ uint32_t h[2048];
    const int row = blockIdx.y;
    const int64_t e0 = (int64_t)blockIdx.x * kTopkSlice + threadIdx.x * kPer;
    constexpr int nb = (P == 2) ? 1024 : 2048;
    for (int i = threadIdx.x; i < nb; i += kThreads) h[i] = 0u;
    __syncthreads();
    RowView r = row_view(a, row);
    const uint32_t prefix = a.state[row * 4 + 0];
    uint32_t x[kPer];
    bool valid[kPer];
    load_slice(r.src, row_n(a, row), e0, x, valid);
    const int sh = pass_shift(P);
    const int hi_sh = sh + pass_bits(P);         // bits above the bucket must equal prefix
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (!valid[i]) continue;
        const bool match = (P == 0) ? true : ((x[i] >> hi_sh) == prefix);
        if (match) atomicAdd(&h[(x[i] >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nb; i += kThreads)
        if (h[i]) atomicAdd(&a.hist[(int64_t)row * 2048 + i], h[i]);
}

// exclusive prefix sum over the 256 threads of a workgroup
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *tmp, uint32_t *total) {
    const int t = threadIdx.x;
    tmp[t] = v;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        uint32_t add = t >= off ? tmp[t - off] : 0u;
        __syncthreads();
        tmp[t] += add;
        __syncthreads();
    }
    const uint32_t incl = tmp[t];
    if (total) *total = tmp[kThreads - 1];
    __syncthreads();
    return incl - v;
}

template <int P>
__global__ __launch_bounds__(kThreads) void topk_pick_kernel(TopkArgs a) {
    __shared__ uint32_t tmp[kThreads];
    const int row = blockIdx.x;
    constexpr int nb = (P == 2) ? 1024 : 2048;
    constexpr int per = nb / kThreads;
    uint32_t *hist = a.hist + (int64_t)row * 2048;
    const uint32_t krem = a.state[row * 4 + 1];
    // thread t owns buckets nb-1-t*per ... nb-per-t*per (top down)
    uint32_t c[per];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        c[i] = hist[nb - 1 - (threadIdx.x * per + i)];
        sum += c[i];
    }
    __syncthreads();
    const uint32_t above = block_exclusive_scan(sum, tmp, nullptr);
#pragma unroll
    for (int i = 0; i < per; ++i) hist[nb - 1 - (threadIdx.x * per + i)] = 0u;   // ready for next pass
    if (above < krem && krem <= above + sum) {
        uint32_t acc = above;
#pragma unroll
        for (int i = 0; i < per; ++i) {
            if (acc < krem && krem <= acc + c[i]) {
                const uint32_t bucket = (uint32_t)(nb - 1 - (threadIdx.x * per + i));
                const uint32_t prefix = a.state[row * 4 + 0];
                a.state[row * 4 + 0] = (prefix << pass_bits(P)) | bucket;
                a.state[row * 4 + 1] = krem - acc;
            }
            acc += c[i];
        }
    }
}

__global__ __launch_bounds__(kThreads) void topk_count_kernel(TopkArgs a) {
    __shared__ uint32_t red[2][kThreads / 64];
    const int row = blockIdx.y;
    const int64_t e0 = (int64_t)blockIdx.x * kTopkSlice + threadIdx.x * kPer;
    RowView r = row_view(a, row);
    const uint32_t T = a.state[row * 4 + 0];
    uint32_t x[kPer];
    bool valid[kPer];
    load_slice(r.src, row_n(a, row), e0, x, valid);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        gt += (valid[i] && x[i] > T) ? 1u : 0u;
        eq += (valid[i] && x[i] == T) ? 1u : 0u;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        gt += __shfl_xor(gt, off, 64);
        eq += __shfl_xor(eq, off, 64);
    }
    if ((threadIdx.x & 63) == 0) { red[0][threadIdx.x >> 6] = gt; red[1][threadIdx.x >> 6] = eq; }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t G = 0, Q = 0;
        for (int w = 0; w < kThreads / 64; ++w) { G += red[0][w]; Q += red[1][w]; }
        const int64_t o = ((int64_t)row * a.nslices + blockIdx.x) * 2;
        a.cnt[o] = G;
        a.cnt[o + 1] = Q;
    }
}

// per row: slice output offsets and equal-entries-before counts
__global__ __launch_bounds__(kThreads) void topk_scan_kernel(TopkArgs a) {
    __shared__ uint32_t tmp[kThreads];
    const int row = blockIdx.x;
    const uint32_t krem = a.state[row * 4 + 1];
    uint32_t eq_run = 0, sel_run = 0;
    for (int s0 = 0; s0 < a.nslices; s0 += kThreads) {
        const int s = s0 + threadIdx.x;
        const int64_t o = ((int64_t)row * a.nslices + s) * 2;
        const uint32_t gt = s < a.nslices ? a.cnt[o] : 0u;
        const uint32_t eq = s < a.nslices ? a.cnt[o + 1] : 0u;
        uint32_t eq_tot;
        const uint32_t eq_before = eq_run + block_exclusive_scan(eq, tmp, &eq_tot);
        const uint32_t chosen = eq_before >= krem ? 0u : min(eq, krem - eq_before);
        uint32_t sel_tot;
        const uint32_t sel_before = sel_run + block_exclusive_scan(gt + chosen, tmp, &sel_tot);
        if (s < a.nslices) {
            a.off[o] = sel_before;
            a.off[o + 1] = eq_before;
        }
        eq_run += eq_tot;
        sel_run += sel_tot;
    }
}

__global__ __launch_bounds__(kThreads) void topk_write_kernel(TopkArgs a) {
    __shared__ uint32_t tmp[kThreads];
    const int row = blockIdx.y;
    const int64_t e0 = (int64_t)blockIdx.x * kTopkSlice + threadIdx.x * kPer;
    RowView r = row_view(a, row);
    const uint32_t T = a.state[row * 4 + 0];
    const uint32_t krem = a.state[row * 4 + 1];
    const int64_t o = ((int64_t)row * a.nslices + blockIdx.x) * 2;
    const uint32_t slice_off = a.off[o], slice_eq = a.off[o + 1];
    uint32_t x[kPer];
    bool valid[kPer];
    load_slice(r.src, row_n(a, row), e0, x, valid);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        gt += (valid[i] && x[i] > T) ? 1u : 0u;
        eq += (valid[i] && x[i] == T) ? 1u : 0u;
    }
    const uint32_t eq_before = slice_eq + block_exclusive_scan(eq, tmp, nullptr);
    const uint32_t chosen = eq_before >= krem ? 0u : min(eq, krem - eq_before);
    uint32_t pos = slice_off + block_exclusive_scan(gt + chosen, tmp, nullptr);
    uint32_t eq_seen = eq_before;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (!valid[i]) continue;
        bool take = x[i] > T;
        if (x[i] == T) {
            take = eq_seen < krem;
            ++eq_seen;
        }
        if (take) {
            if (pos < (uint32_t)r.k) r.dst[pos] = (int32_t)(e0 + i);
            ++pos;
        }
    }
    // a row with fewer than k entries: every entry is taken (positions
    // 0 .. len - 1 above), and the selection goes on with the positions after
    const int64_t len = row_n(a, row);
    if (blockIdx.x == 0)
        for (int64_t i = len + threadIdx.x; i < r.k; i += kThreads) r.dst[i] = (int32_t)i;
}

// ---- One workgroup per row ----
// The same selection in a single launch: a 1024-thread workgroup takes one
// row through the three histogram passes and the ordered write, reading the
// row once per pass (after the first pass from the caches).  For many rows
// at once (the decode step's one row per q head) this replaces the ten
// launches above, most of whose time is the fixed cost of a launch.
constexpr int kRowThreads = 1024;
constexpr int kRowPer = 16;                             // consecutive elements per thread and tile
constexpr int kRowTile = kRowThreads * kRowPer;

// Tiles of kRowTile elements, thread t holding elements e0 + 16t .. e0 + 16t + 15.
// Full tiles stream with one tile loaded ahead and exactly four 16-byte loads
// per thread per tile (so the compiler can wait for the older tile only); the
// partial last tile is read element by element afterwards.  visit(x, cnt, e0)
// sees a tile (cnt valid elements in this thread) and returns false to stop
// (a workgroup-uniform decision).
__device__ __forceinline__ void row_load_full(const uint32_t *src, int64_t e, uint32_t (&x)[kRowPer]) {
#pragma unroll
    for (int c = 0; c < kRowPer / 4; ++c) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(src + e + 4 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * c + i] = w[i];
    }
}
template <typename F>
__device__ __forceinline__ void row_tiles(const uint32_t *src, int64_t n, F &&visit) {
    const int64_t mine = (int64_t)threadIdx.x * kRowPer;
    const int64_t nfull = n / kRowTile * kRowTile;
    uint32_t xa[kRowPer], xb[kRowPer];
    if (nfull > 0) row_load_full(src, mine, xa);
    for (int64_t e0 = 0; e0 < nfull; e0 += kRowTile) {
        // the tile after this one (after the last full tile: that tile again, unused)
        const int64_t nx = e0 + kRowTile < nfull ? e0 + kRowTile : e0;
        row_load_full(src, nx + mine, xb);
        if (!visit(xa, kRowPer, e0)) return;
#pragma unroll
        for (int i = 0; i < kRowPer; ++i) xa[i] = xb[i];
    }
    if (nfull < n) {
        const int64_t e = nfull + mine;
        const int cnt = e < n ? (n - e < kRowPer ? (int)(n - e) : kRowPer) : 0;
#pragma unroll
        for (int i = 0; i < kRowPer; ++i) xa[i] = i < cnt ? src[e + i] : 0u;
        visit(xa, cnt, nfull);
    }
}

// exclusive prefix sum over the workgroup's 1024 threads, and the total
__device__ __forceinline__ uint32_t row_scan(uint32_t v, uint32_t *wsum, uint32_t &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kRowThreads / 64; ++w) {
        const uint32_t sw = wsum[w];
        before += w < wave ? sw : 0u;
        tot += sw;
    }
    __syncthreads();                                    // wsum is free again
    total = tot;
    return before + incl - v;
}

// Entries staged in LDS after the first pass (index and key, 8 bytes each).
constexpr int kStage = 6144;

__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(TopkArgs a) {
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wsum[kRowThreads / 64];
    __shared__ uint32_t sel[3];
    __shared__ uint32_t st_key[kStage];
    __shared__ int32_t st_idx[kStage];
    const int row = blockIdx.x, tid = threadIdx.x;
    const RowView r = row_view(a, row);
    const uint32_t *src = reinterpret_cast<const uint32_t *>(r.src);
    const int64_t n = row_n(a, row);
    const uint32_t k = (uint32_t)r.k;
    uint32_t prefix = 0, krem = k, in_bucket = 0;
    if (n <= (int64_t)k) {                              // every entry, then the positions after the row's end
        for (int i = tid; i < (int)k; i += kRowThreads) r.dst[i] = i;
        return;
    }

    auto clear = [&]() {
        for (int i = tid; i < 2048; i += kRowThreads) hist[i] = 0u;
        __syncthreads();
    };
    // pass p's bucket of x, counted if x matches the prefix found so far
    auto count = [&](int p, uint32_t x) {
        const int sh = pass_shift(p), hi_sh = sh + pass_bits(p);
        if (hi_sh >= 32 || (x >> hi_sh) == prefix) atomicAdd(&hist[(x >> sh) & ((1u << pass_bits(p)) - 1u)], 1u);
    };
    // the bucket holding the krem-th largest counted entry (buckets top down,
    // thread t owning nb-1-t*per .. nb-per-t*per); krem becomes its rank
    // inside the bucket, in_bucket the bucket's count
    auto pick = [&](int p) {
        const int bits = pass_bits(p), nb = 1 << bits, per = nb / kRowThreads;
        const uint32_t c0 = hist[nb - 1 - tid * per], c1 = per == 2 ? hist[nb - 2 - tid * per] : 0u;
        uint32_t tot;
        const uint32_t above = row_scan(c0 + c1, wsum, tot);
        if (above < krem && krem <= above + c0 + c1) {
            const bool first = krem <= above + c0;
            sel[0] = (prefix << bits) | (uint32_t)(nb - 1 - tid * per - (first ? 0 : 1));
            sel[1] = krem - (first ? above : above + c0);
            sel[2] = first ? c0 : c1;
        }
        __syncthreads();
        prefix = sel[0];
        krem = sel[1];
        in_bucket = sel[2];
    };

    clear();
    row_tiles(src, n, [&](const uint32_t (&x)[kRowPer], int cnt, int64_t) {
#pragma unroll
        for (int i = 0; i < kRowPer; ++i)
            if (i < cnt) count(0, x[i]);
        return true;
    });
    __syncthreads();
    pick(0);
    // entries whose top 11 bits reach the chosen bucket: k - krem above it
    // (all selected) and in_bucket inside it
    const uint32_t staged = k - krem + in_bucket;
    if (staged <= (uint32_t)kStage) {
        // the second and last pass over the row stages them in index order;
        // the other two radix steps and the ordered write then run in LDS
        const uint32_t b0 = prefix;
        uint32_t base = 0;
        row_tiles(src, n, [&](const uint32_t (&x)[kRowPer], int cnt, int64_t e0) {
            uint32_t c = 0;
#pragma unroll
            for (int i = 0; i < kRowPer; ++i) c += (i < cnt && (x[i] >> 21) >= b0) ? 1u : 0u;
            uint32_t tot;
            uint32_t pos = base + row_scan(c, wsum, tot);
            const int64_t e = e0 + (int64_t)tid * kRowPer;
#pragma unroll
            for (int i = 0; i < kRowPer; ++i) {
                if (i < cnt && (x[i] >> 21) >= b0) {
                    if (pos < (uint32_t)kStage) {
                        st_key[pos] = x[i];
                        st_idx[pos] = (int32_t)(e + i);
                    }
                    ++pos;
                }
            }
            base += tot;
            return true;
        });
        __syncthreads();
        for (int p = 1; p < 3; ++p) {
            clear();
            for (uint32_t i = tid; i < staged; i += kRowThreads) count(p, st_key[i]);
            __syncthreads();
            pick(p);
        }
        const uint32_t T = prefix;
        uint32_t need = krem, out = 0;
        for (uint32_t i0 = 0; i0 < staged; i0 += kRowThreads) {
            const uint32_t i = i0 + tid;
            const uint32_t x = i < staged ? st_key[i] : 0u;
            const uint32_t gt = (i < staged && x > T) ? 1u : 0u, eq = (i < staged && x == T) ? 1u : 0u;
            uint32_t tot;
            const uint32_t ex = row_scan((gt << 16) | eq, wsum, tot);
            const uint32_t eq_before = ex & 0xffffu;
            if (gt || (eq && eq_before < need)) {
                const uint32_t pos = out + (ex >> 16) + min(eq_before, need);
                if (pos < k) r.dst[pos] = st_idx[i];
            }
            const uint32_t teq = min(tot & 0xffffu, need);
            out += (tot >> 16) + teq;
            need -= teq;
        }
        return;
    }
    // too many entries share the top bits: the other two radix steps and the
    // ordered write each take a pass over the row
    for (int p = 1; p < 3; ++p) {
        clear();
        row_tiles(src, n, [&](const uint32_t (&x)[kRowPer], int cnt, int64_t) {
#pragma unroll
            for (int i = 0; i < kRowPer; ++i)
                if (i < cnt) count(p, x[i]);
            return true;
        });
        __syncthreads();
        pick(p);
    }
    // every entry above T, and the krem lowest-index entries equal to T, in
    // ascending index order; the tile's scan carries both counts (above in
    // the high half, equal in the low half: at most 16384 each)
    const uint32_t T = prefix;
    uint32_t need = krem, base = 0;
    row_tiles(src, n, [&](const uint32_t (&x)[kRowPer], int cnt, int64_t e0) {
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int i = 0; i < kRowPer; ++i) {
            gt += (i < cnt && x[i] > T) ? 1u : 0u;
            eq += (i < cnt && x[i] == T) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t ex = row_scan((gt << 16) | eq, wsum, tot);
        const uint32_t eq_before = ex & 0xffffu;
        uint32_t pos = base + (ex >> 16) + min(eq_before, need);
        uint32_t eq_seen = eq_before;
        const int64_t e = e0 + (int64_t)tid * kRowPer;
#pragma unroll
        for (int i = 0; i < kRowPer; ++i) {
            if (i >= cnt) continue;
            bool take = x[i] > T;
            if (x[i] == T) {
                take = eq_seen < need;
                ++eq_seen;
            }
            if (take) {
                if (pos < k) r.dst[pos] = (int32_t)(e + i);
                ++pos;
            }
        }
        const uint32_t teq = min(tot & 0xffffu, need);
        base += (tot >> 16) + teq;
        need -= teq;
        return base < k;                              // every selected entry written
    });
}

}  // namespace

namespace {
__global__ __launch_bounds__(256) void seq_lengths_kernel(Varlen vl, int64_t nmax, int32_t *len) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= vl.nseq) return;
    const int64_t a = min(max((int64_t)vl.cu[i], (int64_t)0), vl.rows);
    const int64_t b = min(max((int64_t)vl.cu[i + 1], a), vl.rows);
    len[i] = (int32_t)min(b - a, nmax);
}
}  // namespace

hipError_t launch_seq_lengths(const Varlen &vl, int64_t nmax, int32_t *len, hipStream_t s) {
    hipLaunchKernelGGL(seq_lengths_kernel, dim3((unsigned)((vl.nseq + 255) / 256)), dim3(256), 0, s, vl, nmax, len);
    return hipGetLastError();
}

hipError_t launch_topk_rows(const TopkArgs &a, hipStream_t s) {
    const int rows = a.rows > 0 ? a.rows : 2 * a.hq;
    hipLaunchKernelGGL(topk_row_kernel, dim3(rows), dim3(kRowThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
    const int rows = a.rows > 0 ? a.rows : 2 * a.hq;
    hipError_t e;
    hipLaunchKernelGGL(topk_init_kernel, dim3(rows), dim3(kThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 grid(a.nslices, rows);
    hipLaunchKernelGGL(topk_hist_kernel<0>, grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(topk_pick_kernel<0>, dim3(rows), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(topk_hist_kernel<1>, grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(topk_pick_kernel<1>, dim3(rows), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(topk_hist_kernel<2>, grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(topk_pick_kernel<2>, dim3(rows), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(topk_count_kernel, grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(topk_scan_kernel, dim3(rows), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(topk_write_kernel, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace msa
