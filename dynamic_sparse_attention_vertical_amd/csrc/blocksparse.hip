// Block-sparse work lists from mean-pooled block scores, gfx950.
//
// Block-sparse heads (talk slides "System-Algorithm Co-design", patterns
// slide; "MInference 1.0 README", kernel-only block_sparse_attention(q, k, v,
// topk)) attend to a few whole 64x64 blocks.  Reading used here: the block
// score is the scaled dot product of the 64-row means of q and k,
// u[b, c] = scale <qm[b], km[c]> (c <= b), and query block b keeps its
// min(topk, b+1) best key blocks, exact ties to the lower c, listed as
// ascending key starts 64c with no extra columns.
//
//   pool:   one workgroup per (head, block): 128 threads, 16-byte row reads.
//   score:  the block scores of up to 1024 query blocks at a time, as a
//           tiled product of the means: one workgroup per (q head, 64 query
//           blocks, 64 key blocks) below the diagonal, both 64 x 128 tiles of
//           means in LDS, each thread 4 x 4 scores; written to the workspace
//           as order-preserving integer keys.
//   select: one workgroup per (q head, query block): its row of keys into
//           LDS (rows past 15360 key blocks stay in the workspace), 4 x 8-bit
//           radix select for the k-th key (the bin found by a parallel scan),
//           then an in-order compaction (ties -> lower c).
#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;
// Keys of a query block's row held in LDS for its selection (60 KB, within
// the 64 KB of dynamic LDS a launch gets by default); longer rows (query
// blocks past 15360, i.e. keys past 983,040) are read from the workspace.
constexpr int kBsLdsKeys = 15360;

// One workgroup (128 threads) per (head, block): thread t adds up 8
// consecutive dimensions (one 16-byte load for bf16, two for fp32) of rows
// t/16, t/16 + 8, ...; the eight row groups are then summed through LDS.
template <typename T>
__global__ __launch_bounds__(kD) void bs_pool_kernel(BsArgs a) {
    __shared__ float part[8][kD];
    const int64_t nb = (a.n + 63) / 64;              // blocks per head in the pooled arrays
    const int c = blockIdx.x;
    // q heads, then kv heads, of each sequence of a packed batch in turn
    const int seq = blockIdx.y / (a.hq + a.hkv), head = blockIdx.y % (a.hq + a.hkv);
    const SeqSpan sp = seq_span(a.vl.cu, seq, a.vl.rows, a.n);
    if ((int64_t)c * 64 >= sp.n) return;             // past the end of a shorter packed sequence
    const T *src;
    float *dst;
    if (head < a.hq) {
        src = reinterpret_cast<const T *>(a.q) + ((int64_t)head * a.stride + sp.row0) * kD;
        dst = a.qm + (((int64_t)seq * a.hq + head) * nb + c) * kD;
    } else {
        src = reinterpret_cast<const T *>(a.k) + ((int64_t)(head - a.hq) * a.stride + sp.row0) * kD;
        dst = a.km + (((int64_t)seq * a.hkv + head - a.hq) * nb + c) * kD;
    }
    // a short last block (length not a multiple of 64) is the mean of its rows
    const int nrows = (int)min((int64_t)64, sp.n - (int64_t)c * 64);
    const int d0 = (threadIdx.x & 15) * 8, rg = threadIdx.x >> 4;
    float acc[8] = {};
    for (int r = rg; r < nrows; r += 8) {
        const T *row = src + ((int64_t)c * 64 + r) * kD + d0;
        if constexpr (sizeof(T) == 2) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(row);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += __uint_as_float(w[e] << 16);
                acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
            }
        } else {
            const f32x4 x0 = *reinterpret_cast<const f32x4 *>(row), x1 = *reinterpret_cast<const f32x4 *>(row + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] += x0[e];
                acc[4 + e] += x1[e];
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rg][d0 + e] = acc[e];
    __syncthreads();
    const int d = threadIdx.x;
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) s += part[g][d];
    dst[d] = nrows == 64 ? s * (1.f / 64.f) : s / (float)nrows;
}

__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Scores of query blocks row0 + 64 qt .. (+63) against key blocks 64 kt ..
// (+63) of q head h, for kt <= qt (blocks above the diagonal are not needed).
// Thread (ty, tx) computes query blocks 16 i + ty and key blocks 16 j + tx of
// the tile (i, j = 0..3); rows of 132 floats keep the four-wide LDS reads of
// the 16 key-block rows of a wave on distinct banks.
constexpr int kScorePitch = kD + 4;
__global__ __launch_bounds__(kThreads) void bs_score_kernel(BsArgs a) {
    __shared__ alignas(16) float qs[64 * kScorePitch];
    __shared__ alignas(16) float ks[64 * kScorePitch];
    const int kt = blockIdx.x, qt = blockIdx.y, h = blockIdx.z;   // h: head s * hq + h' of sequence s
    const int64_t nbr = (a.n + 63) / 64;                    // blocks per head in the arrays
    const int64_t nb = (seq_span(a.vl.cu, h / a.hq, a.vl.rows, a.n).n + 63) / 64;   // this sequence's
    const int64_t q0 = a.row0 + (int64_t)qt * 64;          // first query block of the tile
    if ((int64_t)kt * 64 > q0 + 63 || q0 >= nb) return;    // above the diagonal, or past the sequence
    const int G = a.hq / a.hkv;
    const float *qm = a.qm + (int64_t)h * nbr * kD;
    const float *km = a.km + (int64_t)(h / G) * nbr * kD;  // h / G: kv head s * hkv + h' / G
    // both tiles: 64 rows x 32 float4, eight per thread (rows past nb read row nb-1)
    for (int i = threadIdx.x; i < 64 * 32; i += kThreads) {
        const int r = i >> 5, c4 = i & 31;
        const int64_t qr = min(q0 + r, nb - 1), kr = min((int64_t)kt * 64 + r, nb - 1);
        *reinterpret_cast<f32x4 *>(&qs[r * kScorePitch + 4 * c4]) = *reinterpret_cast<const f32x4 *>(qm + qr * kD + 4 * c4);
        *reinterpret_cast<f32x4 *>(&ks[r * kScorePitch + 4 * c4]) = *reinterpret_cast<const f32x4 *>(km + kr * kD + 4 * c4);
    }
    __syncthreads();
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
#pragma unroll 4
    for (int d = 0; d < kD; d += 4) {
        f32x4 qv[4], kv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[i] = *reinterpret_cast<const f32x4 *>(&qs[(16 * i + ty) * kScorePitch + d]);
#pragma unroll
        for (int j = 0; j < 4; ++j) kv[j] = *reinterpret_cast<const f32x4 *>(&ks[(16 * j + tx) * kScorePitch + d]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] += qv[i][0] * kv[j][0] + qv[i][1] * kv[j][1] + qv[i][2] * kv[j][2] + qv[i][3] * kv[j][3];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t qb = q0 + 16 * i + ty;
        if (qb >= nb || qb >= a.row0 + a.chunk_rows) continue;
        uint32_t *row = a.keys + ((int64_t)h * a.chunk_rows + (qb - a.row0)) * nbr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t kb = (int64_t)kt * 64 + 16 * j + tx;
            if (kb < nb) row[kb] = order_key(acc[i][j] * a.scale);
        }
    }
}

__device__ __forceinline__ uint32_t scan256(uint32_t v, uint32_t *tmp) {
    const int t = threadIdx.x;
    tmp[t] = v;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        uint32_t add = t >= off ? tmp[t - off] : 0u;
        __syncthreads();
        tmp[t] += add;
        __syncthreads();
    }
    const uint32_t r = tmp[t] - v;
    __syncthreads();
    return r;
}

// Selection over one row of keys held at `keys`: the workgroup's LDS copy of
// the row when it fits (kLds), else the row in the workspace itself (read
// through the caches once per radix pass).
template <bool kLds>
__device__ __forceinline__ void select_row(const uint32_t *keys, int ncand, int kk, int32_t *out, int32_t cap_b,
                                           uint32_t *hist, uint32_t *tmp, uint32_t *sel_state) {
    if (threadIdx.x == 0) { sel_state[0] = 0u; sel_state[1] = (uint32_t)kk; }
    __syncthreads();
    for (int pass = 0; pass < 4; ++pass) {
        const int sh = 24 - 8 * pass;
        hist[threadIdx.x] = 0u;
        __syncthreads();
        const uint32_t prefix = sel_state[0];
        for (int c = threadIdx.x; c < ncand; c += kThreads) {
            const uint32_t x = keys[c];
            if (pass == 0 || (x >> (sh + 8)) == prefix) atomicAdd(&hist[(x >> sh) & 255u], 1u);
        }
        __syncthreads();
        // the bin holding the k-th largest key: thread t owns bin 255 - t, and
        // an exclusive scan over the threads counts the keys in higher bins;
        // exactly one bin has fewer than krem above it and krem or more with it
        const uint32_t krem = sel_state[1];
        const int bk = kThreads - 1 - (int)threadIdx.x;
        const uint32_t hb = hist[bk];
        const uint32_t above = scan256(hb, tmp);
        if (above < krem && above + hb >= krem) {
            sel_state[0] = (prefix << 8) | (uint32_t)bk;
            sel_state[1] = krem - above;
        }
        __syncthreads();
    }
    const uint32_t T = sel_state[0], need_eq = sel_state[1];
    // in-order compaction: thread t owns candidates [t*per, (t+1)*per)
    const int per = (ncand + kThreads - 1) / kThreads;
    const int c0 = threadIdx.x * per, c1 = min(ncand, c0 + per);
    uint32_t gt = 0, eq = 0;
    for (int c = c0; c < c1; ++c) { gt += keys[c] > T; eq += keys[c] == T; }
    const uint32_t eq_before = scan256(eq, tmp);
    const uint32_t chosen = eq_before >= need_eq ? 0u : min(eq, need_eq - eq_before);
    uint32_t pos = scan256(gt + chosen, tmp);
    uint32_t seen = eq_before;
    for (int c = c0; c < c1; ++c) {
        const uint32_t x = keys[c];
        bool take = x > T;
        if (x == T) { take = seen < need_eq; ++seen; }
        if (take) {
            if (pos < (uint32_t)cap_b) out[pos] = c * 64;
            ++pos;
        }
    }
}

__global__ __launch_bounds__(kThreads) void bs_select_kernel(BsArgs a) {
    extern __shared__ uint32_t keys[];              // [min(b + 1, kBsLdsKeys)]
    __shared__ uint32_t hist[256];
    __shared__ uint32_t tmp[kThreads];
    __shared__ uint32_t sel_state[2];
    const int64_t nbr = (a.n + 63) / 64;                 // blocks per head in the arrays
    const int64_t rows = min((int64_t)a.chunk_rows, nbr - a.row0);
    const int64_t b = a.row0 + rows - 1 - blockIdx.x;   // heavy rows first
    const int h = blockIdx.y;                            // head s * hq + h' of sequence s
    if (b * 64 >= seq_span(a.vl.cu, h / a.hq, a.vl.rows, a.n).n) return;   // past the sequence's end
    const int64_t item = (int64_t)h * nbr + b;
    int32_t *out = a.block_offset + item * a.cap_b;
    const int ncand = (int)b + 1;
    const int kk = min(a.topk, ncand);
    if (threadIdx.x == 0) {
        a.block_count[item] = kk;
        a.column_count[item] = 0;
    }
    if (ncand <= a.topk) {
        for (int c = threadIdx.x; c < ncand; c += kThreads) out[c] = c * 64;
        return;
    }
    const uint32_t *krow = a.keys + ((int64_t)h * a.chunk_rows + (b - a.row0)) * nbr;
    if (ncand <= kBsLdsKeys) {
        for (int c = threadIdx.x; c < ncand; c += kThreads) keys[c] = krow[c];
        select_row<true>(keys, ncand, kk, out, a.cap_b, hist, tmp, sel_state);
    } else {
        select_row<false>(krow, ncand, kk, out, a.cap_b, hist, tmp, sel_state);
    }
}

template <typename T> hipError_t launch_t(BsArgs a, hipStream_t s) {
    const int64_t nb = (a.n + 63) / 64;
    hipLaunchKernelGGL(bs_pool_kernel<T>, dim3((unsigned)nb, (a.hq + a.hkv) * a.vl.nseq), dim3(kD), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = (size_t)min(nb, (int64_t)kBsLdsKeys) * sizeof(uint32_t);
    // query blocks in chunks of chunk_rows (a multiple of 64): scores of the
    // chunk into the workspace, then the selection of its rows
    for (int64_t r0 = 0; r0 < nb; r0 += a.chunk_rows) {
        a.row0 = r0;
        const int64_t rows = min((int64_t)a.chunk_rows, nb - r0);
        const unsigned kts = (unsigned)((r0 + rows + 63) / 64), qts = (unsigned)((rows + 63) / 64);
        hipLaunchKernelGGL(bs_score_kernel, dim3(kts, qts, a.hq * a.vl.nseq), dim3(kThreads), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(bs_select_kernel, dim3((unsigned)rows, a.hq * a.vl.nseq), dim3(kThreads), lds, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_estimate_bs(const BsArgs &a, int dtype, hipStream_t s) {
    return dtype == 0 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace msa
