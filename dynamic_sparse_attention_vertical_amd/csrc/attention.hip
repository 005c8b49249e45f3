// Sparse and dense causal prefill attention for gfx950.
//
// One workgroup = one (q head, 64-row query block) work item, two waves of 32
// query rows each.  The work item walks a list of 64-key tiles: for the sparse
// kernel, first the item's 64-wide key blocks (arbitrary start), then its
// leftover vertical columns gathered 64 at a time; for the dense kernel, the
// aligned tiles 0..b.  Per tile:
//   S^T = K Q^T        (MFMA 32x32x16 bf16; K tile from LDS, Q in registers)
//   online softmax in fp32 (exp2 with the log2(e)-folded scale)
//   O^T += V^T P^T     (P stays in registers as the B operand; V^T from LDS)
// Computing S transposed leaves each lane holding one query's scores for 16
// keys, so a row max needs only one cross-lane exchange (lane l with l^32), and
// those scores already sit in the B-operand layout of the PV product up to a
// fixed key permutation, which the V^T tile is written in.
//
// The pages: causal attention computed only over the selected entries, in
// FlashAttention style (talk slides "System-Algorithm Co-design", slide
// "MInference": dynamic sparse attention calculation with PIT and
// FlashAttention); sparse work in large blocks for the matrix units ("How to
// optimise the TTFT of an 8B LLM with 1M tokens to 20 seconds", section on
// co-designing algorithm and system, principle 1).
#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr int kD = 128;          // head_dim
constexpr int kBQ = 64;          // query rows per work item
constexpr int kBK = 64;          // keys per tile
constexpr int kThreads = 128;    // two waves

template <typename T> struct AttnTile {
    static constexpr int kEpv = 16 / Elem<T>::kBytes;        // elements per 16-byte vector
    static constexpr int kKPitch = kD + kEpv;                 // K row pitch (+16 B, no bank conflicts)
    T k[kBK * kKPitch];
    T vt[kD * kBK];                                           // V^T, chunk-swizzled rows
    int32_t kidx[kBK];
};

// Position of tile key e in the V^T row: inside each group of 16 keys the two
// middle quads are swapped, matching where the S^T accumulator keeps them.
__device__ __forceinline__ int vt_pos(int e) {
    int q = (e >> 2) & 3;
    int qn = (q == 1) ? 2 : (q == 2 ? 1 : q);
    return (e & ~15) | (qn << 2) | (e & 3);
}

// 8-element chunk swizzle of V^T row d (conflict-free reads and writes).
__device__ __forceinline__ int vt_swz(int d) { return (d & 7) ^ ((d >> 3) & 7); }

__device__ __forceinline__ int64_t item_of_block(int64_t bid, int64_t total) {
    // Consecutive workgroup ids land on different XCDs; give each XCD a
    // contiguous run of work items (kv-group major) so one XCD's L2 serves the
    // q heads that share K/V.
    if (total % kNumXcd == 0) return (bid % kNumXcd) * (total / kNumXcd) + bid / kNumXcd;
    return bid;
}

template <typename T> struct Store;
template <> struct Store<bf16> {
    __device__ static __forceinline__ void four(bf16 *dst, float a, float b, float c, float d) {
        u32x2 w;
        w[0] = pack_bf16x2(a, b);
        w[1] = pack_bf16x2(c, d);
        *reinterpret_cast<u32x2 *>(dst) = w;
    }
};
template <> struct Store<float> {
    __device__ static __forceinline__ void four(float *dst, float a, float b, float c, float d) {
        f32x4 w = {a, b, c, d};
        *reinterpret_cast<f32x4 *>(dst) = w;
    }
};

// V tile: 16 key quads x 16 d-octets; each task loads 4 rows x 8 elements and
// writes them transposed (8 rows of V^T x 4 keys).
template <typename T>
__device__ __forceinline__ void load_v_task(AttnTile<T> &sm, const T *vbase, int64_t n, int task,
                                            bool is_col, int64_t base) {
    const int kq = task >> 4, d8 = task & 15;
    float x[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int e = kq * 4 + r;
        const int64_t key = is_col ? (int64_t)sm.kidx[e] : base + e;
        if (key >= 0 && key < n) {
            const T *src = vbase + key * kD + d8 * 8;
            if constexpr (sizeof(T) == 2) {
                u32x4 w = *reinterpret_cast<const u32x4 *>(src);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    x[r][2 * c] = __uint_as_float(w[c] << 16);
                    x[r][2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u);
                }
            } else {
                f32x4 a = *reinterpret_cast<const f32x4 *>(src);
                f32x4 b = *reinterpret_cast<const f32x4 *>(src + 4);
#pragma unroll
                for (int c = 0; c < 4; ++c) { x[r][c] = a[c]; x[r][4 + c] = b[c]; }
            }
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) x[r][c] = 0.f;
        }
    }
    const int p = vt_pos(kq * 4);                 // multiple of 4
    const int chunk = p >> 3, within = p & 7;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
        const int d = d8 * 8 + dd;
        T *dst = &sm.vt[d * kBK + ((chunk ^ vt_swz(d)) << 3) + within];
        Store<T>::four(dst, x[0][dd], x[1][dd], x[2][dd], x[3][dd]);
    }
}

template <typename T, bool kDense>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(AttnArgs a) {
    using E = Elem<T>;
    using frag = typename E::frag;
    constexpr int kEpv = AttnTile<T>::kEpv;
    constexpr int kKPitch = AttnTile<T>::kKPitch;
    __shared__ AttnTile<T> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
    const int64_t n = a.n;
    const int64_t nqb = n / kBQ;
    const int G = a.hq / a.hkv;
    const int64_t total = (int64_t)a.hq * nqb;
    const int64_t t = item_of_block(blockIdx.x, total);
    const int64_t per_g = (int64_t)G * nqb;
    const int g = (int)(t / per_g);
    const int64_t rem = t % per_g;
    const int64_t b = nqb - 1 - rem / G;           // heavy (late) query blocks first
    const int h = g * G + (int)(rem % G);
    const int64_t r0 = b * kBQ;
    const int64_t qrow = r0 + wave * 32 + l32;

    const T *qp = reinterpret_cast<const T *>(a.q) + ((int64_t)h * n) * kD;
    const T *kp = reinterpret_cast<const T *>(a.k) + ((int64_t)g * n) * kD;
    const T *vp = reinterpret_cast<const T *>(a.v) + ((int64_t)g * n) * kD;

    int nblk, ncol;
    const int32_t *blist = nullptr, *clist = nullptr;
    if constexpr (kDense) {
        nblk = (int)b + 1;
        ncol = 0;
    } else {
        const int64_t item = (int64_t)h * nqb + b;
        nblk = min(max(a.block_count[item], 0), a.cap_b);
        ncol = min(max(a.column_count[item], 0), a.cap_c);
        blist = a.block_offset + item * a.cap_b;
        clist = a.column_index + item * a.cap_c;
    }
    const int nchunk = (ncol + kBK - 1) / kBK;

    // Q fragments (B operand of S^T = K Q^T): query qrow, d = dk*16 + hl*8 + e
    frag qf[8];
#pragma unroll
    for (int dk = 0; dk < 8; ++dk) qf[dk] = E::load_frag(qp + qrow * kD + dk * 16 + hl * 8);

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    // running row max kept in scaled log2 units as a stored fp32 value, so an
    // unchanged max gives a rescale factor of exactly 1
    float mb_i = -INFINITY, l_i = 0.f;

    for (int it = 0; it < nblk + nchunk; ++it) {
        const bool is_col = it >= nblk;
        int64_t base = 0;
        int c0 = 0;
        if (!is_col) {
            base = kDense ? (int64_t)it * kBK : (int64_t)blist[it];
        } else {
            c0 = (it - nblk) * kBK;
        }
        __syncthreads();                               // previous tile fully consumed
        if (is_col) {
            if (tid < kBK) sm.kidx[tid] = (c0 + tid < ncol) ? clist[c0 + tid] : -1;
            __syncthreads();
        }
        // K tile, row-major with a 16-byte pad per row
        constexpr int kVpr = kD / kEpv;                // 16-byte vectors per row
#pragma unroll
        for (int c = tid; c < kBK * kVpr; c += kThreads) {
            const int row = c / kVpr, cv = c % kVpr;
            const int64_t key = is_col ? (int64_t)sm.kidx[row] : base + row;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (key >= 0 && key < n) val = *reinterpret_cast<const u32x4 *>(kp + key * kD + cv * kEpv);
            *reinterpret_cast<u32x4 *>(&sm.k[row * kKPitch + cv * kEpv]) = val;
        }
#pragma unroll
        for (int task = tid; task < 256; task += kThreads) load_v_task<T>(sm, vp, n, task, is_col, base);
        __syncthreads();

        // S^T for this wave's 32 queries: two 32-key sub-tiles
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
            for (int dk = 0; dk < 8; ++dk) {
                frag kf = E::load_frag(&sm.k[(kt * 32 + l32) * kKPitch + dk * 16 + hl * 8]);
                E::mma(s[kt], kf, qf[dk]);
            }
        }

        // mask: key must exist and satisfy j <= i
        const bool need_mask = is_col || (base + kBK - 1 > r0) || base < 0;
        if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = kt * 32 + jj * 8 + hl * 4 + i;
                        const int64_t key = is_col ? (int64_t)sm.kidx[e] : base + e;
                        if (!(key >= 0 && key <= qrow)) s[kt][jj * 4 + i] = -INFINITY;
                    }
        }

        // online softmax: p = 2^(s*c - mb), c = scale*log2(e)
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
        mx = fmaxf(mx, wave_shfl_xor(mx, 32));
        const float mb_new = fmaxf(mb_i, mx * a.scale_log2);
        const float ref = (mb_new == -INFINITY) ? 0.f : mb_new;
        const float alpha = exp2f(mb_i - ref);
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = exp2f(fmaf(s[kt][i], a.scale_log2, -ref));
                s[kt][i] = p;
                rs += p;
            }
        l_i = l_i * alpha + rs;
        mb_i = mb_new;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;

        // P fragments: k-step kk uses accumulator s[kk/2], elements 8*(kk%2)..+7
        frag pf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float tmp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) tmp[e] = s[kk >> 1][8 * (kk & 1) + e];
            pf[kk] = E::from_f32(tmp);
        }
        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int d = dt * 32 + l32;
            const int sw = vt_swz(d);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                frag vf = E::load_frag(&sm.vt[d * kBK + (((kk * 2 + hl) ^ sw) << 3)]);
                E::mma(o[dt], vf, pf[kk]);
            }
        }
    }

    // finalise: lanes l and l^32 hold halves of the same row's sum
    const float l_tot = l_i + wave_shfl_xor(l_i, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T *op = reinterpret_cast<T *>(a.out) + ((int64_t)h * n + qrow) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int d0 = dt * 32 + jj * 8 + hl * 4;
            Store<T>::four(op + d0, o[dt][jj * 4 + 0] * inv, o[dt][jj * 4 + 1] * inv,
                           o[dt][jj * 4 + 2] * inv, o[dt][jj * 4 + 3] * inv);
        }
    if (a.lse != nullptr && hl == 0)
        a.lse[(int64_t)h * n + qrow] = l_tot > 0.f ? (mb_i * kLn2 + logf(l_tot)) : -INFINITY;
}

template <typename T, bool kDense> hipError_t launch(const AttnArgs &a, hipStream_t s) {
    const int64_t total = (int64_t)a.hq * (a.n / kBQ);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL((attn_fwd_kernel<T, kDense>), dim3((unsigned)total), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_prefill(const AttnArgs &a, int dtype, hipStream_t s) {
    return dtype == 0 ? launch<bf16, false>(a, s) : launch<float, false>(a, s);
}

hipError_t launch_dense_prefill(const AttnArgs &a, int dtype, hipStream_t s) {
    return dtype == 0 ? launch<bf16, true>(a, s) : launch<float, true>(a, s);
}

}  // namespace msa
