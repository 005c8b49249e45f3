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
// Tiles are double-buffered in LDS.  bf16: while a tile is being computed,
// the next tile's K and V rows are already in flight from HBM into registers;
// after the compute they are written (V transposed) to the other stage.  fp32
// (a checking path) loads after the compute.  One barrier per tile.
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

template <typename T> struct AttnStage {
    static constexpr int kEpv = 16 / Elem<T>::kBytes;        // elements per 16-byte vector
    static constexpr int kKPitch = kD + kEpv;                 // K row pitch (+16 B: conflict-free reads)
    T k[kBK * kKPitch];
    T vt[kD * kBK];                                           // V^T, chunk-swizzled rows
    int32_t kidx[kBK];                                        // key of each tile row (-1: none)
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

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> struct Out;
template <> struct Out<bf16> {
    __device__ static __forceinline__ void four(bf16 *dst, float a, float b, float c, float d) {
        u32x2 w;
        w[0] = pk_bf16(a, b);
        w[1] = pk_bf16(c, d);
        *reinterpret_cast<u32x2 *>(dst) = w;
    }
    __device__ static __forceinline__ bf16x8 frag(const float *x) {
        u32x4 r;
        r[0] = pk_bf16(x[0], x[1]);
        r[1] = pk_bf16(x[2], x[3]);
        r[2] = pk_bf16(x[4], x[5]);
        r[3] = pk_bf16(x[6], x[7]);
        return __builtin_bit_cast(bf16x8, r);
    }
};
template <> struct Out<float> {
    __device__ static __forceinline__ void four(float *dst, float a, float b, float c, float d) {
        f32x4 w = {a, b, c, d};
        *reinterpret_cast<f32x4 *>(dst) = w;
    }
    __device__ static __forceinline__ f32x8 frag(const float *x) { return Elem<float>::from_f32(x); }
};

// Where a tile's keys come from: 64 consecutive keys from `base`, or 64
// entries of a column list starting at `c0` (entries past `ncol` are empty).
struct TileSrc {
    bool is_col;
    int64_t base;
    int c0;
};

// Global -> registers -> LDS staging of one K/V tile.  Thread t moves K rows
// (t>>4) + 8i (16-byte column t&15) and V key quads (t>>4) + 8j (d-octet t&15).
template <typename T> struct Loader {
    static constexpr int kEpv = AttnStage<T>::kEpv;
    static constexpr int kVpr = kD / kEpv;                        // 16-byte vectors per row
    static constexpr int kKVec = kBK * kVpr / kThreads;            // K vectors per thread
    static constexpr int kVVec = 8 * Elem<T>::kBytes / 16;         // 16-byte vectors per V row piece
    u32x4 kr[kKVec];
    u32x4 vr[2][4][kVVec];
    int32_t key_lo;                                                // key of tile row tid (tid < 64)

    __device__ __forceinline__ static int64_t key_of(const TileSrc &s, int row, const int32_t *clist,
                                                     int ncol) {
        if (!s.is_col) return s.base + row;
        const int c = s.c0 + row;
        return c < ncol ? (int64_t)clist[c] : -1;
    }

    __device__ __forceinline__ void issue(const TileSrc &s, const T *kp, const T *vp, int64_t n,
                                          const int32_t *clist, int ncol, int tid) {
        const int col = tid & 15;
#pragma unroll
        for (int i = 0; i < kKVec; ++i) {
            const int v = tid + kThreads * i;
            const int row = v / kVpr, cv = v % kVpr;
            const int64_t key = key_of(s, row, clist, ncol);
            u32x4 z = {0u, 0u, 0u, 0u};
            kr[i] = (key >= 0 && key < n) ? *reinterpret_cast<const u32x4 *>(kp + key * kD + cv * kEpv) : z;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kq = (tid >> 4) + 8 * j;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t key = key_of(s, kq * 4 + r, clist, ncol);
                const bool ok = key >= 0 && key < n;
#pragma unroll
                for (int c = 0; c < kVVec; ++c) {
                    u32x4 z = {0u, 0u, 0u, 0u};
                    vr[j][r][c] = ok ? *reinterpret_cast<const u32x4 *>(vp + key * kD + col * 8 + c * kEpv) : z;
                }
            }
        }
        if (tid < kBK) key_lo = (int32_t)key_of(s, tid, clist, ncol);
    }

    __device__ __forceinline__ void commit(AttnStage<T> &st, int tid) {
        const int col = tid & 15;
#pragma unroll
        for (int i = 0; i < kKVec; ++i) {
            const int v = tid + kThreads * i;
            const int row = v / kVpr, cv = v % kVpr;
            *reinterpret_cast<u32x4 *>(&st.k[row * AttnStage<T>::kKPitch + cv * kEpv]) = kr[i];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kq = (tid >> 4) + 8 * j;
            const int p = vt_pos(kq * 4);                             // multiple of 4
            const int chunk = p >> 3, within = p & 7;
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                const int d = col * 8 + dd;
                T *dst = &st.vt[d * kBK + ((chunk ^ vt_swz(d)) << 3) + within];
                if constexpr (sizeof(T) == 2) {
                    // element dd of each of the 4 rows: 16-bit half (dd&1) of word dd>>1
                    const int w = dd >> 1;
                    const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
                    u32x2 out;
                    out[0] = __builtin_amdgcn_perm(vr[j][1][0][w], vr[j][0][0][w], sel);
                    out[1] = __builtin_amdgcn_perm(vr[j][3][0][w], vr[j][2][0][w], sel);
                    *reinterpret_cast<u32x2 *>(dst) = out;
                } else {
                    const int c = dd >> 2, w = dd & 3;
                    u32x4 out;
                    out[0] = vr[j][0][c][w];
                    out[1] = vr[j][1][c][w];
                    out[2] = vr[j][2][c][w];
                    out[3] = vr[j][3][c][w];
                    *reinterpret_cast<u32x4 *>(dst) = out;
                }
            }
        }
        if (tid < kBK) st.kidx[tid] = key_lo;
    }
};

template <typename T, bool kDense>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(AttnArgs a) {
    using E = Elem<T>;
    using frag = typename E::frag;
    constexpr int kKPitch = AttnStage<T>::kKPitch;
    constexpr bool kPipe = sizeof(T) == 2;    // prefetch the next tile into registers during compute
    // Two LDS stages (68 KB for bf16: two workgroups, one wave per SIMD).  A
    // single 34 KB stage would allow two waves per SIMD, but then the register
    // prefetch no longer fits in 256 registers and spills; measured slower.
    constexpr int kStages = 2;
    __shared__ AttnStage<T> stage[kStages];

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
    const int ntile = nblk + (ncol + kBK - 1) / kBK;

    auto src_of = [&](int it) {
        TileSrc s;
        s.is_col = it >= nblk;
        s.base = s.is_col ? 0 : (kDense ? (int64_t)it * kBK : (int64_t)blist[it]);
        s.c0 = s.is_col ? (it - nblk) * kBK : 0;
        return s;
    };

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

    Loader<T> ld;
    if (ntile > 0) {
        ld.issue(src_of(0), kp, vp, n, clist, ncol, tid);
        ld.commit(stage[0], tid);
    }
    __syncthreads();

    for (int it = 0; it < ntile; ++it) {
        const TileSrc cur = src_of(it);
        const bool more = it + 1 < ntile;
        if (kPipe && more) ld.issue(src_of(it + 1), kp, vp, n, clist, ncol, tid);
        const AttnStage<T> &st = stage[it % kStages];

        // S^T for this wave's 32 queries: two 32-key sub-tiles
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
            for (int dk = 0; dk < 8; ++dk) {
                frag kf = E::load_frag(&st.k[(kt * 32 + l32) * kKPitch + dk * 16 + hl * 8]);
                E::mma(s[kt], kf, qf[dk]);
            }
        }

        // mask: the key must exist and satisfy j <= i
        const bool need_mask = cur.is_col || (cur.base + kBK - 1 > r0) || cur.base < 0;
        if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = kt * 32 + jj * 8 + hl * 4 + i;
                        const int64_t key = cur.is_col ? (int64_t)st.kidx[e] : cur.base + e;
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
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][i], a.scale_log2, -ref));
                s[kt][i] = p;
                rs += p;
            }
        // rescale only when some row's max moved (alpha is exactly 1 otherwise)
        if (__builtin_amdgcn_ballot_w64(mb_new != mb_i) != 0) {
            const float alpha = __builtin_amdgcn_exp2f(mb_i - ref);
            l_i *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
        }
        l_i += rs;
        mb_i = mb_new;

        // P fragments: k-step kk uses accumulator s[kk/2], elements 8*(kk%2)..+7
        frag pf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float tmp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) tmp[e] = s[kk >> 1][8 * (kk & 1) + e];
            pf[kk] = Out<T>::frag(tmp);
        }
        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int d = dt * 32 + l32;
            const int sw = vt_swz(d);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                frag vf = E::load_frag(&st.vt[d * kBK + (((kk * 2 + hl) ^ sw) << 3)]);
                E::mma(o[dt], vf, pf[kk]);
            }
        }

        if (more) {
            if (!kPipe) ld.issue(src_of(it + 1), kp, vp, n, clist, ncol, tid);
            ld.commit(stage[(it + 1) % kStages], tid);
        }
        __syncthreads();
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
            Out<T>::four(op + d0, o[dt][jj * 4 + 0] * inv, o[dt][jj * 4 + 1] * inv,
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
