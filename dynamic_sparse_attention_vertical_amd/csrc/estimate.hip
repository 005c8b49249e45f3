// Online vertical-slash score estimation for gfx950.
//
// For q head h (kv head g) and the last 64 query rows p_r = N-64+r:
//   z[r, j] = scale <q_r, k_j> (j <= p_r),  P = row softmax of z,
//   v[j] = sum_r P[r, j],  s[o] = sum_r P[r, p_r - o].
// The pages leave the estimator unwritten beyond "approximate the sparse index
// online" ("MInference 1.0 README", "TL;DR"; talk slides "System-Algorithm
// Co-design", slide "MInference", online estimation of sparsity indices); this
// is the reading in which the last queries' softmax scores are summed per key
// column and per diagonal (the window-averaged column score of "Inf-MLLM: 4M-
// token long-sequence QA on a single 4090D", section 3.2, is v / 64).
//
// Work split: workgroup = (kv head g, contiguous key range), four waves, wave w
// serving q head g*G + w (+4, ...).  The K tile (64 keys) is staged in LDS
// once and shared by the G q heads of the group.  Scores are computed with
// MFMA as S^T = K Q^T (lane = one query row, 16 keys per 32-key sub-tile).
//   pass 1: per-row running max (kept as scale*log2(e)*z) and sum of exp2
//           over the range -> partials
//   combine: partials -> row max m_r and 1 / sum
//   pass 2: recompute S, p = exp(z - m_r) / l_r, written to a per-wave LDS
//           tile; column sums give v directly, diagonal sums are read along
//           diagonals of that tile.  A diagonal spans at most two adjacent
//           tiles; inside a range the carry is kept in a register, across
//           ranges the two partial sums go to the workspace and a fix-up
//           kernel adds them.  No floating-point atomics: results are
//           deterministic.
#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr int kD = 128;
constexpr int kL = 64;           // last_q
constexpr int kTK = 64;          // keys per tile
constexpr int kThreads = 256;    // four waves
constexpr int kPP = 65;          // per-wave P tile pitch (floats)

template <typename T> struct EstSmem {
    static constexpr int kEpv = 16 / Elem<T>::kBytes;
    static constexpr int kKPitch = kD + kEpv;
    T k[kTK * kKPitch];
};

template <typename T>
__device__ __forceinline__ void load_k_tile(T *ks, const T *kp, int64_t base, int tid) {
    constexpr int kEpv = EstSmem<T>::kEpv;
    constexpr int kKPitch = EstSmem<T>::kKPitch;
    constexpr int kVpr = kD / kEpv;
#pragma unroll
    for (int c = tid; c < kTK * kVpr; c += kThreads) {
        const int row = c / kVpr, cv = c % kVpr;
        u32x4 val = *reinterpret_cast<const u32x4 *>(kp + (base + row) * kD + cv * kEpv);
        *reinterpret_cast<u32x4 *>(&ks[row * kKPitch + cv * kEpv]) = val;
    }
}

// S^T for 32 query rows (half) against the 64-key tile: s[kt][jj*4+i] is
// the score of key kt*32 + jj*8 + hl*4 + i for query row half*32 + lane%32.
template <typename T>
__device__ __forceinline__ void tile_scores(f32x16 (&s)[2], const T *ks, const typename Elem<T>::frag *qf,
                                            int l32, int hl) {
    using E = Elem<T>;
    constexpr int kKPitch = EstSmem<T>::kKPitch;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) {
            typename E::frag kf = E::load_frag(&ks[(kt * 32 + l32) * kKPitch + dk * 16 + hl * 8]);
            E::mma(s[kt], kf, qf[dk]);
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void est_pass1_kernel(EstArgs a) {
    using E = Elem<T>;
    __shared__ EstSmem<T> sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
    const int range = blockIdx.x, g = blockIdx.y;
    const int G = a.hq / a.hkv;
    const int64_t n = a.n;
    const int64_t k0 = (int64_t)range * a.range_keys;
    const int64_t k1 = min(n, k0 + a.range_keys);
    const T *kp = reinterpret_cast<const T *>(a.k) + (int64_t)g * n * kD;
    const int nslot = (G + 3) / 4;
    for (int slot = 0; slot < nslot; ++slot) {
        const int hw = wave + 4 * slot;
        const bool active = hw < G;
        const int h = g * G + (active ? hw : 0);
        const T *qp = reinterpret_cast<const T *>(a.q) + ((int64_t)h * n + (n - kL)) * kD;
        typename E::frag qf[2][8];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int dk = 0; dk < 8; ++dk)
                qf[half][dk] = active ? E::load_frag(qp + (half * 32 + l32) * kD + dk * 16 + hl * 8)
                                      : E::zero_frag();
        float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
        for (int64_t base = k0; base < k1; base += kTK) {
            __syncthreads();
            load_k_tile<T>(sm.k, kp, base, tid);
            __syncthreads();
            if (!active) continue;
            const bool last = base + kTK > n - kL;       // keys past some p_r
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x16 s[2];
                tile_scores<T>(s, sm.k, qf[half], l32, hl);
                const int64_t prow = n - kL + half * 32 + l32;
                if (last) {
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int64_t key = base + kt * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
                            if (key > prow) s[kt][i] = -INFINITY;
                        }
                }
                float mx = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
                // running max in scaled log2 units (stored value: an unchanged
                // max rescales by exactly 1)
                const float mn = fmaxf(m[half], mx * a.scale_log2);
                const float ref = (mn == -INFINITY) ? 0.f : mn;
                float acc = l[half] * exp2f(m[half] - ref);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc += exp2f(fmaf(s[kt][i], a.scale_log2, -ref));
                m[half] = mn;
                l[half] = acc;
            }
        }
        if (active) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const float mo = wave_shfl_xor(m[half], 32), lo = wave_shfl_xor(l[half], 32);
                const float mn = fmaxf(m[half], mo);
                const float ref = (mn == -INFINITY) ? 0.f : mn;
                const float lt = l[half] * exp2f(m[half] - ref) + lo * exp2f(mo - ref);
                if (hl == 0) {
                    const int64_t o = ((int64_t)h * kL + half * 32 + l32) * a.nranges + range;
                    a.part_m[o] = mn;
                    a.part_l[o] = lt;
                }
            }
        }
    }
}

// One wave per (q head, row): merge the per-range (max, sum) partials.
__global__ __launch_bounds__(256) void est_combine_kernel(EstArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (int64_t)a.hq * kL) return;
    const float *pm = a.part_m + row * a.nranges;
    const float *pl = a.part_l + row * a.nranges;
    float m = -INFINITY, l = 0.f;
    for (int i = lane; i < a.nranges; i += 64) {
        const float mi = pm[i], li = pl[i];
        const float mn = fmaxf(m, mi);
        const float base = (mn == -INFINITY) ? 0.f : mn;
        l = l * exp2f(m - base) + li * exp2f(mi - base);
        m = mn;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float mo = wave_shfl_xor(m, off), lo = wave_shfl_xor(l, off);
        const float mn = fmaxf(m, mo);
        const float base = (mn == -INFINITY) ? 0.f : mn;
        l = l * exp2f(m - base) + lo * exp2f(mo - base);
        m = mn;
    }
    if (lane == 0) {
        a.row_m[row] = m;
        a.row_il[row] = l > 0.f ? 1.f / l : 0.f;
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void est_pass2_kernel(EstArgs a) {
    using E = Elem<T>;
    __shared__ EstSmem<T> sm;
    __shared__ float pbuf[4][32 * kPP];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
    const int range = blockIdx.x, g = blockIdx.y;
    const int G = a.hq / a.hkv;
    const int64_t n = a.n;
    const int64_t k0 = (int64_t)range * a.range_keys;
    const int64_t k1 = min(n, k0 + a.range_keys);
    const T *kp = reinterpret_cast<const T *>(a.k) + (int64_t)g * n * kD;
    float *pw = pbuf[wave];
    const int nslot = (G + 3) / 4;
    for (int slot = 0; slot < nslot; ++slot) {
        const int hw = wave + 4 * slot;
        const bool active = hw < G;
        const int h = g * G + (active ? hw : 0);
        const T *qp = reinterpret_cast<const T *>(a.q) + ((int64_t)h * n + (n - kL)) * kD;
        typename E::frag qf[2][8];
        float mrow[2], il[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int dk = 0; dk < 8; ++dk)
                qf[half][dk] = active ? E::load_frag(qp + (half * 32 + l32) * kD + dk * 16 + hl * 8)
                                      : E::zero_frag();
            const int64_t ri = (int64_t)h * kL + half * 32 + l32;
            mrow[half] = active ? a.row_m[ri] : 0.f;          // scaled log2 units
            il[half] = active ? a.row_il[ri] : 0.f;
        }
        float *vout = a.v_score + (int64_t)h * n;
        float *sout = a.s_score + (int64_t)h * n;
        float carry = 0.f;
        bool first = true;
        for (int64_t base = k0; base < k1; base += kTK) {
            __syncthreads();
            load_k_tile<T>(sm.k, kp, base, tid);
            __syncthreads();
            const bool last = base + kTK > n - kL;
            float col = 0.f, dg1 = 0.f, dg2 = 0.f;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                if (active) {
                    f32x16 s[2];
                    tile_scores<T>(s, sm.k, qf[half], l32, hl);
                    const int64_t prow = n - kL + half * 32 + l32;
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int e = kt * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
                            float p = exp2f(fmaf(s[kt][i], a.scale_log2, -mrow[half])) * il[half];
                            if (last && base + e > prow) p = 0.f;
                            pw[l32 * kPP + e] = p;
                        }
                }
                __syncthreads();
                if (active) {
                    // rows R = half*32 + r of the head's 64; diagonal d = R - e
#pragma unroll 8
                    for (int r = 0; r < 32; ++r) {
                        col += pw[r * kPP + lane];
                        const int e1 = half * 32 + r + 63 - lane;   // d = lane - 63
                        if (e1 >= 0 && e1 < kTK) dg1 += pw[r * kPP + e1];
                        const int e2 = half * 32 + r - lane - 1;    // d = lane + 1
                        if (e2 >= 0 && e2 < kTK) dg2 += pw[r * kPP + e2];
                    }
                }
                __syncthreads();
            }
            if (active) {
                vout[base + lane] = col;
                const int64_t A = n - kL - base;                 // offset of diagonal d = 0
                if (lane == 63) {
                    sout[A] = dg1;                               // d = 0 lies in this tile only
                } else {
                    const int64_t o2 = A + lane + 1;             // d = lane + 1
                    if (!first) {
                        sout[o2] = dg2 + carry;
                    } else if (range == 0) {
                        sout[o2] = dg2;                          // keys below 0 do not exist
                    } else {
                        a.diag_hi[((int64_t)h * a.nranges + range) * 64 + lane] = dg2;
                    }
                    carry = dg1;                                 // d = lane - 63, finished by the next tile
                }
            }
            first = false;
        }
        if (active && lane < 63 && range != a.nranges - 1)
            a.diag_lo[((int64_t)h * a.nranges + range) * 64 + lane] = carry;
    }
}

// Diagonals that straddle two key ranges: s[o] = hi(range) + lo(range - 1).
__global__ __launch_bounds__(256) void est_fixup_kernel(EstArgs a) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_h = (int64_t)(a.nranges - 1) * 63;
    if (t >= per_h * a.hq) return;
    const int h = (int)(t / per_h);
    const int64_t rem = t % per_h;
    const int range = 1 + (int)(rem / 63);
    const int lane = (int)(rem % 63);
    const int64_t A = a.n - kL - (int64_t)range * a.range_keys;
    const int64_t o = A + lane + 1;
    a.s_score[(int64_t)h * a.n + o] = a.diag_hi[((int64_t)h * a.nranges + range) * 64 + lane] +
                                      a.diag_lo[((int64_t)h * a.nranges + range - 1) * 64 + lane];
}

template <typename T> hipError_t launch_t(const EstArgs &a, hipStream_t s) {
    dim3 grid(a.nranges, a.hkv);
    hipLaunchKernelGGL(est_pass1_kernel<T>, grid, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)a.hq * kL;
    hipLaunchKernelGGL(est_combine_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(est_pass2_kernel<T>, grid, dim3(kThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t fix = (int64_t)(a.nranges - 1) * 63 * a.hq;
    if (fix > 0) {
        hipLaunchKernelGGL(est_fixup_kernel, dim3((unsigned)((fix + 255) / 256)), dim3(256), 0, s, a);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

hipError_t launch_estimate_scores(const EstArgs &a, int dtype, hipStream_t s) {
    return dtype == 0 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace msa
