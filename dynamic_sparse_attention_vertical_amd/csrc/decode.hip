// Decode-side dynamic sparsity for gfx950: one new query row per q head
// attends only to the top-k cached keys by attention score.
//
// The talk slides "System-Algorithm Co-design" (slide "Dynamic sparsity in
// attention", decoding panel) show that the keys a decode step needs change
// from step to step: choosing the top-1000 keys anew at each step keeps far
// more of the attention mass than a fixed choice.  The step here:
//   scores   s[h, j] = scale * <q_h, k_{g(h), j}> in log2 units, for every
//            cached key (K streamed once per kv head, shared by its q heads),
//            written as order-preserving 32-bit keys, with each chunk's
//            running max and sum of 2^s (the dense softmax denominator);
//   stats    the dense log-sum-exp of every q head from those partials;
//   select   exact top-k of the keys per head (ties to the lower index,
//            indices ascending; topk.hip: one workgroup per row when there are
//            many rows, else the sliced radix select), or a given set;
//   attend   softmax over the selected scores and the weighted sum of their V
//            rows; the retrieved share of the dense attention mass is
//            2^(lse_selected - lse_dense).
// Layout: q [hq, 128], K and V [hkv, stride, 128], out [hq, 128], one query
// per head (a batch of sequences is folded into the heads).  Caches may be
// shorter than the capacity n (a length per kv head): a position past a
// cache's length holds no key (score -inf), so no kernel reads its K or V
// row or a score for it: the dense sum and the top-k run over the positions
// before it, and a selection longer than the cache is completed with the
// lowest positions past its end, which get no weight.
#include "common.h"
#include "kernels.h"

#include <climits>
#include <type_traits>

namespace msa {
namespace {

constexpr int kD = 128;           // head_dim
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
constexpr int kThreads = 256;
constexpr int kMaxG = 8;          // q heads scored together per K pass
constexpr int kU = 8;             // rows per 16-lane group in flight

// float score -> 32-bit key that orders like the score (and back)
__device__ __forceinline__ uint32_t order_key(float s) {
    const uint32_t b = __float_as_uint(s);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t u) {
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
// keys in kv head g's cache (the capacity n unless lengths are given)
__device__ __forceinline__ int64_t cache_keys(const DecodeArgs &a, int g) {
    if (a.lens == nullptr) return a.n;
    const int64_t len = a.lens[g];
    return len < 0 ? 0 : (len > a.n ? a.n : len);
}

// 8 consecutive elements of a row as floats (16 lanes cover a 128-wide row)
template <typename T> __device__ __forceinline__ void load8(const T *p, float (&x)[8]);
template <> __device__ __forceinline__ void load8<bf16>(const bf16 *p, float (&x)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
template <> __device__ __forceinline__ void load8<float>(const float *p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = a[i];
        x[4 + i] = b[i];
    }
}

// Lane moves inside a row of 16 lanes (DPP, no LDS): the lane 15 - i of the
// row, the lane 7 - i of its half, and the lanes i ^ 2, i ^ 1 of its quad.
template <int kCtrl> __device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
constexpr int kDppRowMirror = 0x140, kDppHalfMirror = 0x141, kDppQuadXor2 = 0x4e, kDppQuadXor1 = 0xb1;

// The kG dot products of a 16-lane row group (one partial per lane each),
// reduce-scattered: at each step the lower and upper halves of a group of
// lanes pair up (mirror images), each keeps half of the heads and adds the
// partner's partials of them.  Afterwards lane pairs (kG = 8) or quads
// (kG = 4) hold one head's full sum each, head_of(lane).
template <int kG> __device__ __forceinline__ float reduce_scatter16(const float (&v)[kG], int lane);
template <> __device__ __forceinline__ float reduce_scatter16<4>(const float (&v)[4], int lane) {
    const bool u8 = (lane & 8) != 0, u4 = (lane & 4) != 0;
    const float k0 = (u8 ? v[2] : v[0]) + dpp<kDppRowMirror>(u8 ? v[0] : v[2]);
    const float k1 = (u8 ? v[3] : v[1]) + dpp<kDppRowMirror>(u8 ? v[1] : v[3]);
    float k = (u4 ? k1 : k0) + dpp<kDppHalfMirror>(u4 ? k0 : k1);
    k += dpp<kDppQuadXor2>(k);
    return k + dpp<kDppQuadXor1>(k);
}
template <> __device__ __forceinline__ float reduce_scatter16<8>(const float (&v)[8], int lane) {
    const bool u8 = (lane & 8) != 0, u4 = (lane & 4) != 0, u2 = (lane & 2) != 0;
    float k[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = (u8 ? v[i + 4] : v[i]) + dpp<kDppRowMirror>(u8 ? v[i] : v[i + 4]);
    const float m0 = (u4 ? k[2] : k[0]) + dpp<kDppHalfMirror>(u4 ? k[0] : k[2]);
    const float m1 = (u4 ? k[3] : k[1]) + dpp<kDppHalfMirror>(u4 ? k[1] : k[3]);
    const float r = (u2 ? m1 : m0) + dpp<kDppQuadXor2>(u2 ? m0 : m1);
    return r + dpp<kDppQuadXor1>(r);
}
template <int kG> __device__ __forceinline__ int head_of(int lane) {
    return kG == 8 ? ((lane >> 3) & 1) * 4 + ((lane >> 2) & 1) * 2 + ((lane >> 1) & 1)
                   : ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
}

// Grid (chunk, kv head): heads g0 .. g0 + gcount - 1 (gcount <= kG) of the kv
// head's group, keys [chunk * chunk_keys, ...).  A wave scores 4 keys at a
// time (16 lanes per key, 8 elements each, 2 kU keys per row group in flight
// for bf16); after the reduce-scatter each lane owns one head of its key and
// keeps that head's running max and sum.
template <typename T, int kG>
__global__ __launch_bounds__(kThreads) void decode_scores_kernel(DecodeArgs a, int g0) {
    const int kvh = blockIdx.y;
    const int G = a.hq / a.hkv;
    const int gcount = min(G - g0, kG);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = (lane & 15) * 8, sub = lane >> 4;
    const int hl = head_of<kG>(lane);                        // this lane's head after the reduction
    const bool owner = hl < gcount && (lane & (kG == 8 ? 1 : 3)) == 0;
    const int64_t j0 = (int64_t)blockIdx.x * a.chunk_keys;
    const int64_t j1 = min(j0 + a.chunk_keys, a.n);
    const int64_t jv = min(j1, max(j0, cache_keys(a, kvh)));   // keys [j0, jv) are in the cache
    if (jv == j0) {                                            // a chunk past the cache's end: an empty partial
        if (threadIdx.x < gcount) {
            const int64_t h = kvh * G + g0 + threadIdx.x;
            a.part[(h * a.nchunks + blockIdx.x) * 2 + 0] = -INFINITY;
            a.part[(h * a.nchunks + blockIdx.x) * 2 + 1] = 0.f;
        }
        return;
    }
    // bf16: q and K stay bf16 pairs, multiplied by v_dot2 (two products
    // summed into an fp32 accumulator); fp32: fused multiply-adds
    constexpr bool kPairs = sizeof(T) == 2;
    float qv[kG][8];
    bf16x2_t qp[kG][4];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
        const T *src = reinterpret_cast<const T *>(a.q) + (int64_t)(kvh * G + g0 + min(g, gcount - 1)) * kD + col;
        if constexpr (kPairs) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(src);
#pragma unroll
            for (int i = 0; i < 4; ++i) qp[g][i] = __builtin_bit_cast(bf16x2_t, g < gcount ? w[i] : 0u);
        } else {
            load8<T>(src, qv[g]);
            if (g >= gcount)
#pragma unroll
                for (int e = 0; e < 8; ++e) qv[g][e] = 0.f;
        }
    }
    const T *kp = reinterpret_cast<const T *>(a.k) + (int64_t)kvh * a.stride * kD;
    float m = -INFINITY, l = 0.f;
    constexpr int kUs = kPairs ? 2 * kU : kU;               // bf16 rows are half the registers
    // One step: the workgroup's 16 kUs consecutive keys from sb, rows sb +
    // 4 wave + sub + 16 u (u < kUs) in this 16-lane row group; all of them
    // inside the chunk and the cache (kFull: loads without conditions, so
    // that the compiler waits for each row's load alone), or some past the
    // end of either, which are neither read nor given a score key.  The
    // step's score keys are gathered in LDS and leave as 16-byte row stores.
    constexpr int kStep = 16 * kUs;
    __shared__ uint32_t skb[2][kG][kStep];
    int sbuf = 0;
    auto step = [&](int64_t sb, auto full) {
        uint32_t (&sk)[kG][kStep] = skb[sbuf];
        constexpr bool kFull = decltype(full)::value;
        const int64_t jb = sb + wave * 4 + sub;
        float kx[kUs][8];
        u32x4 kw[kUs];
#pragma unroll
        for (int u = 0; u < kUs; ++u) {
            const int64_t j = jb + 16 * u;
            if constexpr (kPairs) {
                // non-temporal: each K row is read once per pass (8% faster at 100K x 64 kv heads)
                kw[u] = (kFull || j < jv) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kp + j * kD + col))
                                          : u32x4{0u, 0u, 0u, 0u};
            } else if (kFull || j < jv) {
                load8<T>(kp + j * kD + col, kx[u]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) kx[u][e] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < kUs; ++u) {
            const int64_t j = jb + 16 * u;
            if (!kFull && j >= jv) break;
            float d[kG];
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                d[g] = 0.f;
                if constexpr (kPairs) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // the element into a scalar first: a bit cast of a
                        // vector element in place reads element 0
                        const uint32_t kpair = kw[u][i];
                        d[g] = __builtin_amdgcn_fdot2_f32_bf16(qp[g][i], __builtin_bit_cast(bf16x2_t, kpair), d[g],
                                                               false);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) d[g] = fmaf(qv[g][e], kx[u][e], d[g]);
                }
            }
            const float sc = reduce_scatter16<kG>(d, lane) * a.scale_log2;
            if (owner) {
                sk[hl][wave * 4 + sub + 16 * u] = order_key(sc);
                const float mn = fmaxf(m, sc);
                l = l * __builtin_amdgcn_exp2f(m - mn) + __builtin_amdgcn_exp2f(sc - mn);
                m = mn;
            }
        }
        __syncthreads();
        // the step's keys of every head: 16 bytes per thread and store
        const bool vec = (a.n & 3) == 0;                   // key rows start 16-byte aligned
        for (int c = threadIdx.x; c < gcount * (kStep / 4); c += kThreads) {
            const int hh = c / (kStep / 4), q4 = c % (kStep / 4);
            const int64_t key = sb + 4 * q4;
            uint32_t *dst = a.keys + (int64_t)(kvh * G + g0 + hh) * a.n + key;
            const uint32_t *srcw = &sk[hh][4 * q4];
            if (vec && (kFull || key + 3 < jv)) {
                *reinterpret_cast<u32x4 *>(dst) = u32x4{srcw[0], srcw[1], srcw[2], srcw[3]};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (key + e < jv) dst[e] = srcw[e];
            }
        }
        sbuf ^= 1;                                         // the next step fills the other buffer
    };
    for (int64_t sb = j0; sb < jv; sb += kStep) {
        if (sb + kStep <= jv)
            step(sb, std::true_type{});
        else
            step(sb, std::false_type{});
    }
    // the chunk's (max, sum) per head: owners of one head sit at the same
    // position in each row group; combine the 4 row groups, then the waves
    auto comb = [](float &mg, float &lg, float mo, float lo) {
        const float mn = fmaxf(mg, mo);
        lg = (mn == -INFINITY) ? 0.f : lg * __builtin_amdgcn_exp2f(mg - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
        mg = mn;
    };
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) comb(m, l, __shfl_xor(m, o, 64), __shfl_xor(l, o, 64));
    __shared__ float pm[4][kG], pl[4][kG];
    if (owner && lane < 16) {
        pm[wave][hl] = m;
        pl[wave][hl] = l;
    }
    __syncthreads();
    if (threadIdx.x < gcount) {
        const int g = threadIdx.x;
        float mg = -INFINITY, lg = 0.f;
        for (int w = 0; w < 4; ++w) comb(mg, lg, pm[w][g], pl[w][g]);
        const int64_t h = kvh * G + g0 + g;
        a.part[(h * a.nchunks + blockIdx.x) * 2 + 0] = mg;
        a.part[(h * a.nchunks + blockIdx.x) * 2 + 1] = lg;
    }
}

// Dense log2-sum-exp of each q head from its chunks' partials (one wave per head).
__global__ __launch_bounds__(64) void decode_stats_kernel(DecodeArgs a) {
    const int h = blockIdx.x, lane = threadIdx.x;
    float m = -INFINITY, l = 0.f;
    for (int c = lane; c < a.nchunks; c += 64) {
        const float mc = a.part[((int64_t)h * a.nchunks + c) * 2], lc = a.part[((int64_t)h * a.nchunks + c) * 2 + 1];
        const float mn = fmaxf(m, mc);
        l = (mn == -INFINITY) ? 0.f : l * __builtin_amdgcn_exp2f(m - mn) + lc * __builtin_amdgcn_exp2f(mc - mn);
        m = mn;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float mo = __shfl_xor(m, o, 64), lo = __shfl_xor(l, o, 64);
        const float mn = fmaxf(m, mo);
        l = (mn == -INFINITY) ? 0.f : l * __builtin_amdgcn_exp2f(m - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
        m = mn;
    }
    if (lane == 0) a.lse2_all[h] = l > 0.f ? m + __log2f(l) : -INFINITY;
}

// One workgroup per q head: softmax over the selected keys' scores and the
// weighted sum of their V rows (16 lanes per row, 64 row slots of kU rows per
// step: the gathers of one head spread over 16 waves).
constexpr int kAttThreads = 1024, kSlots = kAttThreads / 16;
template <typename T>
__global__ __launch_bounds__(kAttThreads) void decode_attend_kernel(DecodeArgs a) {
    const int h = blockIdx.x;
    const int G = a.hq / a.hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = (lane & 15) * 8, slot = wave * 4 + (lane >> 4);   // kSlots row slots
    const int32_t *idx = a.idx + (int64_t)h * a.topk;
    const uint32_t *keys = a.keys + (int64_t)h * a.n;
    const int64_t nv = cache_keys(a, h / G);   // selected positions at or past it hold no key: no score, no V
    __shared__ float red[kAttThreads / 64];
    // the selected scores' maximum
    float mx = -INFINITY;
    for (int t = threadIdx.x; t < a.topk; t += kAttThreads) {
        const int64_t j = min(max((int64_t)idx[t], (int64_t)0), a.n - 1);
        if (j < nv) mx = fmaxf(mx, key_score(keys[j]));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < kAttThreads / 64; ++w) mx = fmaxf(mx, red[w]);
    __syncthreads();
    const T *vp = reinterpret_cast<const T *>(a.v) + (int64_t)(h / G) * a.stride * kD;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    for (int tb = slot; tb < a.topk; tb += kSlots * kU) {
        // kU rows per slot per step, their loads issued together
        float vx[kU][8], p[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int t = tb + kSlots * u;
            p[u] = 0.f;
            const int64_t j = t < a.topk ? min(max((int64_t)idx[t], (int64_t)0), a.n - 1) : a.n;
            if (j < nv) {
                p[u] = __builtin_amdgcn_exp2f(key_score(keys[j]) - mx);
                load8<T>(vp + j * kD + col, vx[u]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) vx[u][e] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(p[u], vx[u][e], acc[e]);
            lsum += p[u];                             // the same p in all 16 lanes of the slot
        }
    }
    // sum the 16 slots: rows of each column slice in LDS, then one thread per column
    __shared__ float part[kSlots][kD];
    __shared__ float lpart[kSlots];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[slot][col + e] = acc[e];
    if ((lane & 15) == 0) lpart[slot] = lsum;
    __syncthreads();
    if (threadIdx.x < kD) {
        float o = 0.f, ls = 0.f;
        for (int r = 0; r < kSlots; ++r) {
            o += part[r][threadIdx.x];
            ls += lpart[r];
        }
        const float inv = ls > 0.f ? 1.f / ls : 0.f;
        T *op = reinterpret_cast<T *>(a.out) + (int64_t)h * kD + threadIdx.x;
        if constexpr (sizeof(T) == 2) {
            reinterpret_cast<uint16_t *>(op)[0] = f32_to_bf16(o * inv);
        } else {
            *reinterpret_cast<float *>(op) = o * inv;
        }
        if (threadIdx.x == 0) {
            const float lse2 = ls > 0.f ? mx + __log2f(ls) : -INFINITY;
            if (a.lse != nullptr) a.lse[h] = lse2 * kLn2;
            if (a.recovery != nullptr) {
                const float all = a.lse2_all[h];
                a.recovery[h] = (ls > 0.f && all != -INFINITY) ? __builtin_amdgcn_exp2f(lse2 - all) : 0.f;
            }
        }
    }
}

}  // namespace

template <typename T> void launch_scores_group(const DecodeArgs &a, int g0, int gcount, hipStream_t s) {
    const dim3 grid((unsigned)a.nchunks, (unsigned)a.hkv);
    if (gcount <= 4)
        hipLaunchKernelGGL((decode_scores_kernel<T, 4>), grid, dim3(kThreads), 0, s, a, g0);
    else
        hipLaunchKernelGGL((decode_scores_kernel<T, 8>), grid, dim3(kThreads), 0, s, a, g0);
}

hipError_t launch_decode_scores(const DecodeArgs &a, int dtype, hipStream_t s) {
    const int G = a.hq / a.hkv;
    for (int g0 = 0; g0 < G; g0 += kMaxG) {
        const int gcount = G - g0 < kMaxG ? G - g0 : kMaxG;
        if (dtype == 0)
            launch_scores_group<bf16>(a, g0, gcount, s);
        else
            launch_scores_group<float>(a, g0, gcount, s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(decode_stats_kernel, dim3((unsigned)a.hq), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode_attend(const DecodeArgs &a, int dtype, hipStream_t s) {
    if (dtype == 0)
        hipLaunchKernelGGL(decode_attend_kernel<bf16>, dim3((unsigned)a.hq), dim3(kAttThreads), 0, s, a);
    else
        hipLaunchKernelGGL(decode_attend_kernel<float>, dim3((unsigned)a.hq), dim3(kAttThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace msa
