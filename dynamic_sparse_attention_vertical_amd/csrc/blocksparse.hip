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
//   pool:   one workgroup per (head, block): 128 threads, one per dimension.
//   select: one workgroup per (q head, query block): scores into LDS as
//           order-preserving integer keys (32 lanes per key block, one
//           coalesced row read each), 4 x 8-bit radix select for the k-th
//           key (the bin found by a parallel scan), then an in-order
//           compaction (ties -> lower c).  Every workgroup reads all earlier
//           key-block means, so the scores are L2-bandwidth bound.
#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;

template <typename T>
__global__ __launch_bounds__(kD) void bs_pool_kernel(BsArgs a) {
    const int64_t nb = (a.n + 63) / 64;
    const int c = blockIdx.x;
    const int head = blockIdx.y;
    const int d = threadIdx.x;
    const T *src;
    float *dst;
    if (head < a.hq) {
        src = reinterpret_cast<const T *>(a.q) + (int64_t)head * a.stride * kD;
        dst = a.qm + ((int64_t)head * nb + c) * kD;
    } else {
        src = reinterpret_cast<const T *>(a.k) + (int64_t)(head - a.hq) * a.stride * kD;
        dst = a.km + ((int64_t)(head - a.hq) * nb + c) * kD;
    }
    // a short last block (length not a multiple of 64) is the mean of its rows
    const int nrows = (int)min((int64_t)64, a.n - (int64_t)c * 64);
    float acc = 0.f;
    for (int r = 0; r < nrows; ++r) {
        const T x = src[((int64_t)c * 64 + r) * kD + d];
        if constexpr (sizeof(T) == 2) acc += bf16_to_f32(x.x);
        else acc += x;
    }
    dst[d] = nrows == 64 ? acc * (1.f / 64.f) : acc / (float)nrows;
}

__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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

__global__ __launch_bounds__(kThreads) void bs_select_kernel(BsArgs a) {
    extern __shared__ uint32_t keys[];              // [b + 1]
    __shared__ alignas(16) float qrow[kD];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t tmp[kThreads];
    __shared__ uint32_t sel_state[2];
    const int64_t nb = (a.n + 63) / 64;
    const int64_t b = nb - 1 - blockIdx.x;          // heavy rows first
    const int h = blockIdx.y;
    const int G = a.hq / a.hkv;
    const int g = h / G;
    const int64_t item = (int64_t)h * nb + b;
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
    if (threadIdx.x < kD) qrow[threadIdx.x] = a.qm[item * kD + threadIdx.x];
    __syncthreads();
    // 32 lanes per candidate key block: lane s holds dimensions 4s .. 4s+3, so
    // each half-wave reads one 512-byte mean row in a single coalesced load,
    // and the 32 partial products are summed across the lanes
    const float *kmg = a.km + (int64_t)g * nb * kD;
    const int sub = threadIdx.x & 31, grp = threadIdx.x >> 5;
    const f32x4 qv = *reinterpret_cast<const f32x4 *>(&qrow[4 * sub]);
    for (int c = grp; c < ncand; c += kThreads / 32) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(kmg + (int64_t)c * kD + 4 * sub);
        float acc = qv[0] * x[0] + qv[1] * x[1] + qv[2] * x[2] + qv[3] * x[3];
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 32);
        if (sub == 0) keys[c] = order_key(acc * a.scale);
    }
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
            if (pos < (uint32_t)a.cap_b) out[pos] = c * 64;
            ++pos;
        }
    }
}

template <typename T> hipError_t launch_t(const BsArgs &a, hipStream_t s) {
    const int64_t nb = (a.n + 63) / 64;
    hipLaunchKernelGGL(bs_pool_kernel<T>, dim3((unsigned)nb, a.hq + a.hkv), dim3(kD), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = (size_t)nb * sizeof(uint32_t);
    hipLaunchKernelGGL(bs_select_kernel, dim3((unsigned)nb, a.hq), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_estimate_bs(const BsArgs &a, int dtype, hipStream_t s) {
    return dtype == 0 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace msa
