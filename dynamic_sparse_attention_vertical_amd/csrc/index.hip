// Work-list construction for vertical-slash heads, gfx950.
//
// One thread per (q head, 64-row query block b): rows r0 = 64b .. r1 = 64b+63.
// Each selected diagonal offset o <= r1 needs keys [max(0, r0-o), r1-o].
// Visiting those ranges by descending o (so ascending start), with cov the end
// of the last emitted block (initially 0): a range ending below cov is already
// covered; otherwise emit a 64-wide block at max(start, cov).  Once cov passes
// r1 every remaining range is covered, so the walk stops.  Then every selected
// column j <= r1 outside the emitted blocks is listed, ascending (merge walk:
// blocks and columns are both ascending).
//
// The pages ask that sparse work come in large contiguous blocks for the
// matrix units and that the index be built online at small cost ("How to
// optimise the TTFT of an 8B LLM with 1M tokens to 20 seconds", section on
// co-designing algorithm and system, principles 1-2); the covering rule is
// this library's reading of that.  The head's offsets and columns are staged
// in LDS, shared by the 256 query blocks of the workgroup.
#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kStageMax = 12288;     // int32 entries staged in LDS (48 KB)

template <bool kStaged>
__global__ __launch_bounds__(kThreads) void build_index_kernel(IndexArgs a) {
    __shared__ int32_t st_s[kStaged ? kStageMax : 1];
    const int h = blockIdx.y;
    const int64_t nqb = a.n / 64;
    const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int32_t *S = a.s_idx + (int64_t)h * a.ks;
    const int32_t *V = a.v_idx + (int64_t)h * a.kv;
    if constexpr (kStaged) {
        for (int i = threadIdx.x; i < a.ks; i += kThreads) st_s[i] = S[i];
        __syncthreads();
        S = st_s;
    }
    if (b >= nqb) return;
    const int64_t r0 = b * 64, r1 = r0 + 63;
    // number of offsets <= r1 (offsets ascending)
    int lo = 0, hi = a.ks;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)S[mid] <= r1) lo = mid + 1; else hi = mid;
    }
    const int64_t item = (int64_t)h * nqb + b;
    int32_t *blk = a.block_offset + item * a.cap_b;
    int64_t cov = 0;
    int cnt = 0;
    for (int i = lo - 1; i >= 0; --i) {
        const int64_t o = S[i];
        if (o < 0) continue;                       // out-of-range entries are ignored
        const int64_t e = r1 - o;
        if (e < cov) continue;
        const int64_t s0 = r0 - o;
        const int64_t st = s0 > cov ? s0 : cov;    // s0 may be negative: cov >= 0 covers it
        if (cnt < a.cap_b) blk[cnt] = (int32_t)st;
        ++cnt;
        cov = st + 64;
        if (cov > r1) break;
    }
    cnt = min(cnt, a.cap_b);
    a.block_count[item] = cnt;

    int32_t *col = a.column_index + item * a.cap_c;
    int p = 0, cc = 0;
    int64_t cur_end = cnt > 0 ? (int64_t)blk[0] + 63 : -1;
    for (int i = 0; i < a.kv; ++i) {
        const int64_t j = V[i];
        if (j > r1) break;
        if (j < 0) continue;
        while (p < cnt && cur_end < j) {
            ++p;
            cur_end = p < cnt ? (int64_t)blk[p] + 63 : -1;
        }
        if (p < cnt && (int64_t)blk[p] <= j) continue;   // inside block p
        if (cc < a.cap_c) col[cc] = (int32_t)j;
        ++cc;
    }
    a.column_count[item] = min(cc, a.cap_c);
}

}  // namespace

hipError_t launch_build_index(const IndexArgs &a, hipStream_t s) {
    const int64_t nqb = a.n / 64;
    dim3 grid((unsigned)((nqb + kThreads - 1) / kThreads), a.hq);
    if (a.ks <= kStageMax)
        hipLaunchKernelGGL(build_index_kernel<true>, grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(build_index_kernel<false>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace msa
