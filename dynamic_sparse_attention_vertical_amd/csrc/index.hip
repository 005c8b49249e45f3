// Work-list construction for vertical-slash heads, gfx950.
//
// One lane per (q head, 64-row query block b): rows r0 = 64b .. r1 = 64b+63.
// Each selected diagonal offset o <= r1 needs keys [max(0, r0-o), r1-o].
// Visiting those ranges by descending o (so ascending start), with cov the end
// of the last emitted block (initially 0): a range ending below cov is already
// covered; otherwise emit a 64-wide block at max(start, cov).  Once cov passes
// r1 every remaining range is covered.  Every selected column j <= r1 outside
// the emitted blocks is listed too, ascending.
//
// The offsets of a head are the same for every lane, so a wave walks them in
// lock step (scalar loads, sixteen at a time, one group ahead) and each lane
// applies the step to its own cover.  Columns are merged into the same walk:
// when a block starts at st, the columns in [cov, st) are exactly the ones no
// block covers.  A lane keeps its next column in a register, so a step that
// passes no column does no memory access: nearly every step has some lane of
// the wave emitting a block, and at about one wave per SIMD a load latency per
// step would set the pace.
//
// The pages ask that sparse work come in large contiguous blocks for the
// matrix units and that the index be built online at small cost ("How to
// optimise the TTFT of an 8B LLM with 1M tokens to 20 seconds", section on
// co-designing algorithm and system, principles 1-2); the covering rule is
// this library's reading of that.
#include "common.h"
#include "kernels.h"

#include <climits>

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kStageMax = 4096;      // columns staged in LDS (16 KB)

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// Scalar loads of the offsets.  The address goes through readfirstlane: the
// walk index is uniform, but the compiler cannot prove it inside a loop with
// divergent branches and would otherwise issue vector loads, whose waits
// (vmcnt, in order) would also wait for every store of the walk before them.
__device__ __forceinline__ int32_t sload(const int32_t *p) {         // p wave-uniform
    return load_uniform(reinterpret_cast<const int32_t *>(to_sgpr(p)));
}
__device__ __forceinline__ i32x4 sload4(const int32_t *p) {          // p 16-byte aligned, wave-uniform
    return *(const __attribute__((address_space(4))) i32x4 *)(uintptr_t)to_sgpr(p);
}

constexpr int kRing = 32;            // per-lane LDS ring of block starts (two 16-entry lines)
// Lane rings lie kRing + 1 words apart: lanes writing the same ring position
// then hit 64 different banks (a pitch of 32 words would put every lane of a
// parity on one bank).
constexpr int kRingPitch = kRing + 1;

template <bool kStaged>
__global__ __launch_bounds__(kThreads) void build_index_kernel(IndexArgs a) {
    __shared__ int32_t stage[kStaged ? kStageMax : 1];
    __shared__ int32_t ring_all[kThreads * kRingPitch];
    const int h = blockIdx.y;                        // head (of its sequence, in a packed batch)
    const SeqSpan sp = seq_span(a.vl.cu, h / a.hq, a.vl.rows, a.n);
    const int n = (int)sp.n;                         // sequence lengths are below 2^31
    const int nqb = (n + 63) / 64;
    const int64_t nqb_rows = (a.n + 63) / 64;        // query blocks per head in the arrays
    const int b = blockIdx.x * kThreads + threadIdx.x;
    const int32_t *S = a.s_idx + (int64_t)h * a.ks;
    const int32_t *V = a.v_idx + (int64_t)h * a.kv;
    if constexpr (kStaged) {
        for (int i = threadIdx.x; i < a.kv; i += kThreads) stage[i] = V[i];
        __syncthreads();
        V = stage;
    }
    if (b >= nqb) return;
    const int r0 = b * 64, r1 = min(r0 + 63, n - 1);          // the last block may be short
    const int64_t item = (int64_t)h * nqb_rows + b;
    int32_t *blk = a.block_offset + item * a.cap_b;
    int32_t *col = a.column_index + item * a.cap_c;
    // Every offset 0 .. r1 selected (the offsets ascend and are distinct, so
    // S[r1] == r1 says so; a sequence of at most ks tokens has all of them):
    // the walk would emit the aligned blocks 0, 64, .., 64 b, which cover
    // every key of the block and so every column.  Write them directly.
    if (r1 < a.ks && S[r1] == r1) {
        const int cnt = min(b + 1, a.cap_b);
        int j = 0;
        if (a.vec_rows)
            for (; j + 4 <= cnt; j += 4) *reinterpret_cast<int4 *>(blk + j) = make_int4(64 * j, 64 * j + 64, 64 * j + 128, 64 * j + 192);
        for (; j < cnt; ++j) blk[j] = 64 * j;
        a.block_count[item] = cnt;
        a.column_count[item] = 0;
        return;
    }

    // offsets that matter to some lane of the wave: those <= r1 of its last item
    const int wave_first = b - (int)(threadIdx.x & 63);
    const int r1_max = min(min(wave_first + 63, nqb - 1) * 64 + 63, n - 1);
    int lo = 0, hi = a.ks;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sload(S + mid) <= r1_max) lo = mid + 1; else hi = mid;
    }

    // Block starts go to a per-lane LDS ring; a lane writes a completed,
    // 16-entry-aligned run of its list as one 64-byte line (four 16-byte
    // stores) instead of 16 scattered 4-byte stores.
    int32_t *ring = ring_all + threadIdx.x * kRingPitch;
    const bool vec = a.vec_rows;                      // rows 16-byte aligned
    int flushed = 0;                                  // entries of blk already written
    auto flush_line = [&]() {                         // entries flushed .. flushed+15, all emitted
        const int32_t *rl = ring + (flushed & (kRing - 1));
        if (vec && flushed + 16 <= a.cap_b) {
#pragma unroll
            for (int k = 0; k < 16; k += 4)
                *reinterpret_cast<int4 *>(blk + flushed + k) = make_int4(rl[k], rl[k + 1], rl[k + 2], rl[k + 3]);
        } else {
            for (int k = 0; k < 16; ++k)
                if (flushed + k < a.cap_b) blk[flushed + k] = rl[k];
        }
        flushed += 16;
    };
    int cov = 0, cnt = 0, vp = 0, cc = 0;
    int vnext = a.kv > 0 ? V[0] : INT_MAX;           // column vp (INT_MAX past the list)
    // columns below `upto` (exclusive): the ones at or past cov are uncovered
    auto columns_below = [&](int upto) {
        while (vnext < upto) {
            if (vnext >= cov) {
                if (cc < a.cap_c) col[cc] = vnext;
                ++cc;
            }
            ++vp;
            vnext = vp < a.kv ? V[vp] : INT_MAX;
        }
    };
    auto step = [&](int o) {
        if (o < 0 || o > r1 || cov > r1) return;     // not this lane's offset, or done
        if (r1 - o < cov) return;                    // range already covered
        const int st = max(r0 - o, cov);             // r0 - o may be negative: cov >= 0 covers it
        columns_below(st);
        ring[cnt & (kRing - 1)] = st;
        ++cnt;
        cov = st + 64;
    };
    int i = lo - 1;
    // unaligned head of the walk (at most 15 steps), one offset at a time,
    // down to a group of sixteen
    for (; i >= 0 && (i & 15) != 15; --i) step(sload(S + i));
    const bool aligned = ((uintptr_t)S & 15) == 0;
    auto load16 = [&](int top) {                      // offsets top-15 .. top
        i32x16 g;
#pragma unroll
        for (int u = 0; u < 16; u += 4) {
            const i32x4 x = aligned ? sload4(S + top - 15 + u)
                                    : i32x4{sload(S + top - 15 + u), sload(S + top - 14 + u),
                                            sload(S + top - 13 + u), sload(S + top - 12 + u)};
            g[u] = x[0];
            g[u + 1] = x[1];
            g[u + 2] = x[2];
            g[u + 3] = x[3];
        }
        return g;
    };
    // each group of sixteen is loaded one iteration ahead, so the scalar loads
    // overlap the previous group's steps
    i32x16 qn = {};
    if (i >= 15) qn = load16(i);
    bool all_done = false;
    for (; i >= 15; i -= 16) {
        const i32x16 q = qn;
        if (i >= 31) qn = load16(i - 16);
#pragma unroll
        for (int u = 15; u >= 0; --u) step(q[u]);
        // at most 31 unflushed entries (15 left + 16 new): at most one line
        // is completed and the 32-entry ring has not wrapped onto it
        if (cnt - flushed >= 16) flush_line();
        if ((i & 63) == 63 && __builtin_amdgcn_ballot_w64(cov <= r1) == 0) {   // every lane is done
            all_done = true;
            break;
        }
    }
    for (; !all_done && i >= 0; --i) {
        step(sload(S + i));
        if (cnt - flushed >= 16) flush_line();
    }
    // the unfinished line
    for (int k = flushed; k < cnt; ++k)
        if (k < a.cap_b) blk[k] = ring[k & (kRing - 1)];
    columns_below(r1 + 1);
    a.block_count[item] = min(cnt, a.cap_b);
    a.column_count[item] = min(cc, a.cap_c);
}

}  // namespace

hipError_t launch_build_index(const IndexArgs &a, hipStream_t s) {
    const int64_t nqb = (a.n + 63) / 64;
    dim3 grid((unsigned)((nqb + kThreads - 1) / kThreads), a.hq * a.vl.nseq);
    if (a.kv <= kStageMax)
        hipLaunchKernelGGL(build_index_kernel<true>, grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(build_index_kernel<false>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace msa
