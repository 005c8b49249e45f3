// Sparse and dense causal prefill attention for gfx950.
//
// One workgroup = one (q head, 64-row query block) work item, two waves of 32
// query rows each.  The work item walks a list of 64-key tiles: for the sparse
// kernel, first the item's 64-wide key blocks (arbitrary start), then its
// leftover vertical columns gathered 64 at a time; for the dense kernel, the
// aligned tiles 0..b.  Per tile:
//   S^T = K Q^T        (MFMA 32x32x16; K tile from LDS, Q in registers)
//   online softmax in fp32 (exp2 with the log2(e)-folded scale)
//   O^T += V^T P^T     (P stays in registers as the B operand; V^T read from
//                       the row-major V tile with the LDS transpose read)
// Computing S transposed leaves each lane holding one query's scores for 16
// keys, so a row max needs only one cross-lane exchange (lane l with l^32), and
// those scores are already the B operand of the PV product.
//
// K and V rows move from HBM straight into LDS (global_load_lds, 16 bytes per
// lane, no registers), 16-byte chunks XOR-swizzled per row so that the MFMA
// operand reads are free of bank conflicts.
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

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

template <typename T> struct Geo {
    static constexpr int kRowBytes = kD * (int)sizeof(T);      // 256 (bf16) / 512 (fp32)
    static constexpr int kChunks = kRowBytes / 16;             // 16-byte chunks per row
    static constexpr int kTileBytes = kBK * kRowBytes;         // 16 KB / 32 KB
    static constexpr int kSlots = kTileBytes / 1024;           // 1 KB direct-load slots per tile
    static constexpr int kRowsPerSlot = 1024 / kRowBytes;
    // 16-byte chunk swizzles (bf16 only; the fp32 checking path keeps plain
    // rows).  Conflict-free whether the LDS serves 128 B or 256 B per clock:
    // K (ds_read_b128, rows r..r+15 at one logical chunk): phys = c ^ (row & 15);
    // V (transpose reads, 4 rows x 4 chunks per 32 lanes): phys = c ^ {0,4,10,14}[row & 3].
    __device__ static __forceinline__ int k_swz(int row) { return sizeof(T) == 2 ? (row & 15) : 0; }
    __device__ static __forceinline__ int v_swz(int row) {
        return sizeof(T) == 2 ? (4 * (row & 3) + 2 * ((row >> 1) & 1)) : 0;
    }
};

template <typename T> struct AttnStage {
    alignas(16) unsigned char k[Geo<T>::kTileBytes];
    alignas(16) unsigned char v[Geo<T>::kTileBytes];
    int32_t kidx[kBK];                                        // key of each tile row (-1: none)
};

// Work item (q head h, query block b) of workgroup bid: kv group by kv group,
// heavy (late) query blocks first, the G q heads of a block next to each
// other.  Consecutive ids are dispatched round-robin over the XCDs, so all
// XCDs stream the same kv head at once through the shared last-level cache
// (measured: as fast as or faster than pinning kv heads to XCDs).
__device__ __forceinline__ void item_of_block(int64_t bid, int64_t nqb, int G, int &h, int64_t &b) {
    const int64_t per_g = (int64_t)G * nqb;
    const int64_t g = bid / per_g, rem = bid % per_g;
    b = nqb - 1 - rem / G;
    h = (int)(g * G + rem % G);
}

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

// Start the HBM -> LDS copy of one tile's K and V rows.  Wave w moves the 1 KB
// slots w*S/2 .. w*S/2 + S/2 - 1 of each tile; in a slot, lane l writes the
// 16-byte physical chunk l % kChunks of row slot*kRowsPerSlot + l / kChunks,
// and so loads the logical chunk that the swizzle puts there.
//
// Fast path (64 consecutive keys inside the sequence): one uniform row address
// plus per-lane offsets that depend only on the lane and the slot.  Otherwise
// each row's key is looked up (column list) and clamped into the sequence: a
// row whose key does not exist (past the end, or column padding) reads an
// existing row, which the softmax mask gives weight zero (its values are
// finite), so no zero fill is needed.
template <typename T>
__device__ __forceinline__ void load_tile(AttnStage<T> &st, const T *kp, const T *vp, const TileSrc &src,
                                          int64_t n, const int32_t *clist, int ncol, int tid) {
    using Gm = Geo<T>;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    constexpr int kHalf = Gm::kSlots / 2;
    const int sub = lane / Gm::kChunks, phys = lane % Gm::kChunks;
    const char *kb = reinterpret_cast<const char *>(kp);
    const char *vb = reinterpret_cast<const char *>(vp);
    LDS_AS unsigned char *kl = (LDS_AS unsigned char *)st.k + wave * kHalf * 1024;
    LDS_AS unsigned char *vl = (LDS_AS unsigned char *)st.v + wave * kHalf * 1024;
    const int row0 = wave * kHalf * Gm::kRowsPerSlot;                 // first row of this wave
    if (!src.is_col && src.base >= 0 && src.base + kBK <= n) {
        const char *kt = kb + (src.base + row0) * Gm::kRowBytes;     // uniform
        const char *vt = vb + (src.base + row0) * Gm::kRowBytes;
#pragma unroll
        for (int i = 0; i < kHalf; ++i) {
            const int row = row0 + i * Gm::kRowsPerSlot + sub;
            const uint32_t rel = (uint32_t)((i * Gm::kRowsPerSlot + sub) * Gm::kRowBytes);
            __builtin_amdgcn_global_load_lds(kt + rel + ((phys ^ Gm::k_swz(row)) << 4),
                                             (LDS_AS void *)(kl + i * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vt + rel + ((phys ^ Gm::v_swz(row)) << 4),
                                             (LDS_AS void *)(vl + i * 1024), 16, 0, 0);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < kHalf; ++i) {
        const int row = row0 + i * Gm::kRowsPerSlot + sub;
        int64_t key = src.is_col ? (int64_t)clist[min(src.c0 + row, ncol - 1)] : src.base + row;
        key = min(max(key, (int64_t)0), n - 1);
        const int64_t rb = key * Gm::kRowBytes;
        __builtin_amdgcn_global_load_lds(kb + rb + ((phys ^ Gm::k_swz(row)) << 4),
                                         (LDS_AS void *)(kl + i * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vb + rb + ((phys ^ Gm::v_swz(row)) << 4),
                                         (LDS_AS void *)(vl + i * 1024), 16, 0, 0);
    }
    if (src.is_col && tid < kBK) {
        const int c = src.c0 + tid;
        st.kidx[tid] = c < ncol ? clist[c] : -1;
    }
}

// K fragment (A operand of S^T = K Q^T): row kt*32 + l32, d = dk*16 + hl*8 .. +7
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag k_frag(const AttnStage<T> &st, int kt, int dk, int l32, int hl) {
    using Gm = Geo<T>;
    const int row = kt * 32 + l32;
    if constexpr (sizeof(T) == 2) {
        const int c = dk * 2 + hl;
        return Elem<T>::load_frag(st.k + row * Gm::kRowBytes + ((c ^ Gm::k_swz(row)) << 4));
    } else {
        return Elem<T>::load_frag(st.k + row * Gm::kRowBytes + (dk * 16 + hl * 8) * 4);
    }
}

// V^T fragment (A operand of O^T = V^T P^T) for d-tile dt and key step kk:
// lane l needs V[key][d = dt*32 + l%32] for keys kk*16 + (e/4)*8 + hl*4 + e%4,
// e = 0..7 -- the order the S^T accumulator holds P in.
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag v_frag(const AttnStage<T> &st, int dt, int kk, int lane) {
    using Gm = Geo<T>;
    const int hl = lane >> 5;
    if constexpr (sizeof(T) == 2) {
        // LDS transpose read: in each 16-lane group, source lane 4i+q reads 4
        // consecutive d (d0 + 4q ..) of key row kb+i; output lane j then holds
        // keys kb..kb+3 of d = d0 + j.
        const int g = lane >> 4, j = lane & 15, i = j >> 2, q = j & 3;
        const int d = dt * 32 + (g & 1) * 16 + 4 * q;
        u32x4 r;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int row = kk * 16 + half * 8 + hl * 4 + i;
            const int c = d >> 3;
            const int off = row * Gm::kRowBytes + ((c ^ Gm::v_swz(row)) << 4) + ((d >> 2) & 1) * 8;
            const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (LDS_AS v4i16 *)(LDS_AS unsigned char *)(st.v + off));
            const u32x2 w = __builtin_bit_cast(u32x2, x);
            r[2 * half] = w[0];
            r[2 * half + 1] = w[1];
        }
        return __builtin_bit_cast(bf16x8, r);
    } else {
        const int d = dt * 32 + (lane & 31);
        f32x8 r;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int row = kk * 16 + (e >> 2) * 8 + hl * 4 + (e & 3);
            r[e] = *reinterpret_cast<const float *>(st.v + row * Gm::kRowBytes + d * 4);
        }
        return r;
    }
}

// bf16: one 33 KB LDS stage and two waves per SIMD (four workgroups per CU hide
// each other's load latency; measured faster than two stages at one wave per
// SIMD).  fp32 (a checking path): two stages, one wave per SIMD.
template <typename T, bool kDense, int kStages>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1, sizeof(T) == 2 ? 2 : 1)))
void attn_fwd_kernel(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // the body uses gfx950-only LDS builtins
    using E = Elem<T>;
    using frag = typename E::frag;
    __shared__ AttnStage<T> stage[kStages];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
    const int64_t n = a.n;
    const int64_t nqb = n / kBQ;
    const int G = a.hq / a.hkv;
    int h;
    int64_t b;
    item_of_block(blockIdx.x, nqb, G, h, b);
    const int g = h / G;
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

    if (kStages == 2 && ntile > 0) {
        load_tile<T>(stage[0], kp, vp, src_of(0), n, clist, ncol, tid);
        wait_vmem();
        __syncthreads();
    }

    for (int it = 0; it < ntile; ++it) {
        const TileSrc cur = src_of(it);
        if (kStages == 1) {
            load_tile<T>(stage[0], kp, vp, cur, n, clist, ncol, tid);
            wait_vmem();
            __syncthreads();
        } else if (it + 1 < ntile) {
            load_tile<T>(stage[(it + 1) & 1], kp, vp, src_of(it + 1), n, clist, ncol, tid);
        }
        const AttnStage<T> &st = stage[kStages == 1 ? 0 : (it & 1)];

        // S^T for this wave's 32 queries: two 32-key sub-tiles
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
            for (int dk = 0; dk < 8; ++dk) E::mma(s[kt], k_frag<T>(st, kt, dk, l32, hl), qf[dk]);
        }

        // mask: the key must exist and satisfy j <= i (keys past the end of the
        // sequence are > i, column padding is -1)
        if (cur.is_col) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int4 kk = *reinterpret_cast<const int4 *>(&st.kidx[kt * 32 + jj * 8 + hl * 4]);
                    const int kx[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (!(kx[i] >= 0 && kx[i] <= (int)qrow)) s[kt][jj * 4 + i] = -INFINITY;
                }
        } else if (cur.base + kBK - 1 > r0 || cur.base < 0) {
            // e allowed iff 0 <= base + e <= qrow
            const int hi = (int)min(max(qrow - cur.base, (int64_t)-1), (int64_t)kBK);
            const int lo = (int)min(max(-cur.base, (int64_t)0), (int64_t)kBK);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = kt * 32 + jj * 8 + hl * 4 + i;
                        if (e > hi || e < lo) s[kt][jj * 4 + i] = -INFINITY;
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
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) E::mma(o[dt], v_frag<T>(st, dt, kk, lane), pf[kk]);

        if (kStages == 2) wait_vmem();              // the next tile has landed
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
#endif
}

template <typename T, bool kDense> hipError_t launch(const AttnArgs &a, hipStream_t s) {
    const int64_t total = (int64_t)a.hq * (a.n / kBQ);
    if (total == 0) return hipSuccess;
    constexpr int kStages = sizeof(T) == 2 ? 1 : 2;
    hipLaunchKernelGGL((attn_fwd_kernel<T, kDense, kStages>), dim3((unsigned)total), dim3(kThreads), 0, s, a);
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
