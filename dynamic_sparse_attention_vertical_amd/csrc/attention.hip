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
    int32_t kidx[2][kBK];                                     // key of each column-tile row (-1: none), by tile parity
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

// HBM -> LDS copies of 16 bytes per lane (lane l's bytes land at lds + 16 l),
// issued from inline assembly: the compiler does not track these copies, so
// it never waits for them on its own (it would otherwise wait for all of them
// before any LDS read it cannot prove disjoint).  Completion is awaited with
// vm_wait<N>() (every copy but the last N issued has landed), then a barrier.
__device__ __forceinline__ void dma16(const void *gaddr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(lds) : "memory", "m0");
}
// same, with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit offset
__device__ __forceinline__ void dma16_sbase(const void *sbase, uint32_t voff, uint32_t lds) {
    const uint64_t u = (uint64_t)(uintptr_t)sbase;     // wave-uniform: move it to SGPRs
    sbase = (const void *)(uintptr_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32)) << 32) |
                                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u));
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
// s_waitcnt immediate for vmcnt(0) with the other counters unconstrained
// (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int kVmcnt0 = 0x0F70;
template <int N> __device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Read a wave-uniform int32 through the constant address space: a scalar load,
// counted by lgkmcnt.  A plain load of kernel-argument memory is a vector load
// (the compiler cannot prove the kernel never writes it), and its vmcnt wait
// would also wait for every HBM -> LDS copy in flight.
__device__ __forceinline__ int32_t load_uniform(const int32_t *p) {
    return *(const __attribute__((address_space(4))) int32_t *)(uintptr_t)p;
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(LDS_AS const unsigned char *)p;
}

// Start the HBM -> LDS copy of one tile's K rows (kIsV false) or V rows.  Wave
// w moves the 1 KB slots w*S/2 .. w*S/2 + S/2 - 1 of the tile (S/2 copies per
// lane); in a slot, lane l writes the 16-byte physical chunk l % kChunks of row
// slot*kRowsPerSlot + l / kChunks, and so loads the logical chunk that the
// swizzle puts there.
//
// Fast path (64 consecutive keys inside the sequence): a uniform base plus
// per-lane offsets that depend only on the lane and the slot.  Otherwise each
// row's key is looked up (column list) and clamped into the sequence: a row
// whose key does not exist (past the end, or column padding) reads an existing
// row, which the softmax mask gives weight zero (its values are finite).
template <typename T, bool kIsV>
__device__ __forceinline__ void load_half(unsigned char *dst, const T *src_rows, const TileSrc &src, int64_t n,
                                          const int32_t *clist, int ncol, int tid) {
    using Gm = Geo<T>;
    constexpr int kHalf = Gm::kSlots / 2;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int sub = lane / Gm::kChunks, phys = lane % Gm::kChunks;
    const char *rows = reinterpret_cast<const char *>(src_rows);
    const uint32_t l0 = lds_addr(dst) + wave * kHalf * 1024;
    const int row0 = wave * kHalf * Gm::kRowsPerSlot;                 // first row of this wave
    if (!src.is_col && src.base >= 0 && src.base + kBK <= n) {
        const char *tb = rows + (src.base + row0) * Gm::kRowBytes;     // uniform
#pragma unroll
        for (int i = 0; i < kHalf; ++i) {
            const int r = i * Gm::kRowsPerSlot + sub;                    // row - row0
            const int swz = kIsV ? Gm::v_swz(row0 + r) : Gm::k_swz(row0 + r);
            dma16_sbase(tb, (uint32_t)(r * Gm::kRowBytes + ((phys ^ swz) << 4)), l0 + i * 1024);
        }
        return;
    }
    // all key lookups first: each copy below is a compiler barrier for memory
    // operations, so a lookup placed after one would wait for every copy
    int64_t key[kHalf];
    if (src.is_col) {
#pragma unroll
        for (int i = 0; i < kHalf; ++i)
            key[i] = clist[min(src.c0 + row0 + i * Gm::kRowsPerSlot + sub, ncol - 1)];
    } else {
#pragma unroll
        for (int i = 0; i < kHalf; ++i) key[i] = src.base + row0 + i * Gm::kRowsPerSlot + sub;
    }
#pragma unroll
    for (int i = 0; i < kHalf; ++i) {
        const int row = row0 + i * Gm::kRowsPerSlot + sub;
        const int64_t kc = min(max(key[i], (int64_t)0), n - 1);
        const int swz = kIsV ? Gm::v_swz(row) : Gm::k_swz(row);
        dma16(rows + kc * Gm::kRowBytes + ((phys ^ swz) << 4), l0 + i * 1024);
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


// One 64-key tile of K and one of V in LDS (33 KB for bf16: four workgroups
// and two waves per SIMD), loaded out of phase so that every copy overlaps
// compute of the same workgroup:
//   top of tile t:  wait K[t]; barrier; start V[t]
//   S^T = K Q^T;    barrier; start K[t+1]
//   mask, online softmax, P
//   wait V[t];      barrier
//   O^T += V^T P^T
// V[t] has QK and softmax of tile t to land, K[t+1] has softmax and PV.  The
// per-row key list of a column tile is double buffered by tile parity.
// fp32 (a checking path) uses the same scheme with 64 KB of LDS.
template <typename T, bool kDense>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1, sizeof(T) == 2 ? 2 : 1)))
void attn_fwd_kernel(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // the body uses gfx950-only LDS builtins
    using E = Elem<T>;
    using frag = typename E::frag;
    constexpr int kHalf = Geo<T>::kSlots / 2;     // copies per lane per K or V tile
    __shared__ AttnStage<T> st;

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
        s.base = s.is_col ? 0 : (kDense ? (int64_t)it * kBK : (int64_t)load_uniform(blist + it));
        s.c0 = s.is_col ? (it - nblk) * kBK : 0;
        return s;
    };
    // start K of tile it (and record a column tile's keys for its mask)
    auto start_k = [&](int it, const TileSrc &s) {
        if (s.is_col && tid < kBK) st.kidx[it & 1][tid] = s.c0 + tid < ncol ? clist[s.c0 + tid] : -1;
        load_half<T, false>(st.k, kp, s, n, clist, ncol, tid);
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
    // Q has landed.  A compiler-visible wait: otherwise the compiler places its
    // waits for these loads inside the tile loop, where they would also wait
    // for the K/V copies in flight.
    __builtin_amdgcn_s_waitcnt(kVmcnt0);

    if (ntile > 0) start_k(0, src_of(0));

    for (int it = 0; it < ntile; ++it) {
        const TileSrc cur = src_of(it);
        vm_wait<0>();                                   // K[it] has landed (this wave's part)
        __syncthreads();                                // ... all parts; V is free
        load_half<T, true>(st.v, vp, cur, n, clist, ncol, tid);

        // S^T for this wave's 32 queries: two 32-key sub-tiles
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
            for (int dk = 0; dk < 8; ++dk) E::mma(s[kt], k_frag<T>(st, kt, dk, l32, hl), qf[dk]);
        }
        __syncthreads();                                // every wave is done with K
        const bool more = it + 1 < ntile;
        if (more) start_k(it + 1, src_of(it + 1));

        // mask: the key must exist and satisfy j <= i (keys past the end of the
        // sequence are > i, column padding is -1)
        if (cur.is_col) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int4 kk = *reinterpret_cast<const int4 *>(&st.kidx[it & 1][kt * 32 + jj * 8 + hl * 4]);
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
        mx = pair32_max(mx);
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

        if (more) vm_wait<kHalf>(); else vm_wait<0>();  // V[it] has landed (K[it+1] may not)
        __syncthreads();
        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) E::mma(o[dt], v_frag<T>(st, dt, kk, lane), pf[kk]);
    }

    // finalise: lanes l and l^32 hold halves of the same row's sum
    const float l_tot = pair32_sum(l_i);
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
