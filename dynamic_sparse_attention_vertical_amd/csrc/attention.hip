// Sparse and dense causal prefill attention for gfx950.
//
// One workgroup = one (q head, 64-row query block) work item, two waves of 32
// query rows each.  The work item walks a list of keys in 32-key chunks: for
// the sparse kernel, first the item's 64-wide key blocks (arbitrary start, two
// chunks each), then its leftover vertical columns gathered 32 at a time; for
// the dense kernel, the aligned tiles 0..b.  Per chunk:
//   S^T = K Q^T        (MFMA 32x32x16; K rows from LDS, Q in registers)
//   online softmax in fp32 (exp2 with the log2(e)-folded scale)
//   O^T += V^T P^T     (P stays in registers as the B operand; V^T read from
//                       the row-major V rows with the LDS transpose read)
// Computing S transposed leaves each lane holding one query's scores for 16
// keys, so a row max needs only one cross-lane exchange (lane l with l^32), and
// those scores are already the B operand of the PV product.
//
// The three stages are software pipelined across chunks: while a wave's VALU
// runs the softmax of chunk c, its matrix unit works on S of chunk c+1 and on
// O += V^T P^T of chunk c-1.
//
// K and V rows move from HBM straight into LDS (global_load_lds, 16 bytes per
// lane, no registers), 16-byte chunks XOR-swizzled per row so that the MFMA
// operand reads are free of bank conflicts.
//
// Long sparse sequences run in key phases, one launch per range of keys (12K
// by default): each launch takes the block tiles starting in its range, so the
// workgroups in flight read K/V from one cache-sized range of a kv head, and a
// query block's fp32 softmax state (O, row max, row sum) waits in a caller
// workspace between launches; its columns and its output go to the launch that
// holds its own rows.
//
// Before the phases, a query block whose lists leave few keys out for every
// q head of a kv group (a unit) runs as one walk over the aligned tiles 0..b,
// as in the dense kernel: one K/V copy per tile serves the group's heads, and
// each head masks the keys outside its own blocks and columns (its "holes").
// The walk marks the units it takes; the per-head launches skip them.
//
// The pages: causal attention computed only over the selected entries, in
// FlashAttention style (talk slides "System-Algorithm Co-design", slide
// "MInference": dynamic sparse attention calculation with PIT and
// FlashAttention); sparse work in large blocks for the matrix units ("How to
// optimise the TTFT of an 8B LLM with 1M tokens to 20 seconds", section on
// co-designing algorithm and system, principle 1).
#include "common.h"
#include "kernels.h"

#include <climits>

#include <type_traits>

namespace msa {
namespace {

constexpr int kD = 128;          // head_dim
constexpr int kBQ = 64;          // query rows per work item
constexpr int kBK = 64;          // keys per tile
constexpr int kThreads = 128;    // two waves per q head of a workgroup
constexpr int kStateFloats = 64 * 64 + 2 * 64;   // sparse phase state of one wave: O, max, sum
// A query block with fewer block tiles than this in a key phase (not its own)
// leaves them to the next phase: starting a work item (searching, loading Q
// and the state, filling the copy pipeline) costs about as much as four
// tiles, and storing the state again as much more, which a handful of tiles
// would not repay.  The tiles keep their order, so results do not change.
constexpr int kMinPhaseTiles = 16;
// A unit of the grouped walk (the q heads of one kv group sharing a workgroup,
// one query block) qualifies when every head's blocks and columns leave at
// most 1/8 of the keys [0, r1] out, in at most kGrpHoles ranges, with at most
// kGrpCols columns: walking all aligned tiles 0..b with one copy per tile for
// the group then costs at most an eighth more matrix work than the lists.
constexpr int kGrpHoles = 192;
constexpr int kGrpCols = 64;
// Fused mode (work lists built inside the kernel): the block starts of one
// item and key phase, and the item's leftover columns, held in LDS.  Blocks
// starting in one phase are disjoint and start inside its keys, so a phase of
// at most kFusedMaxPhase keys has at most kFusedMaxPhase / 64 of them, plus
// fewer than kMinPhaseTiles left over from earlier phases.
constexpr int kFusedMaxPhase = 16384;
constexpr int kFusedBlocks = kFusedMaxPhase / 64 + 32;
constexpr int kFusedCols = 1024;

typedef short v4i16 __attribute__((ext_vector_type(4)));

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
    int32_t kidx[4][32];                                      // key of each column-chunk row (-1: none), by chunk % 4
};

// Work item (q head h, query block b) of workgroup bid: kv group by kv group,
// heavy (late) query blocks first, the G q heads of a block next to each
// other.  Consecutive ids are dispatched round-robin over the XCDs, so all
// XCDs stream the same kv head at once through the shared last-level cache
// (measured: as fast as or faster than pinning kv heads to XCDs).  For a
// workgroup serving kH q heads, G here is the number of kH-head groups per kv
// head and h indexes those groups.
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

// Where a chunk's 32 keys come from: consecutive keys from `base`, or entries
// c0 .. c0+31 of the column list (entries past `ncol` are empty).  Key
// arithmetic is 32-bit: sequence lengths are below 2^31.
struct ChunkSrc {
    bool is_col;
    bool fast;      // 32 consecutive keys inside the sequence (both chunks of the tile)
    bool masked;    // some score of the tile needs the mask
    int base;
    int c0;
    uint64_t allow; // grouped walk: bit e set iff key base + e is in this wave's head's lists
    bool causal;    // some key of the tile is past a row or outside the sequence
};
// The exact union mask also carries words of the selected-offset bitmap from
// bit sbase on (the tile's offsets) and of the selected-column bitmap from bit
// vbase on (the tile's keys).
struct ExactSrc : ChunkSrc {
    uint32_t sx0, sx1, sx2, sx3, sx4, vx0, vx1, vx2;
    int sbase, vbase;
};

// Per-lane constants of the chunk copies.  A chunk (32 rows) is moved by the
// 2 kH waves of the workgroup, kRpw = 16 / kH rows each (wave w: chunk rows
// w kRpw .. w kRpw + kRpw - 1) as kPer 1 KB slots; in slot i, lane l writes the
// 16-byte physical chunk l % kChunks of row i*kRowsPerSlot + l / kChunks and so
// reads the logical chunk that the swizzle puts there.  The swizzles depend on
// row & 15 and row & 3, and 16 divides 32 half, so the fast-path offsets of a
// wave are the same for every chunk.
template <typename T, int kH> struct CopyLanes {
    static constexpr int kRpw = 16 / kH;                                // rows per wave and chunk
    static constexpr int kPer = kRpw * Geo<T>::kRowBytes / 1024;        // 1 KB copies per wave and chunk
    uint32_t k[kPer], v[kPer];      // fast path: byte offset from the wave's first row
    int sub, phys;
    __device__ __forceinline__ void init(int lane, int wave) {
        using Gm = Geo<T>;
        sub = lane / Gm::kChunks;
        phys = lane % Gm::kChunks;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int r = i * Gm::kRowsPerSlot + sub;
            const int row = wave * kRpw + r;                            // row in the chunk
            k[i] = (uint32_t)(r * Gm::kRowBytes + ((phys ^ Gm::k_swz(row)) << 4));
            v[i] = (uint32_t)(r * Gm::kRowBytes + ((phys ^ Gm::v_swz(row)) << 4));
        }
    }
};

// Start the HBM -> LDS copy of one chunk's K rows (kIsV false) or V rows into
// rows 32*half .. 32*half+31 of the K or V tile (this wave's 16 of them).
//
// Fast path (32 consecutive keys inside the sequence): one uniform base.
// Otherwise each row's key is looked up and clamped into the sequence: a row
// whose key does not exist (past the end, or column padding) reads an existing
// row, which the softmax mask gives weight zero (its values are finite).  The
// keys of a column chunk come from the list for K, and from LDS for V (recorded
// when its K was started).
template <typename T, int kH, bool kIsV>
__device__ __forceinline__ void load_chunk(const CopyLanes<T, kH> &cl, uint32_t lds_wave, const T *src_rows,
                                           const ChunkSrc &src, int half, int wave, int n, const int32_t *clist,
                                           int ncol, const int32_t *keys_lds) {
    using Gm = Geo<T>;
    constexpr int kPer = CopyLanes<T, kH>::kPer;
    constexpr int kRpw = CopyLanes<T, kH>::kRpw;
    const char *rows = reinterpret_cast<const char *>(src_rows);
    const uint32_t l0 = lds_wave + half * 32 * Gm::kRowBytes;
    const uint32_t *off = kIsV ? cl.v : cl.k;
    if (src.fast) {
        const char *tb = rows + (int64_t)(src.base + wave * kRpw) * Gm::kRowBytes;
        if constexpr (kPer % 4 == 0) {
#pragma unroll
            for (int i = 0; i < kPer; i += 4) dma_x4(tb, off[i], off[i + 1], off[i + 2], off[i + 3], l0 + i * 1024);
        } else {
#pragma unroll
            for (int i = 0; i < kPer; ++i) dma_x1(tb, off[i], l0 + i * 1024);
        }
        return;
    }
    // all key lookups first: each copy below is a compiler barrier for memory
    // operations, so a lookup placed after one would wait for every copy
    int key[kPer];
    if (src.is_col && kIsV) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) key[i] = keys_lds[wave * kRpw + i * Gm::kRowsPerSlot + cl.sub];
    } else if (src.is_col) {
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            key[i] = clist[min(src.c0 + wave * kRpw + i * Gm::kRowsPerSlot + cl.sub, ncol - 1)];
    } else {
#pragma unroll
        for (int i = 0; i < kPer; ++i) key[i] = src.base + wave * kRpw + i * Gm::kRowsPerSlot + cl.sub;
    }
    const char *a[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int row = wave * kRpw + i * Gm::kRowsPerSlot + cl.sub;    // row in the chunk
        const int kc = min(max(key[i], 0), n - 1);
        const int swz = kIsV ? Gm::v_swz(row) : Gm::k_swz(row);
        a[i] = rows + (int64_t)kc * Gm::kRowBytes + ((cl.phys ^ swz) << 4);
    }
    if constexpr (kPer % 4 == 0) {
#pragma unroll
        for (int i = 0; i < kPer; i += 4) dma_x4(a[i], a[i + 1], a[i + 2], a[i + 3], l0 + i * 1024);
    } else {
#pragma unroll
        for (int i = 0; i < kPer; ++i) dma_x1(a[i], l0 + i * 1024);
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


// Per-lane choice under a wave-uniform 64-bit lane mask: lane l gets `b`
// where bit l of `mask` is set, else `a` (one v_cndmask with an SGPR pair).
__device__ __forceinline__ float lane_select(float a, float b, uint64_t mask) {
    float r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(mask));
    return r;
}

// First index i in [0, cnt) with list[i] >= key (cnt if none) in an ascending
// list.  The 64 lanes of the wave probe 64 evenly spaced entries per round and
// the ballot of the comparisons narrows the range 64-fold, so a list of up to
// 4096 entries takes two rounds of loads.
__device__ __forceinline__ int lower_bound_wave(const int32_t *list, int cnt, int key, int lane) {
    int lo = 0, hi = cnt;
    while (lo < hi) {
        const int step = (hi - lo + 63) >> 6;
        const int pos = lo + lane * step;
        const bool ge = pos < hi && list[pos] >= key;
        const uint64_t m = __builtin_amdgcn_ballot_w64(ge);
        if (m != 0) {
            const int f = __builtin_ctzll(m);
            const int nhi = lo + f * step;
            lo = f > 0 ? lo + (f - 1) * step + 1 : nhi;
            hi = nhi;
        } else {
            lo += ((hi - 1 - lo) / step) * step + 1;    // past the last probe
        }
    }
    return lo;
}

// The same for a key whose index is usually among the first 128 entries (the
// end of a key phase, counted from its start): one lower_bound_wave over
// those first, so the common case takes two rounds of loads.
__device__ __forceinline__ int lower_bound_near(const int32_t *list, int cnt, int key, int lane) {
    const int w = min(cnt, 128);
    const int i = lower_bound_wave(list, w, key, lane);
    return (i < w || cnt <= 128) ? i : 128 + lower_bound_wave(list + 128, cnt - 128, key, lane);
}

// One 64-key tile of K and one of V in LDS (33 KB for bf16: four workgroups
// and two waves per SIMD), each holding two 32-key chunks; chunk c lives in
// half c % 2.  Step c of the pipeline (after a wait and a barrier):
//   start the copies of K of chunk c+2 and V of chunk c
//   mask S(c) where needed
//   MFMA: S(c+1) = K(c+1) Q^T,  O^T += V(c-1)^T P(c-1)
//   VALU: online softmax of S(c) -> P(c)
//   rescale O if a row maximum moved (after PV(c-1), before PV(c))
// K of chunk c+1 and V of chunk c-1 were started one step earlier.  The last
// step computes an S that is never used (from K rows still in LDS), which
// keeps the step free of branches around the matrix work.
// fp32 (a checking path) uses the same scheme with 64 KB of LDS.
// kH q heads of one kv group per workgroup (2 kH waves) share every K/V copy;
// used by the dense kernel, whose heads all walk the same tiles.
// kVar: a packed batch of sequences of different lengths (AttnArgs.vl), each
// workgroup's heads belonging to one of them; otherwise one sequence.
template <typename T, bool kDense, int kH, bool kGrp = false, bool kFused = false, bool kExact = false,
          bool kVar = false>
__global__ __launch_bounds__(kThreads * kH) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1, sizeof(T) == 2 ? 2 : 1)))
void attn_fwd_kernel(AttnArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)   // the body uses gfx950-only LDS builtins
    using E = Elem<T>;
    using frag = typename E::frag;
    __shared__ AttnStage<T> st;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
    // query blocks per head in the per-head arrays (those of the longest
    // sequence of a packed batch)
    const int64_t nqb = (a.n + kBQ - 1) / kBQ;
    const int64_t heads = kVar ? (int64_t)a.hq * a.vl.nseq : a.hq;   // heads in the per-head arrays
    const int G = a.hq / a.hkv;
    int hgrp;
    int64_t b;
    const int64_t qb0 = kDense ? 0 : a.qb_lo;         // first query block of this launch
    item_of_block(blockIdx.x, nqb - qb0, G / kH, hgrp, b);
    b += qb0;
    const int h = hgrp * kH + (wave >> 1);           // this wave's q head (in the per-head arrays)
    // its sequence (the workgroup's heads share it) and the head within it
    int seq = 0;
    SeqSpan span{0, a.n};
    if constexpr (kVar) {
        seq = (hgrp * kH) / a.hq;
        span = seq_span(a.vl.cu, seq, a.vl.rows, a.n);
        if (b * kBQ >= span.n) return;               // past the end of a shorter sequence
    }
    const int64_t n = span.n;
    const int n32 = (int)n;                          // below 2^31
    const int hs = h - seq * a.hq;
    const int g = hs / G;
    const int r0 = (int)b * kBQ;
    const int qrow = r0 + (wave & 1) * 32 + l32;

    const T *qp = reinterpret_cast<const T *>(a.q) + ((int64_t)hs * a.stride + span.row0) * kD;
    const T *kp = reinterpret_cast<const T *>(a.k) + ((int64_t)g * a.stride + span.row0) * kD;
    const T *vp = reinterpret_cast<const T *>(a.v) + ((int64_t)g * a.stride + span.row0) * kD;

    // Q fragments (B operand of S^T = K Q^T): query qrow, d = dk*16 + hl*8 + e.
    // A per-head sparse item in a key phase that surely runs (its own rows'
    // phase) or likely runs (it holds a state from an earlier phase) loads
    // them, and its state, before finding its part of the lists, so those
    // latencies overlap; other items, which often leave a phase with few
    // tiles to the next one, load Q once they know they run.  The dense and
    // grouped kernels load Q after qualifying.
    frag qf[8];
    bool q_loaded = false;
    auto load_q = [&]() {
#pragma unroll
        for (int dk = 0; dk < 8; ++dk)
            qf[dk] = E::load_frag(qp + (int64_t)min(qrow, n32 - 1) * kD + dk * 16 + hl * 8);
        q_loaded = true;
    };
    auto load_q_early = [&]() {
        if (!q_loaded) load_q();
    };
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    // running row max kept in scaled log2 units as a stored fp32 value, so an
    // unchanged max gives a rescale factor of exactly 1
    float mb_i = -INFINITY, l_i = 0.f;
    auto load_state = [&](const float *sw) {         // this wave's state: 16 float4 of O per lane, max, sum
#pragma unroll
        for (int v4 = 0; v4 < 16; ++v4) {
            const float4 x = *reinterpret_cast<const float4 *>(sw + (v4 * 64 + lane) * 4);
            o[v4 >> 2][(v4 & 3) * 4 + 0] = x.x;
            o[v4 >> 2][(v4 & 3) * 4 + 1] = x.y;
            o[v4 >> 2][(v4 & 3) * 4 + 2] = x.z;
            o[v4 >> 2][(v4 & 3) * 4 + 3] = x.w;
        }
        mb_i = sw[4096 + lane];
        l_i = sw[4096 + 64 + lane];
    };

    // Grouped walk: each wave lists its head's holes (key ranges in [0, r1]
    // outside the head's blocks, ascending) and columns in LDS, and the unit
    // goes ahead only if every head qualifies; the verdict goes to grp.
    __shared__ int32_t glist[kGrp ? 2 * kH : 1][2 * kGrpHoles + kGrpCols];
    int nhole = 0, ncl_g = 0;
    if constexpr (kGrp) {
        const int lim = min(r0 + kBQ, n32);                // keys [0, r1]
        const int64_t item = (int64_t)h * nqb + b;
        const int nbk = min(max(load_uniform(a.block_count + item), 0), a.cap_b);
        ncl_g = min(max(load_uniform(a.column_count + item), 0), a.cap_c);
        bool ok = ncl_g <= kGrpCols && (int64_t)kBK * nbk + ncl_g >= lim - lim / 8;
        int32_t *hw = glist[wave];
        if (ok) {
            const int32_t *bl = a.block_offset + item * a.cap_b;
            int prev = 0;                                  // end of the blocks so far
            int prev_s = 0;                                // start of the last block so far
            bool bad = false;                              // blocks not ascending and disjoint
            int s_next = lane < nbk ? bl[lane] : lim;      // one round of loads ahead
            for (int base = 0; base < nbk && nhole <= kGrpHoles; base += 64) {
                const int i = base + lane;
                const int s = s_next;
                s_next = i + 64 < nbk ? bl[i + 64] : lim;
                const int lo = min(max(s, 0), lim), hi = min(max(s + kBK, 0), lim);
                int pe = __shfl_up(hi, 1, 64);
                int ps = __shfl_up(s, 1, 64);
                if (lane == 0) {
                    pe = prev;
                    ps = prev_s;
                }
                bad |= i < nbk && i > 0 && (int64_t)s < (int64_t)ps + kBK;
                const bool gap = i < nbk && lo > pe;
                const uint64_t m = __builtin_amdgcn_ballot_w64(gap);
                const int pos = nhole + __builtin_popcountll(m & ((1ull << lane) - 1));
                if (gap && pos < kGrpHoles) {
                    hw[2 * pos] = pe;
                    hw[2 * pos + 1] = lo;
                }
                nhole += __builtin_popcountll(m);
                prev = __shfl(hi, min(nbk - base, 64) - 1, 64);
                prev_s = __shfl(s, min(nbk - base, 64) - 1, 64);
            }
            ok = __builtin_amdgcn_ballot_w64(bad) == 0;
            if (prev < lim) {
                if (lane == 0 && nhole < kGrpHoles) {
                    hw[2 * nhole] = prev;
                    hw[2 * nhole + 1] = lim;
                }
                ++nhole;
            }
            ok = ok && nhole <= kGrpHoles;
            if (ok) {
                // the walk below reads the columns in ascending order; a list
                // in any other order runs per head instead
                const int32_t *cl = a.column_index + item * a.cap_c;
                bool unsorted = false;
                for (int i = lane; i < ncl_g; i += 64) {
                    const int c = cl[i];
                    hw[2 * kGrpHoles + i] = c;
                    unsorted |= i > 0 && c <= cl[i - 1];
                }
                ok = __builtin_amdgcn_ballot_w64(unsorted) == 0;
                // uncovered keys: the holes less the columns (which all lie in holes)
                int len = 0;
                for (int j = lane; j < nhole; j += 64) len += hw[2 * j + 1] - hw[2 * j];
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) len += __shfl_xor(len, o, 64);
                ok = ok && len - ncl_g <= lim / 8;
            }
        }
        const bool unit_ok = __syncthreads_and(ok) != 0;
        if (tid == 0) a.grp[(int64_t)hgrp * nqb + b] = unit_ok ? 1 : 0;
        if (!unit_ok) return;
    }

    int nblk, ncol;
    const int32_t *blist = nullptr, *clist = nullptr;
    __shared__ int32_t fblk[kFused ? kFusedBlocks : 1];
    __shared__ int32_t fcol[kFused ? kFusedCols : 1];
    __shared__ int32_t fwalk[5];                     // fused walk: blocks, columns, offset index, cover end, column index
    int fcov_next = 0, fcol_next = 0;
    if constexpr (kFused) clist = fcol;
    // key phases (sparse, ws set): the first starts from an empty state, and
    // the query block's output is written in the phase holding its own rows
    // (no later key is visible to it); in between the state lives in ws
    bool first = true, final_ = true, have_state = false;
    float *sw = nullptr;                             // this wave's state: 16 float4 of O per lane, max, sum
    int2 *phase_rec = nullptr;                       // (state stored, first block of the next phase)
    int b_next = 0;                                  // first block of the next phase
    if constexpr (kDense) {
        nblk = (int)b + 1;
        ncol = 0;
    } else if constexpr (kFused) {
        // Fused mode: this phase's blocks are the part of the greedy cover
        // (the one msa_build_index writes) that starts before k_hi, walked
        // here over the head's ascending diagonal offsets from where the
        // previous phase stopped; its columns are the selected ones in
        // [cover end before, cover end after) that its blocks leave out (the
        // final phase: up to r1), so every uncovered column falls in exactly
        // one phase.  Carried between phases: the offset index (record .y),
        // the column index (record .x >> 1, next to the state flag in bit 0)
        // and the cover end (fused_cov).
        const int64_t item = (int64_t)h * nqb + b;
        const int32_t *S = a.s_idx + (int64_t)h * a.ks;
        const int32_t *V = a.v_idx + (int64_t)h * a.kv;
        const int r1 = min(r0 + kBQ - 1, n32 - 1);
        first = a.ws == nullptr || a.k_lo == INT_MIN;
        final_ = a.ws == nullptr || (int64_t)r0 + kBQ - 1 < (int64_t)a.k_hi;
        const int k_hi = final_ ? INT_MAX : a.k_hi;
        if (final_) load_q_early();
        int i_in, cov_in = 0, ci_in = 0;
        if (a.ws != nullptr) {
            phase_rec = reinterpret_cast<int2 *>(a.ws + heads * nqb * 2 * kStateFloats) + item;
            sw = a.ws + item * (2 * kStateFloats) + wave * kStateFloats;
        }
        if (first) {
            i_in = lower_bound_wave(S, a.ks, r1 + 1, lane) - 1;       // offsets <= r1 are S[0 .. i_in]
        } else {
            const int2 rec = *phase_rec;
            const int rx = __builtin_amdgcn_readfirstlane(rec.x);
            have_state = (rx & 1) != 0;
            if (have_state) {
                load_q_early();
                load_state(sw);
            }
            ci_in = min(max(rx >> 1, 0), a.kv);
            i_in = min(__builtin_amdgcn_readfirstlane(rec.y), a.ks - 1);
            cov_in = max(__builtin_amdgcn_readfirstlane(load_uniform(a.fused_cov + item)), 0);
        }
        // A phase emits at most as many blocks as it has offsets whose ranges
        // start before k_hi (a run of k ranges takes at most k blocks): when
        // the 16th offset from i_in on already starts at or past k_hi, the
        // phase cannot reach kMinPhaseTiles and is left to the next one
        // without a walk.
        if (a.ws != nullptr && !final_ &&
            (i_in < kMinPhaseTiles - 1 ||
             (int64_t)r0 - load_uniform(S + (i_in - (kMinPhaseTiles - 1))) >= (int64_t)k_hi)) {
            if (first && tid == 0) {
                *phase_rec = make_int2(0, i_in);
                a.fused_cov[item] = 0;
            }
            return;
        }
        if (wave == 0) {                                // one wave walks, both read the lists after the barrier
            // the first two windows of columns, loaded now so that they land during the walk
            int cw = ci_in + lane < a.kv ? V[ci_in + lane] : INT_MAX;
            int cw_n = ci_in + 64 + lane < a.kv ? V[ci_in + 64 + lane] : INT_MAX;
            // Blocks, 64 offsets per step, one per lane in walk order (lane L:
            // offset index i - L, so range starts a = r0 - o ascend over the
            // lanes).  Ranges [a, a + d] that touch or overlap their
            // predecessor form a run whose union is one interval [L, R]; the
            // greedy cover tiles a run with consecutive blocks from its first
            // uncovered key, so a run m emits ceil((len - e) / 64) blocks from
            // L + e, e = max(s - g, 0), where g is the gap from the previous
            // run's end and s that run's overhang past its end, s' = (e - len)
            // mod 64 (len = R - L + 1).  The overhangs form a short chain,
            // solved by iterating to the fixed point (exact after as many
            // rounds as the longest chain of runs closer than 64 keys); a
            // prefix sum places the blocks.  The offsets come through LDS
            // (the tile stage is free until the pipeline starts), 1024 per
            // memory round trip.
            constexpr int kRound = 1024;
            int32_t *stage = reinterpret_cast<int32_t *>(st.k);
            const int d = r1 - r0;                      // a range covers keys [a, a + d]
            int i = i_in, cov = cov_in, nb = 0;
            int rhi = -1, rlo = 0;                      // staged: indices rlo .. rhi in slots rhi - index
            while (i >= 0 && cov <= r1) {
                if (i > rhi || (i - 63 < rlo && rlo > 0)) {
                    rhi = i;
                    rlo = max(i - (kRound - 1), 0);
                    int v[kRound / 64];
#pragma unroll
                    for (int k = 0; k < kRound / 64; ++k) {
                        const int idx = rhi - (k * 64 + lane);
                        v[k] = idx >= rlo ? S[idx] : -1;
                    }
#pragma unroll
                    for (int k = 0; k < kRound / 64; ++k) stage[k * 64 + lane] = v[k];
                }
                const int o = i - lane >= 0 ? stage[rhi - i + lane] : -1;
                // offsets below 0 (and indices below 0) select nothing and end the walk
                const uint64_t vmask = __builtin_amdgcn_ballot_w64(o >= 0);
                const int nvalid = vmask == ~0ull ? 64 : __builtin_ctzll(~vmask);
                const int a_ = r0 - o;
                // ranges the cover already holds
                const uint64_t cmask = __builtin_amdgcn_ballot_w64(lane < nvalid && a_ + d < cov);
                const int nskip = cmask == ~0ull ? 64 : __builtin_ctzll(~cmask);
                const bool live = lane >= nskip && lane < nvalid;
                const int a_prev = __shfl_up(a_, 1, 64);
                const bool head = live && (lane == nskip || a_ > a_prev + d + 1);
                const uint64_t heads = __builtin_amdgcn_ballot_w64(head);
                bool stopped = false;
                if (heads != 0) {
                    const uint64_t after = lane == 63 ? 0ull : heads & (~0ull << (lane + 1));
                    const int next_h = after != 0 ? __builtin_ctzll(after) : nvalid;
                    const int R = __shfl(a_, max(next_h - 1, 0), 64) + d;
                    const int len = R - a_ + 1;
                    const int g = lane == nskip ? a_ - cov : a_ - (a_prev + d) - 1;
                    const uint64_t before = heads & ((1ull << lane) - 1);
                    const int prev_h = before != 0 ? 63 - __builtin_clzll(before) : -1;
                    int sv = (-len) & 63, e = 0;
                    while (true) {
                        const int sp_ = __shfl(sv, max(prev_h, 0), 64);
                        e = max((prev_h >= 0 ? sp_ : 0) - g, 0);
                        const int s_new = (e - len) & 63;
                        const bool changed = __builtin_amdgcn_ballot_w64(head && s_new != sv) != 0;
                        sv = s_new;
                        if (!changed) break;
                    }
                    const int start = a_ + e;
                    const int cnt = head && e < len ? (len - e + kBK - 1) / kBK : 0;
                    int cnt2 = cnt;
                    if (k_hi != INT_MAX)
                        cnt2 = (int)min((int64_t)cnt, max((int64_t)0, ((int64_t)k_hi - start + kBK - 1) / kBK));
                    const uint64_t cut = __builtin_amdgcn_ballot_w64(cnt2 < cnt);
                    if (cut != 0) {                     // a later phase's block: this phase ends there
                        stopped = true;
                        if (lane > __builtin_ctzll(cut)) cnt2 = 0;
                    }
                    int incl = cnt2;                    // inclusive prefix sum over the lanes
#pragma unroll
                    for (int off = 1; off < 64; off <<= 1) {
                        const int t = __shfl_up(incl, off, 64);
                        if (lane >= off) incl += t;
                    }
                    const int pos = nb + incl - cnt2;
                    for (int j = 0; j < cnt2 && pos + j < kFusedBlocks; ++j) fblk[pos + j] = start + kBK * j;
                    nb += __shfl(incl, 63, 64);
                    const uint64_t emitted = __builtin_amdgcn_ballot_w64(cnt2 > 0);
                    if (emitted != 0) cov = __shfl(start + kBK * cnt2, 63 - __builtin_clzll(emitted), 64);
                }
                if (stopped) {                          // resume at the first range the cover does not hold
                    const uint64_t unc = __builtin_amdgcn_ballot_w64(lane < nvalid && a_ + d >= cov);
                    i -= unc != 0 ? __builtin_ctzll(unc) : nvalid;
                    break;
                }
                i = nvalid < 64 ? -1 : i - 64;
            }
            if (cov > r1) i = -1;                       // every remaining range is covered
            const int nbl = min(nb, kFusedBlocks);
            // Columns, lane-parallel: this phase takes the selected columns in
            // [cov_in, x_end) that none of its blocks covers (the blocks of
            // earlier phases end by cov_in, those of later phases start at or
            // past x_end); the final phase takes the rest up to r1.
            const int x_end = final_ ? r1 + 1 : cov;
            const uint64_t below = (1ull << lane) - 1;
            int ci = ci_in, nc = 0;
            if (final_ && a.fused_cols != nullptr && ci_in > 0) {
                // the columns earlier phases took: set bits of the bitmap,
                // all below ci_in, in index (so key) order
                const uint32_t *bm = a.fused_cols + item * a.fused_cw;
                const uint32_t word = lane < a.fused_cw ? bm[lane] : 0u;
                int vwin = lane < ci_in ? V[lane] : INT_MAX;
                for (int base = 0; base < ci_in; base += 64) {
                    const int vnext = base + 64 + lane < ci_in ? V[base + 64 + lane] : INT_MAX;
                    const uint32_t lo = __builtin_amdgcn_readlane(word, base >> 5);
                    const uint32_t hi = (base >> 5) + 1 < a.fused_cw ? __builtin_amdgcn_readlane(word, (base >> 5) + 1) : 0u;
                    const uint64_t bits = ((uint64_t)hi << 32 | lo);
                    const bool take = base + lane < ci_in && ((bits >> lane) & 1) != 0;
                    const uint64_t m = __builtin_amdgcn_ballot_w64(take);
                    const int at = nc + __builtin_popcountll(m & below);
                    if (take && at < kFusedCols) fcol[at] = vwin;
                    nc += __builtin_popcountll(m);
                    vwin = vnext;
                }
            }
            int top_bit = 1;                            // the largest power of two <= nbl
            while (top_bit * 2 <= nbl) top_bit *= 2;
            while (true) {
                const bool in = cw >= cov_in && cw < x_end;
                if (__builtin_amdgcn_ballot_w64(in) != 0) {
                    int pos = 0;                        // blocks starting at or before cw
                    if (nbl > 0)
                        for (int bit = top_bit; bit > 0; bit >>= 1)
                            if (pos + bit <= nbl && fblk[pos + bit - 1] <= cw) pos += bit;
                    const bool take = in && !(pos > 0 && cw < fblk[pos - 1] + kBK);
                    const uint64_t m = __builtin_amdgcn_ballot_w64(take);
                    const int at = nc + __builtin_popcountll(m & below);
                    // the final phase lists the keys; an earlier one their
                    // indices in v_idx, for the bitmap the final phase reads
                    if (take && at < kFusedCols) fcol[at] = final_ ? cw : ci + lane;
                    nc += __builtin_popcountll(m);
                }
                const uint64_t lower = __builtin_amdgcn_ballot_w64(cw < x_end);
                if (lower != ~0ull) {                   // the first column at or past x_end is here
                    ci += __builtin_popcountll(lower);
                    break;
                }
                ci += 64;
                cw = cw_n;
                cw_n = ci + 64 + lane < a.kv ? V[ci + 64 + lane] : INT_MAX;
            }
            if (lane == 0) {
                fwalk[0] = nbl;
                fwalk[1] = min(nc, kFusedCols);
                fwalk[2] = i;
                fwalk[3] = cov;
                fwalk[4] = ci;
            }
        }
        __syncthreads();
        nblk = __builtin_amdgcn_readfirstlane(fwalk[0]);
        ncol = __builtin_amdgcn_readfirstlane(fwalk[1]);
        b_next = __builtin_amdgcn_readfirstlane(fwalk[2]);
        fcov_next = __builtin_amdgcn_readfirstlane(fwalk[3]);
        fcol_next = __builtin_amdgcn_readfirstlane(fwalk[4]);
        if (a.ws != nullptr && !final_ && nblk < kMinPhaseTiles) {
            // too little here: leave it to the next phase, which starts from the same place
            if (first && tid == 0) {
                *phase_rec = make_int2(0, i_in);
                a.fused_cov[item] = 0;
            }
            return;
        }
        if (!q_loaded) load_q();
        if (!final_) {                                  // this phase's columns run in the final phase
            if (wave == 0)
                for (int t = lane; t < ncol; t += 64) {
                    const int idx = fcol[t];
                    atomicOr(a.fused_cols + item * a.fused_cw + (idx >> 5), 1u << (idx & 31));
                }
            ncol = 0;
        }
    } else {
        if (a.grp != nullptr &&
            load_uniform(a.grp + (int64_t)(h / a.grp_kh) * nqb + b) != 0)   // done by the grouped walk
            return;
        const int64_t item = (int64_t)h * nqb + b;
        nblk = min(max(a.block_count[item], 0), a.cap_b);
        ncol = min(max(a.column_count[item], 0), a.cap_c);
        blist = a.block_offset + item * a.cap_b;
        clist = a.column_index + item * a.cap_c;
        if (a.ws != nullptr) {
            // this phase's part: the block tiles from where the previous phase
            // stopped up to the first start at or past k_hi (the lists are
            // ascending; that is the tiles starting in [k_lo, k_hi) plus any
            // left over from earlier phases, and the last phase takes the rest).
            // The columns all go to the final phase: every block of a head
            // draws them from the same few keys, so they need no splitting for
            // locality.
            first = a.k_lo == INT_MIN;
            final_ = (int64_t)r0 + kBQ - 1 < (int64_t)a.k_hi;
            if (final_) load_q_early();
            // every query block passes the first phase, which writes its
            // record; each phase with work updates it, so the next one finds
            // where its blocks start without a search
            phase_rec = reinterpret_cast<int2 *>(a.ws + heads * nqb * 2 * kStateFloats) + item;
            int2 rec = make_int2(0, 0);
            sw = a.ws + item * (2 * kStateFloats) + wave * kStateFloats;
            if (!first) {
                rec = *phase_rec;
                rec.x = __builtin_amdgcn_readfirstlane(rec.x);
                rec.y = __builtin_amdgcn_readfirstlane(rec.y);
                have_state = rec.x != 0;
                if (have_state) {
                    load_q_early();
                    load_state(sw);
                }
            }
            const int b0 = min(max(rec.y, 0), nblk);
            const int b1 = a.k_hi == INT_MAX ? nblk : b0 + lower_bound_near(blist + b0, nblk - b0, a.k_hi, lane);
            b_next = b1;
            blist += b0;
            nblk = b1 - b0;
            if (!final_) ncol = 0;
            if (!final_ && nblk < kMinPhaseTiles) {     // too little here: leave it to the next phase
                if (first && tid == 0) *phase_rec = make_int2(0, 0);
                return;
            }
        }
        if (!q_loaded) load_q();
    }
    // an even number of chunks (column chunks padded with an empty one), so
    // that the steps come in pairs
    const int nchunk = 2 * (nblk + (ncol + kBK - 1) / kBK);

    // where tile t's keys come from (one scalar load per block tile), and the
    // chunk of it in half hf
    // grouped walk: the hole at or after the current tile (hx, hy), the hole
    // after it (nx, ny) and the first column not before the tile (cv, at
    // index cp), each read from LDS one use ahead so that a tile touching a
    // hole rarely waits for a read; calls come with t non-decreasing
    // (The prefetched values stay as loaded, in vector registers, and become
    // uniform only where they are used, so the LDS read is waited for there.)
    int hp = 0, cp = 0, hx = INT_MAX, hy = INT_MAX, nxv = INT_MAX, nyv = INT_MAX, cvv = INT_MAX;
    auto hole_at = [&](int j, int &x, int &y) {
        x = j < nhole ? __builtin_amdgcn_readfirstlane(glist[wave][2 * j]) : INT_MAX;
        y = j < nhole ? __builtin_amdgcn_readfirstlane(glist[wave][2 * j + 1]) : INT_MAX;
    };
    auto hole_ahead = [&](int j) {
        nxv = j < nhole ? glist[wave][2 * j] : INT_MAX;
        nyv = j < nhole ? glist[wave][2 * j + 1] : INT_MAX;
    };
    auto col_ahead = [&](int c) { cvv = c < ncl_g ? glist[wave][2 * kGrpHoles + c] : INT_MAX; };
    auto col_at = [&](int c) {
        return c < ncl_g ? __builtin_amdgcn_readfirstlane(glist[wave][2 * kGrpHoles + c]) : INT_MAX;
    };
    if constexpr (kGrp) {
        hole_at(0, hx, hy);
        hole_ahead(1);
        col_ahead(0);
    }
    using Src = typename std::conditional<kExact, ExactSrc, ChunkSrc>::type;
    auto tile_of = [&](int t) {
        Src s;
        s.is_col = t >= nblk;
        if constexpr (kFused) s.base = s.is_col ? 0 : __builtin_amdgcn_readfirstlane(fblk[t]);
        else s.base = s.is_col ? 0 : (kDense ? t * kBK : load_uniform(blist + t));
        s.c0 = s.is_col ? (t - nblk) * kBK : 0;
        s.fast = !s.is_col && s.base >= 0 && s.base <= n32 - kBK;
        s.masked = !s.fast || s.base + kBK - 1 > r0;
        s.causal = s.masked;
        s.allow = ~0ull;
        if constexpr (kExact) {
            if (!s.is_col) {
                // the tile's offsets qrow - key span [r0 - base - 63, r0 + 63 - base]:
                // five words from the one holding the lowest; its keys: three words
                const uint32_t *sb = a.ex_s + (int64_t)h * a.ex_words;
                const uint32_t *vb = a.ex_v + (int64_t)h * a.ex_words;
                const int lo = r0 - s.base - 63;
                const int w0 = lo >= 0 ? lo >> 5 : -((31 - lo) >> 5);          // floor(lo / 32)
                s.sbase = 32 * w0;
                auto word = [&](const uint32_t *bits, int i) {
                    return i >= 0 && i < a.ex_words ? (uint32_t)load_uniform(reinterpret_cast<const int32_t *>(bits + i))
                                                    : 0u;
                };
                s.sx0 = word(sb, w0);
                s.sx1 = word(sb, w0 + 1);
                s.sx2 = word(sb, w0 + 2);
                s.sx3 = word(sb, w0 + 3);
                s.sx4 = word(sb, w0 + 4);
                const int v0 = s.base >> 5;                                       // base >= 0
                s.vbase = 32 * v0;
                s.vx0 = word(vb, v0);
                s.vx1 = word(vb, v0 + 1);
                s.vx2 = word(vb, v0 + 2);
                s.masked = true;
            }
        }
        if constexpr (kGrp) {
            const int t0 = t * kBK;
            while (hy <= t0) {
                ++hp;
                hx = __builtin_amdgcn_readfirstlane(nxv);
                hy = __builtin_amdgcn_readfirstlane(nyv);
                hole_ahead(hp + 1);
            }
            if (hx < t0 + kBK) {                            // some hole reaches into the tile
                uint64_t cut = 0;
                int j = hp, x = hx, y = hy;
                while (x < t0 + kBK) {
                    const int lo = max(x, t0) - t0, len = min(y, t0 + kBK) - t0 - lo;
                    cut |= len >= 64 ? ~0ull : ((1ull << len) - 1) << lo;
                    if (y > t0 + kBK) break;
                    ++j;
                    if (j == hp + 1) {
                        x = __builtin_amdgcn_readfirstlane(nxv);
                        y = __builtin_amdgcn_readfirstlane(nyv);
                    } else {
                        hole_at(j, x, y);
                    }
                }
                int cv = __builtin_amdgcn_readfirstlane(cvv);
                if (cv < t0) {
                    do cv = col_at(++cp);
                    while (cv < t0);
                    col_ahead(cp);
                }
                for (int c = cp, key = cv; key < t0 + kBK; key = col_at(++c)) cut &= ~(1ull << (key - t0));
                s.allow = ~cut;
                s.masked = true;
            }
        }
        return s;
    };
    auto half_of = [](Src s, int hf) {
        s.base += 32 * hf;
        s.c0 += 32 * hf;
        s.allow >>= 32 * hf;
        return s;
    };
    // start K of chunk c (and record a column chunk's keys for its mask)
    CopyLanes<T, kH> cl;
    cl.init(lane, wave);
    const uint32_t lds_k = lds_addr(st.k) + wave * CopyLanes<T, kH>::kRpw * Geo<T>::kRowBytes;
    const uint32_t lds_v = lds_addr(st.v) + wave * CopyLanes<T, kH>::kRpw * Geo<T>::kRowBytes;
    auto start_k = [&](int c, const ChunkSrc &s) {
        if (!s.fast && s.is_col && tid < 32) st.kidx[c & 3][tid] = s.c0 + tid < ncol ? clist[s.c0 + tid] : -1;
        load_chunk<T, kH, false>(cl, lds_k, kp, s, c & 1, wave, n32, clist, ncol, nullptr);
    };
    auto start_v = [&](int c, const ChunkSrc &s) {
        load_chunk<T, kH, true>(cl, lds_v, vp, s, c & 1, wave, n32, clist, ncol, st.kidx[c & 3]);
    };

    if constexpr (kDense) load_q();
    // Q has landed.  A compiler-visible wait: otherwise the compiler places its
    // waits for these loads inside the chunk loop, where they would also wait
    // for the K/V copies in flight.
    __builtin_amdgcn_s_waitcnt(kVmcnt0);

    // S(c) = K(c) Q^T for the 32 keys of the chunk in K half c % 2
    auto qk = [&](int c, f32x16 &s) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) E::mma(s, k_frag<T>(st, c & 1, dk, l32, hl), qf[dk]);
    };
    // O^T += V(c)^T P(c) for the chunk in V half c % 2
    auto pv = [&](int c, const frag (&p)[2]) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) E::mma(o[dt], v_frag<T>(st, dt, 2 * (c & 1) + kk, lane), p[kk]);
    };
    // mask: the key must exist and satisfy j <= i (keys past the end of the
    // sequence are > i, column padding is -1).  Lane value jj*4+i of S^T is
    // chunk key jj*8 + hl*4 + i.
    auto mask = [&](int c, const Src &cs, f32x16 &s) {
        if (!cs.masked) return;
        if (cs.is_col) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int4 kk = *reinterpret_cast<const int4 *>(&st.kidx[c & 3][jj * 8 + hl * 4]);
                const int kx[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!(kx[i] >= 0 && kx[i] <= qrow)) s[jj * 4 + i] = -INFINITY;
            }
        } else {
            // e allowed iff 0 <= base + e <= qrow
            if (cs.causal) {
            const int hi = min(max(qrow - cs.base, -1), 32);
            const int lo = min(max(-cs.base, 0), 32);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = jj * 8 + hl * 4 + i;
                    if (e > hi || e < lo) s[jj * 4 + i] = -INFINITY;
                }
            }
            if constexpr (kExact) {
                // key base + e is allowed iff its offset from the row is a
                // selected diagonal or it is a selected column.  x: the
                // offset bits from qrow - base - 31 up, bit 31 - e for key e
                const int rel = qrow - cs.base - 31 - cs.sbase;                 // 0 .. 126
                const int w = rel >> 5;
                // the words as scalar values first (a select between fields
                // of one struct would otherwise become an indexed load from
                // scratch memory)
                const uint32_t x0 = __builtin_amdgcn_readfirstlane(cs.sx0), x1 = __builtin_amdgcn_readfirstlane(cs.sx1),
                               x2 = __builtin_amdgcn_readfirstlane(cs.sx2), x3 = __builtin_amdgcn_readfirstlane(cs.sx3),
                               x4 = __builtin_amdgcn_readfirstlane(cs.sx4);
                const uint32_t lo = w == 0 ? x0 : w == 1 ? x1 : w == 2 ? x2 : x3;
                const uint32_t hi = w == 0 ? x1 : w == 1 ? x2 : w == 2 ? x3 : x4;
                const uint32_t x = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)(rel & 31));
                const int vr = cs.base - cs.vbase;                              // 0 .. 63, uniform
                const uint32_t vlo = vr < 32 ? cs.vx0 : cs.vx1, vhi = vr < 32 ? cs.vx1 : cs.vx2;
                const uint32_t cols = __builtin_amdgcn_alignbit(vhi, vlo, (uint32_t)(vr & 31));
                // lane value jj*4+i is key jj*8 + hl*4 + i: bit jj*8+i of m
                const uint32_t m = (__builtin_bitreverse32(x) | cols) >> (4 * hl);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (((m >> (jj * 8 + i)) & 1u) == 0) s[jj * 4 + i] = -INFINITY;
            }
            if constexpr (kGrp) {
                const uint32_t al = (uint32_t)cs.allow;     // keys base .. base+31 of the chunk
                if (al != ~0u) {
                    // score jj*4+i is key jj*8+i in lanes 0-31 and key
                    // jj*8+4+i in lanes 32-63: one select per score under a
                    // 64-bit lane mask built from the two bits on the scalar unit
                    const float ninf = -INFINITY;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t lo = __builtin_amdgcn_readfirstlane(0u - ((al >> (jj * 8 + i)) & 1u));
                            const uint32_t hi = __builtin_amdgcn_readfirstlane(0u - ((al >> (jj * 8 + 4 + i)) & 1u));
                            s[jj * 4 + i] = lane_select(ninf, s[jj * 4 + i], ((uint64_t)hi << 32) | lo);
                        }
                }
            }
        }
    };
    // online softmax of S(c) -> P(c); returns the factor for O (1 if no row
    // maximum moved in this wave)
    auto softmax = [&](f32x16 &s, frag (&p)[2], float &alpha, bool &moved) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
        mx = pair32_max(mx);
        const float mb_new = fmaxf(mb_i, mx * a.scale_log2);
        const float ref = (mb_new == -INFINITY) ? 0.f : mb_new;
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float e = __builtin_amdgcn_exp2f(fmaf(s[i], a.scale_log2, -ref));
            s[i] = e;
            rs += e;
        }
        moved = __builtin_amdgcn_ballot_w64(mb_new != mb_i) != 0;
        alpha = moved ? __builtin_amdgcn_exp2f(mb_i - ref) : 1.f;
        l_i = l_i * alpha + rs;
        mb_i = mb_new;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            float tmp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) tmp[e] = s[8 * kk + e];
            p[kk] = Out<T>::frag(tmp);
        }
    };
    // one pipeline step for chunk c (source cs); kn is the source of chunk c+2
    auto step = [&](int c, const Src &cs, const Src &kn, f32x16 &s_cur, f32x16 &s_next,
                    frag (&p_cur)[2], const frag (&p_prev)[2], auto with_pv) {
        vm_wait<0>();                                   // K(c+1), V(c-1) have landed (this wave's part)
        __syncthreads();                                // ... all parts; K(c) and V(c-2) are free
        start_k(c + 2, kn);     // past the end: a copy of the last tile's K, never read
        start_v(c, cs);
        mask(c, cs, s_cur);
        qk(c + 1, s_next);
        float alpha;
        bool moved;
        softmax(s_cur, p_cur, alpha, moved);
        if constexpr (decltype(with_pv)::value) pv(c - 1, p_prev);
        // keep P(c) and the row sum computed here, next to the matrix work of
        // this step (the compiler would otherwise sink them to their use in
        // the next step)
        asm volatile("" ::"v"(p_cur[0]), "v"(p_cur[1]), "v"(l_i));
        if (moved) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
        }
    };

    if (nchunk > 0) {
        const int ntile = nchunk / 2;
        f32x16 sa, sb;
        frag pa[2], pb[2];
        Src cur = tile_of(0);
        Src nxt = tile_of(min(1, ntile - 1));
        start_k(0, half_of(cur, 0));
        start_k(1, half_of(cur, 1));
        vm_wait<0>();
        __syncthreads();
        qk(0, sa);
        // tile 0: no PV yet in its first step
        {
            const Src after = tile_of(min(2, ntile - 1));
            step(0, half_of(cur, 0), half_of(nxt, 0), sa, sb, pa, pb, std::false_type{});
            step(1, half_of(cur, 1), half_of(nxt, 1), sb, sa, pb, pa, std::true_type{});
            cur = nxt;
            nxt = after;
        }
        for (int t = 1; t < ntile; ++t) {
            const Src after = tile_of(min(t + 2, ntile - 1));          // needed one pair later
            step(2 * t, half_of(cur, 0), half_of(nxt, 0), sa, sb, pa, pb, std::true_type{});
            step(2 * t + 1, half_of(cur, 1), half_of(nxt, 1), sb, sa, pb, pa, std::true_type{});
            cur = nxt;
            nxt = after;
        }
        vm_wait<0>();                                   // V of the last chunk
        __syncthreads();
        pv(nchunk - 1, pb);
    }

    if (!final_) {
#pragma unroll
        for (int v4 = 0; v4 < 16; ++v4)
            *reinterpret_cast<float4 *>(sw + (v4 * 64 + lane) * 4) =
                make_float4(o[v4 >> 2][(v4 & 3) * 4 + 0], o[v4 >> 2][(v4 & 3) * 4 + 1],
                            o[v4 >> 2][(v4 & 3) * 4 + 2], o[v4 >> 2][(v4 & 3) * 4 + 3]);
        sw[4096 + lane] = mb_i;
        sw[4096 + 64 + lane] = l_i;
        if (tid == 0) {
            if constexpr (kFused) {
                *phase_rec = make_int2(1 | (fcol_next << 1), b_next);
                a.fused_cov[(int64_t)h * nqb + b] = fcov_next;
            } else {
                *phase_rec = make_int2(1, b_next);
            }
        }
        return;
    }
    // finalise: lanes l and l^32 hold halves of the same row's sum
    const float l_tot = pair32_sum(l_i);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow >= n32) return;                            // rows past the end of a short last block
    T *op = reinterpret_cast<T *>(a.out) + ((int64_t)hs * a.stride + span.row0 + qrow) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int d0 = dt * 32 + jj * 8 + hl * 4;
            Out<T>::four(op + d0, o[dt][jj * 4 + 0] * inv, o[dt][jj * 4 + 1] * inv,
                         o[dt][jj * 4 + 2] * inv, o[dt][jj * 4 + 3] * inv);
        }
    if (a.lse != nullptr && hl == 0)
        a.lse[(int64_t)hs * a.stride + span.row0 + qrow] = l_tot > 0.f ? (mb_i * kLn2 + logf(l_tot)) : -INFINITY;
#endif
}

template <typename T, bool kDense, int kH, bool kGrp = false, bool kFused = false, bool kExact = false,
          bool kVar = false>
hipError_t launch_h(const AttnArgs &a, hipStream_t s) {
    const int64_t total = (int64_t)a.hq * a.vl.nseq / kH * ((a.n + kBQ - 1) / kBQ - (kDense ? 0 : a.qb_lo));
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL((attn_fwd_kernel<T, kDense, kH, kGrp, kFused, kExact, kVar>), dim3((unsigned)total),
                       dim3(kThreads * kH), 0, s, a);
    return hipGetLastError();
}

__global__ void clear_words_kernel(uint32_t *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// The exact union mask's bitmaps: selected offsets and selected column keys
// of each q head (entries outside [0, n) select nothing), set on cleared words.
__global__ void exact_bits_kernel(const int32_t *v_idx, int32_t kv, const int32_t *s_idx, int32_t ks, int32_t hq,
                                  int64_t n, int32_t words, uint32_t *ex_s, uint32_t *ex_v) {
    const int64_t per = (int64_t)kv + ks, total = per * hq;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t h = e / per, r = e % per;
        const int32_t x = r < kv ? v_idx[h * kv + r] : s_idx[h * ks + (r - kv)];
        if (x < 0 || x >= n) continue;
        uint32_t *bits = (r < kv ? ex_v : ex_s) + h * words;
        atomicOr(bits + (x >> 5), 1u << (x & 31));
    }
}

hipError_t clear_words(uint32_t *p, int64_t words, hipStream_t s) {
    if (words <= 0) return hipSuccess;
    const int64_t blocks = (words + 255) / 256 < 65536 ? (words + 255) / 256 : 65536;
    hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, words);
    return hipGetLastError();
}

// Fused mode: no grouped walk (there are no lists to qualify), the key phases
// of the per-head kernel each walking its part of the cover.  The exact
// union mask's bitmaps follow the phase state and column bitmaps in ws.
template <typename T, bool kExact> hipError_t launch_fused(AttnArgs a, hipStream_t s) {
    const int64_t R = a.phase_keys;
    const bool phases = a.ws != nullptr && R > 0 && R < a.n;
    a.grp = nullptr;
    if constexpr (kExact) {
        a.ex_words = (int32_t)((a.n + 31) / 32);
        uint32_t *bits = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(a.ws) +
                                                      (phases ? fused_state_bytes(a.hq, a.n, R, a.kv, false) : 0));
        a.ex_s = bits;
        a.ex_v = bits + (int64_t)a.hq * a.ex_words;
        hipError_t e = clear_words(bits, 2 * (int64_t)a.hq * a.ex_words, s);
        if (e != hipSuccess) return e;
        const int64_t total = ((int64_t)a.kv + a.ks) * a.hq;
        if (total > 0) {
            const int64_t blocks = (total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096;
            hipLaunchKernelGGL(exact_bits_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.v_idx, a.kv, a.s_idx,
                               a.ks, a.hq, a.n, a.ex_words, bits, bits + (int64_t)a.hq * a.ex_words);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    if (!phases) {
        a.ws = nullptr;
        a.k_lo = INT_MIN;
        a.k_hi = INT_MAX;
        a.qb_lo = 0;
        return launch_h<T, false, 1, false, true, kExact>(a, s);
    }
    a.fused_cov = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(a.ws) + sparse_walk_marks_offset(a.hq, a.n));
    a.fused_cw = (a.kv + 31) / 32;
    a.fused_cols = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(a.ws) + sparse_state_bytes(a.hq, a.n, R));
    {
        const hipError_t e = clear_words(a.fused_cols, (int64_t)a.hq * ((a.n + kBQ - 1) / kBQ) * a.fused_cw, s);
        if (e != hipSuccess) return e;
    }
    const int64_t np = (a.n + R - 1) / R;
    for (int64_t j = 0; j < np; ++j) {
        a.k_lo = j == 0 ? INT_MIN : (int32_t)(j * R);
        a.k_hi = j == np - 1 ? INT_MAX : (int32_t)((j + 1) * R);
        a.qb_lo = j * R / kBQ;
        const hipError_t e = launch_h<T, false, 1, false, true, kExact>(a, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Sparse: one q head per workgroup (each head has its own work lists).  Dense:
// up to four q heads of a kv group per workgroup, sharing every K/V tile.
// Sparse in phases: launch j covers the keys [j R, (j+1) R) for the query
// blocks from j R / 64 on, so the workgroups in flight read K/V from one
// R-key range of a kv head (a working set the last-level cache holds) rather
// than from the whole sequence.
template <typename T, bool kDense, bool kVar = false> hipError_t launch(AttnArgs a, hipStream_t s) {
    if constexpr (kDense) {
        const int G = a.hq / a.hkv;
        if (G % 4 == 0) return launch_h<T, true, 4, false, false, false, kVar>(a, s);
        if (G % 2 == 0) return launch_h<T, true, 2, false, false, false, kVar>(a, s);
        return launch_h<T, true, 1, false, false, false, kVar>(a, s);
    } else {
        const int64_t R = a.phase_keys;
        if (a.ws == nullptr || R <= 0 || R >= a.n) {
            a.ws = nullptr;
            a.k_lo = INT_MIN;
            a.k_hi = INT_MAX;
            a.qb_lo = 0;
            return launch_h<T, false, 1, false, false, false, kVar>(a, s);
        }
        // first the grouped walk over the units that qualify (it marks them),
        // then the key phases of the per-head kernel over the rest
        a.grp = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(a.ws) +
                                            sparse_walk_marks_offset((int64_t)a.hq * a.vl.nseq, a.n));
        a.grp_kh = walk_heads_per_unit(a.hq, a.hkv);
        {
            const hipError_t e = a.grp_kh == 4   ? launch_h<T, true, 4, true, false, false, kVar>(a, s)
                                 : a.grp_kh == 2 ? launch_h<T, true, 2, true, false, false, kVar>(a, s)
                                                 : launch_h<T, true, 1, true, false, false, kVar>(a, s);
            if (e != hipSuccess) return e;
        }
        const int64_t np = (a.n + R - 1) / R;
        for (int64_t j = 0; j < np; ++j) {
            a.k_lo = j == 0 ? INT_MIN : (int32_t)(j * R);
            a.k_hi = j == np - 1 ? INT_MAX : (int32_t)((j + 1) * R);
            a.qb_lo = j * R / kBQ;
            const hipError_t e = launch_h<T, false, 1, false, false, false, kVar>(a, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
}

}  // namespace

size_t sparse_walk_marks_offset(int64_t hq, int64_t n) {
    return (size_t)hq * (size_t)((n + kBQ - 1) / kBQ) * (2 * kStateFloats * sizeof(float) + sizeof(int2));
}

int walk_heads_per_unit(int hq, int hkv) {
    const int G = hq / hkv;
    return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
}

size_t sparse_state_bytes(int64_t hq, int64_t n, int64_t phase_keys) {
    if (phase_keys <= 0 || phase_keys >= n) return 0;
    return (size_t)hq * (size_t)((n + kBQ - 1) / kBQ) * (2 * kStateFloats * sizeof(float) + sizeof(int2) + sizeof(int32_t));
}

size_t fused_state_bytes(int64_t hq, int64_t n, int64_t phase_keys, int64_t kv, bool exact) {
    const size_t state = sparse_state_bytes(hq, n, phase_keys);
    size_t bytes = 0;
    if (state != 0) bytes = state + (size_t)hq * (size_t)((n + kBQ - 1) / kBQ) * (size_t)((kv + 31) / 32) * sizeof(uint32_t);
    if (exact) bytes += 2 * (size_t)hq * (size_t)((n + 31) / 32) * sizeof(uint32_t);
    return bytes;
}

hipError_t launch_sparse_prefill(const AttnArgs &a, int dtype, hipStream_t s) {
    if (a.vl.cu != nullptr) return dtype == 0 ? launch<bf16, false, true>(a, s) : launch<float, false, true>(a, s);
    return dtype == 0 ? launch<bf16, false>(a, s) : launch<float, false>(a, s);
}

hipError_t launch_sparse_prefill_fused(const AttnArgs &a, int dtype, bool exact, hipStream_t s) {
    if (exact) return dtype == 0 ? launch_fused<bf16, true>(a, s) : launch_fused<float, true>(a, s);
    return dtype == 0 ? launch_fused<bf16, false>(a, s) : launch_fused<float, false>(a, s);
}

int fused_max_phase_keys() { return kFusedMaxPhase; }
int fused_max_columns() { return kFusedCols; }

hipError_t launch_dense_prefill(const AttnArgs &a, int dtype, hipStream_t s) {
    if (a.vl.cu != nullptr) return dtype == 0 ? launch<bf16, true, true>(a, s) : launch<float, true, true>(a, s);
    return dtype == 0 ? launch<bf16, true>(a, s) : launch<float, true>(a, s);
}

}  // namespace msa
