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
// serving q head g*G + w (+4, ...).  K tiles (64 keys) stream HBM -> LDS with
// direct copies, double buffered, and are shared by the G q heads of the group.
//   pass 1 (S^T = K Q^T, lane = query row, 16 keys per lane and sub-tile):
//           per-row running max (kept as scale*log2(e)*z) and sum of exp2
//           over the range -> partials
//   combine: partials -> per-row log2 normaliser  m_r + log2(l_r)
//   pass 2 (S = Q K^T, lane = key, 16 query rows per lane and sub-tile):
//           p = exp2(scale*log2(e)*z - normaliser).  Column sums v stay in
//           registers.  For the diagonal sums, each wave writes its 32 x 64
//           block of p into LDS skewed, row r shifted by -r, so that a diagonal
//           becomes a column; cells outside the written parallelogram are zero
//           from the start and never written, so the column reads need no
//           bounds tests.  A diagonal spans at most two adjacent tiles: inside
//           a range the carry is kept in a register, across ranges the two
//           partial sums go to the workspace and a fix-up kernel adds them.
//           No floating-point atomics: results are deterministic.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace msa {
namespace {

constexpr int kD = 128;
constexpr int kL = 64;           // last_q
constexpr int kTK = 64;          // keys per tile
constexpr int kThreads = 256;    // four waves
constexpr int kSkew = 95;        // skewed p block: 32 rows x 95 columns (row pitch)

// K tile geometry: rows of kRowBytes, 1 KB copy slots, 16-byte chunks XOR
// swizzled per row (bf16) so that the MFMA operand reads (rows r..r+15 at one
// logical chunk) are free of bank conflicts.
template <typename T> struct KGeo {
    static constexpr int kRowBytes = kD * (int)sizeof(T);
    static constexpr int kChunks = kRowBytes / 16;
    static constexpr int kTileBytes = kTK * kRowBytes;
    static constexpr int kRowsPerSlot = 1024 / kRowBytes;
    static constexpr int kPer = kTileBytes / 1024 / 4;           // copies per lane (4 waves)
    __device__ static __forceinline__ int swz(int row) { return sizeof(T) == 2 ? (row & 15) : 0; }
};

template <typename T> struct EstSmem {
    alignas(16) unsigned char k[2][KGeo<T>::kTileBytes];
};

// Start the copy of the 64-key tile at `base` into LDS buffer `buf`: wave w
// moves rows 16w .. 16w+15 (kPer 1 KB slots).
template <typename T>
__device__ __forceinline__ void start_tile(unsigned char *buf, const T *kp, int64_t base, int wave,
                                           const uint32_t (&off)[KGeo<T>::kPer]) {
    using Gm = KGeo<T>;
    const char *tb = reinterpret_cast<const char *>(kp) + (base + wave * 16) * Gm::kRowBytes;
    const uint32_t l0 = lds_addr(buf) + wave * 16 * Gm::kRowBytes;
#pragma unroll
    for (int i = 0; i < Gm::kPer; i += 4) dma_x4(tb, off[i], off[i + 1], off[i + 2], off[i + 3], l0 + i * 1024);
}

// The copy of the frame tile at vbase (frame keys vbase .. vbase+63 are
// sequence keys vbase - pad ..): a tile reaching before key 0 (the first one
// when pad > 0) reads key 0 for the missing rows, whose scores are masked.
template <typename T>
__device__ __forceinline__ void start_frame_tile(unsigned char *buf, const T *kp, int64_t vbase, int pad,
                                                 int wave, const uint32_t (&off)[KGeo<T>::kPer], int lane) {
    using Gm = KGeo<T>;
    const int64_t rbase = vbase - pad;
    if (rbase >= 0) {
        start_tile<T>(buf, kp, rbase, wave, off);
        return;
    }
    const char *rows = reinterpret_cast<const char *>(kp);
    const int sub = lane / Gm::kChunks;
    const uint32_t l0 = lds_addr(buf) + wave * 16 * Gm::kRowBytes;
    const char *ad[Gm::kPer];
#pragma unroll
    for (int i = 0; i < Gm::kPer; ++i) {
        const int r = i * Gm::kRowsPerSlot + sub;                     // row of this wave's 16
        const int64_t row = max(rbase + wave * 16 + r, (int64_t)0);
        ad[i] = rows + row * Gm::kRowBytes + (off[i] - (uint32_t)(r * Gm::kRowBytes));
    }
#pragma unroll
    for (int i = 0; i < Gm::kPer; i += 4) dma_x4(ad[i], ad[i + 1], ad[i + 2], ad[i + 3], l0 + i * 1024);
}

template <typename T>
__device__ __forceinline__ void copy_offsets(uint32_t (&off)[KGeo<T>::kPer], int lane) {
    using Gm = KGeo<T>;
    const int sub = lane / Gm::kChunks, phys = lane % Gm::kChunks;
#pragma unroll
    for (int i = 0; i < Gm::kPer; ++i) {
        const int r = i * Gm::kRowsPerSlot + sub;          // rows 16w + r share the swizzle of r
        off[i] = (uint32_t)(r * Gm::kRowBytes + ((phys ^ Gm::swz(r)) << 4));
    }
}

// K fragment of tile rows kt*32 + l32, d = dk*16 + hl*8 .. +7
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag k_frag(const unsigned char *buf, int kt, int dk, int l32, int hl) {
    using Gm = KGeo<T>;
    const int row = kt * 32 + l32;
    const int c = (dk * 16 + hl * 8) * (int)sizeof(T) / 16;
    if constexpr (sizeof(T) == 2) {
        return Elem<T>::load_frag(buf + row * Gm::kRowBytes + ((c ^ Gm::swz(row)) << 4));
    } else {
        return Elem<T>::load_frag(buf + row * Gm::kRowBytes + c * 16);
    }
}

// Number of q heads waves serve per pass over the key range.
__device__ __forceinline__ int n_slots(int G) { return (G + 3) / 4; }

// One sequence's frame: its first row, keys, frame keys (keys rounded up to
// 64), frame shift and key ranges.  A packed batch shares the range length;
// its per-head arrays hold the longest sequence's nranges and n per head.
struct EstGeom {
    int64_t row0, n, nv;
    int pad, nranges;
};
__device__ __forceinline__ EstGeom est_geom(const EstArgs &a, int seq) {
    if (a.vl.cu == nullptr) return EstGeom{0, a.n, a.nv, a.pad, a.nranges};
    const SeqSpan sp = seq_span(a.vl.cu, seq, a.vl.rows, a.n);
    EstGeom e;
    e.row0 = sp.row0;
    e.n = sp.n;
    e.nv = (sp.n + kTK - 1) / kTK * kTK;
    e.pad = (int)(e.nv - e.n);
    e.nranges = (int)((e.nv + a.range_keys - 1) / a.range_keys);
    return e;
}

template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void est_pass1_kernel(EstArgs a) {
    using E = Elem<T>;
    using Gm = KGeo<T>;
    __shared__ EstSmem<T> sm;
    const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int range = blockIdx.x, seq = blockIdx.y / a.hkv, g = blockIdx.y % a.hkv;
    const int G = a.hq / a.hkv;
    const EstGeom gm = est_geom(a, seq);
    if (gm.n == 0 || range >= gm.nranges) return;      // an empty packed sequence, or past its keys
    const int64_t n = gm.n, nv = gm.nv;                 // sequence keys, frame keys
    const int pad = gm.pad;
    const int64_t k0 = (int64_t)range * a.range_keys;   // frame keys of this range
    const int64_t k1 = min(nv, k0 + a.range_keys);
    const int ntile = (int)((k1 - k0) / kTK);
    const T *kp = reinterpret_cast<const T *>(a.k) + ((int64_t)g * a.stride + gm.row0) * kD;
    uint32_t off[Gm::kPer];
    copy_offsets<T>(off, lane);
    for (int slot = 0; slot < n_slots(G); ++slot) {
        const int hw = wave + 4 * slot;
        const bool active = hw < G;
        const int h = g * G + (active ? hw : 0);
        const int64_t vh = (int64_t)seq * a.hq + h;     // the head in the per-head arrays
        const T *qp = reinterpret_cast<const T *>(a.q) + ((int64_t)h * a.stride + gm.row0) * kD;
        typename E::frag qf[2][8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            // window row half*32 + l32 is sequence row n - 64 + that; in a
            // sequence shorter than the window the rows before its start read
            // row 0, and every key of theirs is masked
            const int64_t qr = max(n - kL + half * 32 + l32, (int64_t)0);
#pragma unroll
            for (int dk = 0; dk < 8; ++dk) qf[half][dk] = E::load_frag(qp + qr * kD + dk * 16 + hl * 8);
        }
        __builtin_amdgcn_s_waitcnt(kVmcnt0);        // Q has landed (compiler-visible wait)
        float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
        __syncthreads();                            // the previous slot is done with both buffers
        start_frame_tile<T>(sm.k[0], kp, k0, pad, wave, off, lane);
        for (int t = 0; t < ntile; ++t) {
            const int64_t base = k0 + (int64_t)t * kTK;
            vm_wait<0>();
            __syncthreads();                        // tile t visible; tile t-1's buffer is free
            // tiles after a range's first start at frame key 64 or later: all rows exist
            if (t + 1 < ntile) start_tile<T>(sm.k[(t + 1) & 1], kp, base + kTK - pad, wave, off);
            if (!active) continue;
            const unsigned char *buf = sm.k[t & 1];
            const bool last = base + kTK > nv - kL;  // keys past some p_r
            const bool before = base < pad;         // frame keys before key 0
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x16 s[2];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
                    for (int dk = 0; dk < 8; ++dk) E::mma(s[kt], k_frag<T>(buf, kt, dk, l32, hl), qf[half][dk]);
                }
                if (last || before) {
                    const int64_t prow = nv - kL + half * 32 + l32;
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int64_t key = base + kt * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
                            if (key > prow || key < pad) s[kt][i] = -INFINITY;
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
                float acc = l[half] * __builtin_amdgcn_exp2f(m[half] - ref);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc += __builtin_amdgcn_exp2f(fmaf(s[kt][i], a.scale_log2, -ref));
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
                const float lt = l[half] * __builtin_amdgcn_exp2f(m[half] - ref) + lo * __builtin_amdgcn_exp2f(mo - ref);
                if (hl == 0) {
                    const int64_t o = (vh * kL + half * 32 + l32) * a.nranges + range;
                    a.part_m[o] = mn;
                    a.part_l[o] = lt;
                }
            }
        }
    }
}

// One wave per (q head, row): merge the per-range (max, sum) partials into the
// row's log2 normaliser m + log2(l) (scaled log2 units), so that
// p = exp2(scale*log2(e)*z - normaliser).
__global__ __launch_bounds__(256) void est_combine_kernel(EstArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (int64_t)a.vl.nseq * a.hq * kL) return;
    const EstGeom gm = est_geom(a, (int)(row / kL / a.hq));
    if (gm.n == 0) return;
    const float *pm = a.part_m + row * a.nranges;
    const float *pl = a.part_l + row * a.nranges;
    float m = -INFINITY, l = 0.f;
    for (int i = lane; i < gm.nranges; i += 64) {
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
    // a window row has at least one key (l > 0) unless it lies before the
    // start of a sequence shorter than the window: -inf, and its p is masked
    if (lane == 0) a.row_norm[row] = m + log2f(l);
}

// Pass 2: eight waves, two per q head; wave 2k + hf holds query rows 32 hf ..
// 32 hf + 31 of head slot k (a wave's Q fragments and normalisers then fit in
// half the registers, which gives two waves per SIMD).  The half-1 wave passes
// its column and diagonal partials of tile t to the half-0 wave through LDS
// (double buffered by tile parity); the half-0 wave adds them after the next
// tile's barrier and writes the scores.
constexpr int kThreads2 = 512;
template <typename T> struct Pass2Smem {
    static constexpr int kKBuf = sizeof(T) == 2 ? 2 : 1;     // fp32 tiles: single buffer (LDS size)
    alignas(16) unsigned char k[kKBuf][KGeo<T>::kTileBytes];
    float p[8][32 * kSkew];                                    // per-wave skewed p block
    float x[2][4][3][64];                                      // half-1 partials: v, D1, D2
};

template <typename T>
__global__ __launch_bounds__(kThreads2) void est_pass2_kernel(EstArgs a) {
    using E = Elem<T>;
    using Gm = KGeo<T>;
    using Sm = Pass2Smem<T>;
    __shared__ Sm sm;
    const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hs = wave >> 1, hf = wave & 1;                    // head slot, row half
    const int range = blockIdx.x, seq = blockIdx.y / a.hkv, g = blockIdx.y % a.hkv;
    const int G = a.hq / a.hkv;
    const EstGeom gm = est_geom(a, seq);
    if (gm.n == 0 || range >= gm.nranges) return;              // as in pass 1
    const int64_t n = gm.n, nv = gm.nv;                        // sequence keys, frame keys
    const int pad = gm.pad;
    const int64_t k0 = (int64_t)range * a.range_keys;           // frame keys of this range
    const int64_t k1 = min(nv, k0 + a.range_keys);
    const int ntile = (int)((k1 - k0) / kTK);
    const T *kp = reinterpret_cast<const T *>(a.k) + ((int64_t)g * a.stride + gm.row0) * kD;
    const bool loader = wave < 4;                               // waves 0-3 copy the K tiles
    uint32_t off[Gm::kPer];
    copy_offsets<T>(off, lane);
    float *pw = sm.p[wave];
    // Skewed block: p of (row r, key e) at pw[r*kSkew + e - r + 31]; the cells
    // never written (outside the parallelogram) stay zero.
    for (int i = lane; i < 32 * kSkew; i += 64) pw[i] = 0.f;
    // Lane t owns the tile diagonals D1 = t - 63 and D2 = t + 1 (D = R - e for
    // global row R = 32 hf + r).  Diagonal D is column 32 hf + 31 - D; a column
    // outside [0, 94] holds no element of this half.
    const int c1 = hf * 32 + 94 - lane, c2 = hf * 32 + 30 - lane;
    const float use1 = (c1 >= 0 && c1 <= 94) ? 1.f : 0.f, use2 = (c2 >= 0 && c2 <= 94) ? 1.f : 0.f;
    const int col1 = min(max(c1, 0), 94), col2 = min(max(c2, 0), 94);
    for (int slot = 0; slot < n_slots(G); ++slot) {
        const int hw = hs + 4 * slot;
        const bool active = hw < G;
        const int h = g * G + (active ? hw : 0);
        const int64_t vh = (int64_t)seq * a.hq + h;             // the head in the per-head arrays
        const T *qp = reinterpret_cast<const T *>(a.q) + ((int64_t)h * a.stride + gm.row0) * kD;
        // A operand of S = Q K^T: query 32 hf + l32, d = dk*16 + hl*8 + e
        // (rows before the start of a short sequence read row 0, as in pass 1)
        const int64_t qr = max(n - kL + hf * 32 + l32, (int64_t)0);
        typename E::frag qf[8];
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) qf[dk] = E::load_frag(qp + qr * kD + dk * 16 + hl * 8);
        // normaliser of the 16 rows this lane holds: row 32 hf + jj*8 + hl*4 + i at jj*4 + i
        float nrm[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) nrm[x] = a.row_norm[vh * kL + hf * 32 + (x >> 2) * 8 + hl * 4 + (x & 3)];
        __builtin_amdgcn_s_waitcnt(kVmcnt0);        // Q and the normalisers have landed
        float *vout = a.v_score + vh * a.n;                     // rows of the longest sequence's length
        float *sout = a.s_score + vh * a.n;
        float carry = 0.f;
        float v_own = 0.f, d1_own = 0.f, d2_own = 0.f;          // half-0 partials of the pending tile
        // tile t's scores (half-0 wave): add the half-1 partials, write, carry
        auto finish = [&](int t) {
            const float *xs = &sm.x[t & 1][hs][0][0];
            const float vt = v_own + xs[lane];
            const float dg1 = d1_own + xs[64 + lane], dg2 = d2_own + xs[128 + lane];
            const int64_t base = k0 + (int64_t)t * kTK;
            if (base + lane >= pad) vout[base + lane - pad] = vt; // frame key -> sequence key
            const int64_t A = nv - kL - base;                    // offset of diagonal D = 0
            if (lane == 63) {
                sout[A] = dg1;                                   // D = 0 lies in this tile only
            } else {
                const int64_t o2 = A + lane + 1;                 // D = lane + 1
                if (t > 0) {
                    sout[o2] = dg2 + carry;
                } else if (range == 0) {
                    // keys below 0 do not exist; offsets from n on reach no key
                    if (o2 < n) sout[o2] = dg2;
                } else {
                    a.diag_hi[(vh * a.nranges + range) * 64 + lane] = dg2;
                }
                carry = dg1;                                     // D = lane - 63, finished by the next tile
            }
        };
        // scores of tile t for this wave's 32 rows: p into the skewed block, the
        // column sums (lane t: key t) and the two diagonal partials
        auto tile = [&](const unsigned char *buf, int64_t base, auto masked) {
            float vk[2] = {0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                f32x16 sc;
#pragma unroll
                for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
                for (int dk = 0; dk < 8; ++dk) E::mma(sc, qf[dk], k_frag<T>(buf, kt, dk, l32, hl));
                const int e = kt * 32 + l32;                      // key of this lane in the tile
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int r = (x >> 2) * 8 + hl * 4 + (x & 3);
                    float p = __builtin_amdgcn_exp2f(fmaf(sc[x], a.scale_log2, -nrm[x]));
                    if constexpr (decltype(masked)::value)
                        if (base + e > nv - kL + hf * 32 + r || base + e < pad) p = 0.f;
                    vk[kt] += p;
                    pw[r * kSkew + e - r + 31] = p;
                }
            }
            float d1 = 0.f, d2 = 0.f;
#pragma unroll 8
            for (int r = 0; r < 32; ++r) {
                d1 += pw[r * kSkew + col1];
                d2 += pw[r * kSkew + col2];
            }
            // lanes l and l^32 hold the two 16-row halves of each key:
            // v_permlane32_swap(old = vk[0], src = vk[1]) returns lanes 0-31 of
            // vk[0] and of vk[1] in the first result and lanes 32-63 in the
            // second, so lane t gets the 32-row sum of key t
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(vk[0]), __float_as_uint(vk[1]), false, false);
            return f32x4{__uint_as_float(sw[0]) + __uint_as_float(sw[1]), d1 * use1, d2 * use2, 0.f};
        };
        __syncthreads();                            // the previous slot is done with every buffer
        if (loader) start_frame_tile<T>(sm.k[0], kp, k0, pad, wave, off, lane);
        for (int t = 0; t < ntile; ++t) {
            const int64_t base = k0 + (int64_t)t * kTK;
            vm_wait<0>();
            __syncthreads();                        // tile t visible; half-1 partials of t-1 visible
            // tiles after a range's first start at frame key 64 or later: all rows exist
            if (Sm::kKBuf == 2 && loader && t + 1 < ntile) start_tile<T>(sm.k[(t + 1) & 1], kp, base + kTK - pad, wave, off);
            if (active && hf == 0 && t > 0) finish(t - 1);
            if (active) {
                const unsigned char *buf = sm.k[Sm::kKBuf == 2 ? (t & 1) : 0];
                const f32x4 r = (base + kTK > nv - kL || base < pad) ? tile(buf, base, std::true_type{})
                                                                      : tile(buf, base, std::false_type{});
                if (hf == 0) {
                    v_own = r[0];
                    d1_own = r[1];
                    d2_own = r[2];
                } else {
                    float *xs = &sm.x[t & 1][hs][0][0];
                    xs[lane] = r[0];
                    xs[64 + lane] = r[1];
                    xs[128 + lane] = r[2];
                }
            }
            if (Sm::kKBuf == 1) {
                __syncthreads();                    // every wave is done with the single tile buffer
                if (loader && t + 1 < ntile) start_tile<T>(sm.k[0], kp, base + kTK - pad, wave, off);
            }
        }
        __syncthreads();                            // half-1 partials of the last tile
        if (active && hf == 0 && ntile > 0) {
            finish(ntile - 1);
            if (lane < 63 && range != gm.nranges - 1)
                a.diag_lo[(vh * a.nranges + range) * 64 + lane] = carry;
        }
    }
}

// Diagonals that straddle two key ranges: s[o] = hi(range) + lo(range - 1).
__global__ __launch_bounds__(256) void est_fixup_kernel(EstArgs a) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_h = (int64_t)(a.nranges - 1) * 63;
    if (t >= per_h * a.hq * a.vl.nseq) return;
    const int64_t vh = t / per_h;
    const int64_t rem = t % per_h;
    const int range = 1 + (int)(rem / 63);
    const int lane = (int)(rem % 63);
    const EstGeom gm = est_geom(a, (int)(vh / a.hq));
    if (gm.n == 0 || range >= gm.nranges) return;
    const int64_t A = gm.nv - kL - (int64_t)range * a.range_keys;
    const int64_t o = A + lane + 1;                     // below n: range >= 1 starts past frame key 255
    if (o >= gm.n) return;
    a.s_score[vh * a.n + o] = a.diag_hi[(vh * a.nranges + range) * 64 + lane] +
                              a.diag_lo[(vh * a.nranges + range - 1) * 64 + lane];
}

template <typename T> hipError_t launch_t(const EstArgs &a, hipStream_t s) {
    dim3 grid(a.nranges, a.hkv * a.vl.nseq);
    hipLaunchKernelGGL(est_pass1_kernel<T>, grid, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)a.hq * a.vl.nseq * kL;
    hipLaunchKernelGGL(est_combine_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(est_pass2_kernel<T>, grid, dim3(kThreads2), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t fix = (int64_t)(a.nranges - 1) * 63 * a.hq * a.vl.nseq;
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
