// Shared device helpers for the gfx950 kernels: element types, 16-byte
// vector access, and the 32x32 MFMA step used by every contraction here.
//
// MFMA operand convention used throughout (one 32x32 output tile, K chunk 16):
//   A fragment: lane l holds A[row = l%32][k = (l/32)*8 + e], e = 0..7
//   B fragment: lane l holds B[k = (l/32)*8 + e][col = l%32], e = 0..7
//   C/D:        lane l holds C[row = jj*8 + (l/32)*4 + i][col = l%32] in
//               acc[jj*4 + i], jj, i = 0..3.
// Only the row/column placement matters for correctness: A and B use the same
// (lane, e) -> k labelling, so any hardware permutation of k cancels out.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct bf16 { uint16_t x; };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// round-to-nearest-even float -> bfloat16 (inputs here are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Element traits: an MFMA fragment holds 8 consecutive k values.
template <typename T> struct Elem;

template <> struct Elem<bf16> {
    typedef bf16x8 frag;                          // 16 bytes
    static constexpr int kBytes = 2;
    __device__ static __forceinline__ frag load_frag(const void *p) {
        u32x4 r = *reinterpret_cast<const u32x4 *>(p);
        return __builtin_bit_cast(frag, r);
    }
    __device__ static __forceinline__ frag zero_frag() {
        u32x4 z = {0u, 0u, 0u, 0u};
        return __builtin_bit_cast(frag, z);
    }
    // C += A * B over one K chunk of 16
    __device__ static __forceinline__ void mma(f32x16 &c, const frag &a, const frag &b) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ frag from_f32(const float *x) {
        u32x4 r;
        r[0] = pack_bf16x2(x[0], x[1]);
        r[1] = pack_bf16x2(x[2], x[3]);
        r[2] = pack_bf16x2(x[4], x[5]);
        r[3] = pack_bf16x2(x[6], x[7]);
        return __builtin_bit_cast(frag, r);
    }
    __device__ static __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
};

template <> struct Elem<float> {
    typedef f32x8 frag;                           // 32 bytes
    static constexpr int kBytes = 4;
    __device__ static __forceinline__ frag load_frag(const void *p) {
        const f32x4 *q = reinterpret_cast<const f32x4 *>(p);
        f32x4 a = q[0], b = q[1];
        frag r;
        r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
        r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
        return r;
    }
    __device__ static __forceinline__ frag zero_frag() {
        frag r;
        for (int i = 0; i < 8; ++i) r[i] = 0.f;
        return r;
    }
    // Eight K=2 steps: step e contracts k = e (lanes 0-31) and k = 8+e (lanes 32-63).
    __device__ static __forceinline__ void mma(f32x16 &c, const frag &a, const frag &b) {
#pragma unroll
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
    }
    __device__ static __forceinline__ frag from_f32(const float *x) {
        frag r;
        for (int i = 0; i < 8; ++i) r[i] = x[i];
        return r;
    }
};

__device__ __forceinline__ float wave_shfl_xor(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

// Max / sum of a value over the lane pair (l, l ^ 32) in one VALU permute,
// v_permlane32_swap, instead of an LDS permute.  With both operands v, the
// swap returns, in every lane, its own value in one result and its partner's
// in the other, so a symmetric operation over the two results is the pair's.
__device__ __forceinline__ float pair32_max(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- HBM -> LDS copies and wait helpers (gfx950) ----

#define LDS_AS __attribute__((address_space(3)))

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

// Rows of sequence `seq` of a packed batch (cu: device int32 offsets, read
// as scalars; seq wave-uniform): the first row and the length, clamped into
// the rows of a head and to at most nmax.  cu NULL: one sequence of nmax rows.
struct SeqSpan {
    int64_t row0, n;
};
__device__ __forceinline__ SeqSpan seq_span(const int32_t *cu, int seq, int64_t rows, int64_t nmax) {
    if (cu == nullptr) return SeqSpan{0, nmax};
    int64_t a = load_uniform(cu + seq), b = load_uniform(cu + seq + 1);
    a = a < 0 ? 0 : (a > rows ? rows : a);
    b = b < a ? a : (b > rows ? rows : b);
    return SeqSpan{a, b - a < nmax ? b - a : nmax};
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(LDS_AS const unsigned char *)p;
}

__device__ __forceinline__ const void *to_sgpr(const void *p) {   // p is wave-uniform
    const uint64_t u = (uint64_t)(uintptr_t)p;
    return (const void *)(uintptr_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32)) << 32) |
                                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u));
}

// HBM -> LDS copies, 16 bytes per lane (lane l's bytes land at M0 + 16 l), four
// 1 KB copies into consecutive LDS slots from `lds` on.  Issued from inline
// assembly: the compiler does not track these copies, so it never waits for
// them on its own (it would otherwise wait for all of them before any LDS read
// it cannot prove disjoint).  Completion is awaited with vm_wait<N>() (every
// copy but the last N issued has landed), then a barrier.
// M0 holds the LDS destination while a copy issues (the hardware reads it at
// issue).  M0 is a reserved register the compiler may keep values in, so each
// block saves it into a scratch SGPR first and puts it back before it ends:
// the compiler sees M0 unchanged, as it assumes.
// Uniform 64-bit base in SGPRs plus a per-lane 32-bit offset per copy:
__device__ __forceinline__ void dma_x4(const void *sbase, uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3,
                                       uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %6\n\t"
        "global_load_lds_dwordx4 %1, %5\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "global_load_lds_dwordx4 %2, %5\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "global_load_lds_dwordx4 %3, %5\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "global_load_lds_dwordx4 %4, %5\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(to_sgpr(sbase)), "s"(lds)
        : "memory", "scc");
}
// One 1 KB copy (uniform base in SGPRs plus a per-lane offset):
__device__ __forceinline__ void dma_x1(const void *sbase, uint32_t v0, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(v0), "s"(to_sgpr(sbase)), "s"(lds)
        : "memory");
}
// One 1 KB copy from per-lane 64-bit addresses:
__device__ __forceinline__ void dma_x1(const void *a0, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(a0), "s"(lds)
        : "memory");
}
// Per-lane 64-bit addresses:
__device__ __forceinline__ void dma_x4(const void *a0, const void *a1, const void *a2, const void *a3, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %5\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "global_load_lds_dwordx4 %3, off\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "global_load_lds_dwordx4 %4, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "s"(lds)
        : "memory", "scc");
}

// Number of XCDs on MI355X; consecutive workgroup ids are spread round-robin
// over them, and each XCD has its own L2.
constexpr int kNumXcd = 8;

}  // namespace msa
