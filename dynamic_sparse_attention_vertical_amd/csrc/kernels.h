// Launch interfaces between the C-ABI layer (msa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// A packed batch of sequences of different lengths (cu NULL: one sequence of
// the problem's length).  Sequence s holds rows cu[s] .. cu[s+1]-1 of every
// head of q, k, v, out and lse (device int32 [nseq + 1]); in the per-head
// arrays (scores, index sets, work lists, state) head h of sequence s is the
// head s * heads + h, with room for the longest sequence (the problem's n).
// Entries are clamped into [0, rows] and lengths to n, so that any contents
// keep every access inside the buffers.
struct Varlen {
    const int32_t *cu = nullptr;
    int32_t nseq = 1;
    int64_t rows = 0;            // rows of each head of q, k, v (and out, lse)
};

struct AttnArgs {
    const void *q, *k, *v;
    const int32_t *block_count, *block_offset, *column_count, *column_index;
    int32_t cap_b, cap_c;
    void *out;
    float *lse;
    int32_t hq, hkv;
    int64_t n;
    int64_t stride;      // rows from one head's start to the next (q, k, v, out, lse)
    float scale_log2;    // sm_scale * log2(e)
    float scale;         // sm_scale
    // key phases of the sparse kernel (one launch each): block tiles whose
    // start and columns that lie in [k_lo, k_hi), for the query blocks
    // b >= qb_lo; the running softmax state of a query block that is not
    // finished in a phase goes to ws (NULL: a single phase over all keys)
    int32_t phase_keys;  // keys per phase (multiple of 64); >= n: one phase
    int32_t k_lo, k_hi;
    int64_t qb_lo;
    float *ws;
    // units of grp_kh q heads of one kv group and one query block whose lists
    // leave few keys out run first as one aligned-tile walk with a shared
    // copy per tile; grp[(h / grp_kh) * nblocks + b] = 1 marks them for the
    // per-head launches to skip (NULL: no such walk)
    int32_t *grp;
    int32_t grp_kh;
    // fused mode: the index sets themselves instead of work lists, and the
    // cover end each query block's walk has reached (in the workspace)
    const int32_t *v_idx, *s_idx;
    int32_t kv, ks;
    int32_t *fused_cov;
    // fused mode in key phases: per (q head, query block) a bitmap over
    // v_idx of the columns that earlier phases passed and left uncovered,
    // fused_cw 32-bit words each (all of them run in the final phase)
    uint32_t *fused_cols;
    int32_t fused_cw;
    Varlen vl;           // hq, hkv: heads per sequence; n: the longest sequence
    // fused mode with the exact union mask: per q head, a bitmap of the
    // selected diagonal offsets over [0, n) and one of the selected column
    // keys, ex_words 32-bit words each (unused otherwise)
    const uint32_t *ex_s, *ex_v;
    int32_t ex_words;
};

// Bytes of sparse-prefill state for hq heads and n keys in phases of
// phase_keys keys (0 when one phase covers all keys).
size_t sparse_state_bytes(int64_t hq, int64_t n, int64_t phase_keys);
// Where the grouped walk's per-unit marks start in that workspace, and how
// many q heads of a kv group one unit holds.
size_t sparse_walk_marks_offset(int64_t hq, int64_t n);
// Bytes of fused-mode workspace: that state, then (when phases are used) one
// bitmap of kv bits, rounded up to 32-bit words, per (q head, query block).
// With exact, two bitmaps of n bits per q head follow (the exact union mask
// needs them even when one phase covers all keys).
size_t fused_state_bytes(int64_t hq, int64_t n, int64_t phase_keys, int64_t kv, bool exact);
int walk_heads_per_unit(int hq, int hkv);

// dtype: 0 = bf16, 1 = fp32
hipError_t launch_sparse_prefill(const AttnArgs &a, int dtype, hipStream_t s);
hipError_t launch_dense_prefill(const AttnArgs &a, int dtype, hipStream_t s);
// Sparse prefill that walks the cover of s_idx / v_idx itself (no work lists).
hipError_t launch_sparse_prefill_fused(const AttnArgs &a, int dtype, bool exact, hipStream_t s);
int fused_max_phase_keys();
int fused_max_columns();

struct EstArgs {
    const void *q, *k;
    int64_t n;           // keys (and rows of Q, K and the score arrays)
    int64_t stride;      // rows from one head's start to the next in Q and K
    // Keys are tiled in a frame shifted by pad = nv - n (nv: n rounded up to
    // 64), so that tiles end at key n - 1 as the last 64 query rows do; frame
    // keys 0 .. pad-1 do not exist and score zero.
    int64_t nv;
    int32_t pad;
    int32_t hq, hkv;
    float scale_log2;
    int64_t range_keys;  // keys per workgroup range (multiple of 64)
    int32_t nranges;
    float *part_m, *part_l;      // [hq][64][nranges]
    float *row_norm;             // [hq][64] per-row log2 normaliser (scaled max + log2 sum)
    float *v_score, *s_score;    // [hq][n]
    float *diag_hi, *diag_lo;    // [hq][nranges][64]
    Varlen vl;                   // hq, hkv: heads per sequence; n, nv, pad, nranges: the longest
};

hipError_t launch_estimate_scores(const EstArgs &a, int dtype, hipStream_t s);

struct TopkArgs {
    const float *src0, *src1;    // [hq][n] each
    int32_t *dst0, *dst1;        // [hq][k0], [hq][k1]
    int32_t k0, k1;
    int32_t hq;
    int64_t n;
    int32_t nslices;
    uint32_t *hist;              // [2*hq][2048]
    uint32_t *state;             // [2*hq][4]
    uint32_t *cnt;               // [2*hq][nslices][2]
    uint32_t *off;               // [2*hq][nslices][2]
    int32_t rows;                // rows selected: 0 = 2*hq (both sets); else the first rows, all from src0
    const int32_t *row_len = nullptr;   // NULL: every row has n entries; else row r has
    int32_t row_len_div = 1;            //   row_len[(r % hq) / row_len_div], clamped into [0, n]; a row
                                        //   with at most k of them selects 0 .. k - 1
};

constexpr int kTopkSlice = 4096;   // elements per top-k workgroup slice

hipError_t launch_topk(const TopkArgs &a, hipStream_t s);
// The same selection with one 1024-thread workgroup per row, in one launch
// (uses none of hist / state / cnt / off).
hipError_t launch_topk_rows(const TopkArgs &a, hipStream_t s);
// The lengths of a packed batch's sequences (as the kernels clamp them), for
// TopkArgs.row_len: len [vl.nseq].
hipError_t launch_seq_lengths(const Varlen &vl, int64_t nmax, int32_t *len, hipStream_t s);

// Decode-side top-k attention: one query row per q head over a cache of n keys.
struct DecodeArgs {
    const void *q;               // [hq][128]
    const void *k, *v;           // [hkv][stride][128]
    void *out;                   // [hq][128]
    float *lse;                  // [hq] natural log over the selected keys (NULL: not written)
    float *recovery;             // [hq] share of the dense attention mass selected (NULL: not written)
    int32_t hq, hkv;
    int64_t n, stride;
    float scale_log2;
    int32_t topk;
    const int32_t *idx;          // [hq][topk] the selected keys
    uint32_t *keys;              // [hq][n] order-preserving keys of the scores (log2 units)
    float *part;                 // [hq][nchunks][2] running max and sum of 2^s per key chunk
    float *lse2_all;             // [hq] dense log2-sum-exp
    int64_t chunk_keys;
    int32_t nchunks;
    const int32_t *lens;         // [hkv] keys in each kv head's cache, clamped into [0, n] (NULL: n)
};

hipError_t launch_decode_scores(const DecodeArgs &a, int dtype, hipStream_t s);
hipError_t launch_decode_attend(const DecodeArgs &a, int dtype, hipStream_t s);

struct IndexArgs {
    const int32_t *v_idx, *s_idx;
    int32_t kv, ks;
    int64_t n;
    int32_t hq;
    int32_t *block_count, *block_offset, *column_count, *column_index;
    int32_t cap_b, cap_c;
    bool vec_rows;               // every block_offset row starts 16-byte aligned (16-byte stores)
    Varlen vl;                   // hq: heads per sequence; n: the longest sequence
};

hipError_t launch_build_index(const IndexArgs &a, hipStream_t s);

struct BsArgs {
    const void *q, *k;
    int64_t n;
    int64_t stride;              // rows from one head's start to the next in q and k
    int32_t hq, hkv;
    float scale;
    int32_t topk;
    float *qm, *km;              // pooled means [hq][nb][128], [hkv][nb][128]
    uint32_t *keys;              // score keys of one chunk of query blocks [hq][chunk_rows][nb]
    int32_t chunk_rows;          // query blocks per chunk: min(nb, kBsChunkRows), so a multiple of 64
                                 // whenever there is more than one chunk
    int64_t row0;                // first query block of the chunk (set per launch)
    int32_t *block_count, *block_offset, *column_count;
    int32_t cap_b;
    Varlen vl;                   // hq, hkv: heads per sequence; n: the longest sequence
};

// Query blocks per block-sparse scoring chunk.
constexpr int32_t kBsChunkRows = 1024;

hipError_t launch_estimate_bs(const BsArgs &a, int dtype, hipStream_t s);

}  // namespace msa
