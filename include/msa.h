/*
 * msa.h -- vertical-slash dynamic sparse prefill attention for MI355X (gfx950).
 *
 * The method (MInference): each attention head follows a sparse pattern; at
 * prefill time the head's sparse index is estimated online from the input and
 * attention is computed only over the selected entries ("MInference 1.0
 * README", section "TL;DR"; talk slides "System-Algorithm Co-design", slide
 * "MInference", steps 1-2).  For vertical-slash heads the index is a set of key
 * columns (vertical lines) and a set of diagonals (slash lines) (same slides,
 * slide "Dynamic sparsity in attention").  The README's kernel-only interface
 * is one fused call per pattern returning the attention output
 * (vertical_slash_sparse_attention(q, k, v, vertical_topk, slash),
 * block_sparse_attention(q, k, v, topk), section "How to use MInference",
 * kernel-only usage).  This library splits that call into its steps:
 *
 *   msa_estimate_vs      -> vertical and slash index sets (top-k)
 *   msa_build_index      -> per-query-block work lists (64-wide key blocks
 *                           covering the diagonals, plus leftover columns)
 *   msa_sparse_prefill   -> causal attention over the work lists
 *   msa_dense_prefill    -> dense causal attention (the speedup denominator)
 *   msa_estimate_bs      -> block-sparse work lists (mean-pooled block scores)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Tensors are device memory owned by the caller, batch 1, [heads, seq_len,
 *    head_dim] row-major with head h starting at row h * seq_stride
 *    (seq_stride = seq_len: contiguous).  A packed batch of sequences, stored
 *    as [heads, total, head_dim], is one call per sequence with the pointers
 *    at its first row and seq_stride = total.  Q has n_q_heads heads; K and V have
 *    n_kv_heads; q head h reads kv head h / (n_q_heads / n_kv_heads).
 *  * head_dim must be 128; seq_len must be positive and below 2^31
 *    (msa_estimate_vs needs at least 64); n_q_heads must be a multiple of
 *    n_kv_heads.  Query blocks are 64 rows; when seq_len is not a multiple of
 *    64 the last one is shorter (rows 64b .. seq_len-1), and per-block arrays
 *    have ceil(seq_len / 64) entries per head.
 *  * A subset of heads is selected by offsetting the pointers (q by h0 heads,
 *    k/v by h0/G heads) and passing the subset's head counts.
 *  * q, k, v, out and every workspace must be 16-byte aligned (any whole
 *    tensor from a device allocator is; so is a view that starts at a row or
 *    head boundary), the int32 and float arrays 4-byte aligned.  Anything
 *    else returns MSA_ERR_RANGE.
 *  * The library never allocates or frees device memory.  Scratch memory comes
 *    from a caller-provided workspace whose size the *_workspace call returns.
 *  * `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously; nothing is copied to the host.
 *  * Every call validates its arguments on the host before touching the
 *    device, and returns MSA_OK or an error status without enqueuing anything.
 *    msa_last_error() then gives a message (thread-local).  Launch failures
 *    return MSA_ERR_LAUNCH.  Faults inside kernels surface at the caller's next
 *    synchronisation.  No C++ exception crosses this interface.
 *  * Calls keep no state between them; concurrent calls on different streams
 *    with disjoint outputs and workspaces are safe.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MSA_OK = 0,
    MSA_ERR_NULL = 1,       /* a required pointer is NULL */
    MSA_ERR_SHAPE = 2,      /* unsupported head counts, seq_len or head_dim */
    MSA_ERR_DTYPE = 3,      /* unknown element type */
    MSA_ERR_RANGE = 4,      /* a scalar argument is out of range (top-k, block, last_q) */
    MSA_ERR_CAPACITY = 5,   /* an index capacity is smaller than msa_index_caps returns */
    MSA_ERR_WORKSPACE = 6,  /* workspace smaller than the *_workspace size */
    MSA_ERR_LAUNCH = 7      /* the HIP runtime refused a launch */
} msa_status;

typedef enum {
    MSA_BF16 = 0,           /* bfloat16 Q/K/V/out, fp32 accumulation */
    MSA_F32 = 1             /* float32 Q/K/V/out, fp32 accumulation */
} msa_dtype;

typedef struct {
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int64_t seq_len;
    int32_t head_dim;       /* must be 128 */
    int32_t dtype;          /* msa_dtype */
    float sm_scale;         /* softmax scale; 0 selects 1/sqrt(head_dim) */
    int64_t seq_stride;     /* rows from one head's start to the next in q, k, v,
                               out and lse; 0 selects seq_len (contiguous) */
} msa_problem;

/* Human-readable name of a status code (static storage). */
const char *msa_status_str(int status);

/* Detail of the last error returned on this thread ("" if none). */
const char *msa_last_error(void);

/* Capacities of the work lists for one query block (block = 64):
 *   cap_blocks = min(slash_topk, ceil(seq_len / 64))   (blocks are disjoint and start
 *                at or before the block's last row, so at most b+1 of them)
 *   cap_cols   = min(vertical_topk, seq_len).                               */
int msa_index_caps(const msa_problem *p, int32_t vertical_topk, int32_t slash_topk, int32_t block,
                   int32_t *cap_blocks, int32_t *cap_cols);

/* Workspace bytes msa_estimate_vs needs for these arguments. */
size_t msa_estimate_vs_workspace(const msa_problem *p, int32_t last_q, int32_t vertical_topk,
                                 int32_t slash_topk);

/* Online vertical-slash index estimation.
 * For every q head h (kv head g = h / G) and the last L = last_q query rows
 * p_r = N - L + r (the pages: the index is approximated online per head,
 * "MInference 1.0 README", "TL;DR"; talk slides "System-Algorithm
 * Co-design", slide "MInference", online estimation of sparsity indices):
 *     z[r, j]  = sm_scale * <q[h, p_r], k[g, j]>  for j <= p_r   (causal)
 *     P[r, :]  = softmax over j
 *     v[j]     = sum_r P[r, j]                  (vertical score)
 *     s[o]     = sum_r P[r, p_r - o], o = i - j (slash score)
 * then v_idx[h] = the vertical_topk largest v, s_idx[h] = the slash_topk
 * largest s, exact ties going to the lower index, each written in ascending
 * order.  last_q must be 64.  1 <= vertical_topk, slash_topk <= seq_len.
 *   q [n_q_heads, N, 128], k [n_kv_heads, N, 128]      (dtype of p)
 *   v_idx [n_q_heads, vertical_topk] int32, s_idx [n_q_heads, slash_topk] int32
 *   v_score, s_score [n_q_heads, N] float32: optional outputs of the scores
 *   (NULL: kept in the workspace).                                          */
int msa_estimate_vs(const msa_problem *p, const void *q, const void *k, int32_t last_q,
                    int32_t vertical_topk, int32_t slash_topk, int32_t *v_idx, int32_t *s_idx,
                    float *v_score, float *s_score, void *workspace, size_t workspace_bytes,
                    void *stream);

/* msa_estimate_vs without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results and errors as
 * msa_estimate_vs, minus the workspace: its scratch is a fixed array of
 * 80 MiB that the library holds on each GPU it runs on until the process
 * ends (32 q heads up to 262,144 tokens; 8 q heads up to 1M).  A problem
 * needing more (msa_estimate_vs_workspace) returns MSA_ERR_WORKSPACE;
 * splitting the heads over several calls (head subsets, see above) fits it.
 * The call works on the GPU current on the calling thread, which must be
 * `stream`'s; it allocates and frees nothing.  Every call on one GPU shares
 * that GPU's array (each call initialises what it reads): calls that overlap
 * in time on one GPU, on any streams, race and give undefined results. */
int msa_estimate_vs_noalloc(const msa_problem *p, const void *q, const void *k, int32_t last_q,
                            int32_t vertical_topk, int32_t slash_topk, int32_t *v_idx, int32_t *s_idx,
                            float *v_score, float *s_score, void *stream);

/* Work lists from index sets (block = 64).  For query block b (rows r0 = 64b to
 * r1 = min(64b+63, N-1)), each selected offset o <= r1 needs keys [max(0, r0-o), r1-o];
 * visiting those ranges by descending o, a range not yet covered emits a
 * 64-wide block starting at max(range start, end of the previous block).
 * Columns: every selected j <= r1 outside all emitted blocks, ascending.
 * The pages ask for sparse work in large contiguous blocks suited to the matrix
 * units, built online at small cost ("How to optimise the TTFT of an 8B LLM
 * with 1M tokens to 20 seconds", section on co-designing algorithm and system,
 * principles 1-2); the covering rule itself is this library's reading.
 *   v_idx [n_q_heads, vertical_topk], s_idx [n_q_heads, slash_topk]: ascending,
 *     distinct, in [0, N); out-of-range entries are ignored.
 *   block_count, column_count [n_q_heads, ceil(N/64)] int32
 *   block_offset [n_q_heads, ceil(N/64), cap_blocks] int32 (key start of each block)
 *   column_index [n_q_heads, ceil(N/64), cap_cols] int32
 * Entries past each count are unspecified.                                  */
int msa_build_index(const msa_problem *p, const int32_t *v_idx, int32_t vertical_topk,
                    const int32_t *s_idx, int32_t slash_topk, int32_t block,
                    int32_t *block_count, int32_t *block_offset, int32_t cap_blocks,
                    int32_t *column_count, int32_t *column_index, int32_t cap_cols, void *stream);

/* Sparse causal attention over the work lists (talk slides "System-Algorithm
 * Co-design", slide "MInference": dynamic sparse attention calculation).  Row i
 * of query block b attends to key j iff j <= i and j lies in one of b's blocks
 * [st, st+63] or in b's column list:
 *     out[h, i] = sum_j softmax_j(sm_scale <q_i, k_j>) v_j,
 *     lse[h, i] = log sum_j exp(sm_scale <q_i, k_j>)   (natural log)
 * A row with no allowed key gives out = 0 and lse = -inf.  Counts above the
 * capacities are clamped; keys outside [0, N) are ignored.
 *
 * Preconditions on the lists of each query block (msa_build_index and
 * msa_estimate_bs write lists that meet them):
 *   - block starts ascending and pairwise disjoint: each start at least 64
 *     past the one before;
 *   - column keys distinct and outside every block of the same query block,
 *     in any order.
 * The sum above runs over the listed keys, so a key listed twice (a column
 * inside a block, overlapping blocks, a repeated column) would be counted
 * twice; such lists give unspecified (finite) results, never an access
 * outside q, k, v, out, lse or the workspace.
 *
 * Key phases.  With R = phase_keys (0 selects MSA_DEFAULT_PHASE_KEYS) below
 * seq_len, the work runs as ceil(N / R) launches in order on `stream`; launch
 * j takes the block tiles whose start lies in [jR, (j+1)R) (the first also
 * starts below 0, the last every start from jR on), so the K/V read at any
 * time come mostly from one R-key range of a kv head; a query block with only
 * a few tiles in a range leaves them to the next launch, and its columns go
 * to the launch that holds its own rows.  The running softmax state of each
 * query block (fp32) passes between launches through `workspace`.  Before
 * them, one launch takes the query blocks whose lists, for every q head of a
 * kv group (up to four heads), leave at most 1/8 of the keys [0, r1] out: it
 * walks all 64-key tiles 0..b once for those heads together and masks each
 * head to its own blocks and columns.  It takes a query block only if every
 * such head's blocks are ascending and disjoint and its columns strictly
 * ascending (others run per head); the result is the same up to fp32
 * rounding order.  With
 * R >= seq_len there is one launch over the lists in their given order and no
 * workspace is used (it may be NULL).
 *   phase_keys: 0 or a positive multiple of 64, else MSA_ERR_RANGE.
 *   workspace: msa_sparse_prefill_workspace() bytes, 16-byte aligned, owned by
 *     the caller, no initial contents; calls sharing one must not overlap.
 *   out [n_q_heads, N, 128] (dtype of p); lse [n_q_heads, N] float32 or NULL. */
int msa_sparse_prefill(const msa_problem *p, const void *q, const void *k, const void *v,
                       const int32_t *block_count, const int32_t *block_offset, int32_t cap_blocks,
                       const int32_t *column_count, const int32_t *column_index, int32_t cap_cols,
                       int32_t phase_keys, void *workspace, size_t workspace_bytes, void *out, float *lse,
                       void *stream);

/* Keys per phase of msa_sparse_prefill when phase_keys is 0 (K+V of one kv
 * head over this many keys: 6 MB in bf16). */
#define MSA_DEFAULT_PHASE_KEYS 12288

/* Workspace bytes msa_sparse_prefill needs (0 when one phase covers seq_len;
 * 0 for invalid arguments):
 *   n_q_heads * ceil(seq_len / 64) * (2 * (64 * 64 + 2 * 64) * 4 + 12). */
size_t msa_sparse_prefill_workspace(const msa_problem *p, int32_t phase_keys);

/* msa_build_index followed by msa_sparse_prefill in one call that builds no
 * work lists: each query block's 64-wide key blocks are the same greedy cover
 * of its selected diagonals (msa_build_index above), walked inside the
 * attention kernel over the sorted s_idx, one key phase at a time, and its
 * leftover columns are found from v_idx in the phases that pass them; no
 * block_offset / column_index arrays exist (12.8 + 2.1 GB at 1M tokens and 32
 * heads).  The pages ask for an index built online at minimal overhead ("How
 * to optimise the TTFT of an 8B LLM with 1M tokens to 20 seconds", section on
 * co-designing algorithm and system, principle 2).  Same attention and key
 * phases as msa_sparse_prefill over msa_build_index's lists, the same tiles
 * in the same order (blocks per phase, every column in the query block's
 * final phase), but without the grouped walk, so where that walk runs the
 * results agree up to fp32 rounding order and elsewhere bit for bit.  Same
 * errors, and:
 *   v_idx [n_q_heads, vertical_topk], s_idx [n_q_heads, slash_topk] int32,
 *     ascending and distinct, as msa_estimate_vs writes them; entries outside
 *     [0, N) select nothing (other orders give unspecified but finite
 *     results, never an access out of bounds);
 *   vertical_topk <= 1024 and phase keys (phase_keys, 0 = the default) at most
 *     16384, else MSA_ERR_RANGE (the kernel holds a block's columns and a
 *     phase's block starts in LDS);
 *   flags: 0, or MSA_FUSED_EXACT for the exact union mask: entry (i, j) is
 *     attended iff j <= i and (j is a selected column or i - j a selected
 *     diagonal) -- the selected lines themselves, as the talk slides draw
 *     the vertical-slash pattern (slide "Dynamic sparsity in attention"),
 *     instead of the 64-key blocks that cover them; the same tiles are
 *     visited, with the entries off those lines masked; other bits:
 *     MSA_ERR_RANGE;
 *   workspace: msa_sparse_prefill_fused_workspace(p, vertical_topk,
 *     phase_keys, flags) bytes, 16-byte aligned (the key-phase state of
 *     msa_sparse_prefill_workspace, then one bitmap of vertical_topk bits per
 *     q head and query block, then with MSA_FUSED_EXACT two bitmaps of N bits
 *     per q head; 0 bytes: none needed); no initial contents assumed.      */
#define MSA_FUSED_EXACT 1
size_t msa_sparse_prefill_fused_workspace(const msa_problem *p, int32_t vertical_topk, int32_t phase_keys,
                                          int32_t flags);
int msa_sparse_prefill_fused(const msa_problem *p, const void *q, const void *k, const void *v,
                             const int32_t *v_idx, int32_t vertical_topk, const int32_t *s_idx, int32_t slash_topk,
                             int32_t phase_keys, int32_t flags, void *workspace, size_t workspace_bytes, void *out,
                             float *lse, void *stream);

/* Where msa_sparse_prefill records which query blocks the grouped walk took
 * (a diagnostic: the walk executes every aligned tile 0..b of such a block for
 * each of its heads, masked to the head's lists, so its executed tiles are
 * not the listed ones).  After a msa_sparse_prefill call with the same
 * problem and phase_keys, the int32 at byte
 *     offset + 4 * ((h / heads_per_unit) * ceil(N/64) + b)
 * of its workspace is 1 if query block b of q head h ran in the walk, else 0.
 * heads_per_unit = 0 (and offset = 0) when the call uses no workspace (one
 * phase), and then no block runs in the walk.  Errors as for
 * msa_sparse_prefill_workspace's arguments. */
int msa_sparse_prefill_walk_marks(const msa_problem *p, int32_t phase_keys, size_t *offset,
                                  int32_t *heads_per_unit);

/* Dense causal attention (every j <= i), same layouts as msa_sparse_prefill:
 * out[h, i] = sum_{j <= i} softmax_j(sm_scale <q_i, k_j>) v_j, lse as above.
 * This is the FlashAttention baseline the pages measure the sparse method
 * against ("How to optimise the TTFT of an 8B LLM with 1M tokens to 20
 * seconds", section on the speedup needed relative to FlashAttention; talk
 * slides "System-Algorithm Co-design", slide "MInference": FlashAttn vs
 * MInference latency at 1M tokens on one A100), computed here on the same
 * GPU as the speedup denominator.  No workspace; errors as for every call. */
int msa_dense_prefill(const msa_problem *p, const void *q, const void *k, const void *v,
                      void *out, float *lse, void *stream);

/* Workspace bytes msa_estimate_bs needs. */
size_t msa_estimate_bs_workspace(const msa_problem *p, int32_t block);

/* Block-sparse work lists (talk slides "System-Algorithm Co-design", patterns
 * slide: block-sparse heads; "MInference 1.0 README", kernel-only
 * block_sparse_attention(q, k, v, topk)).  Reading: with qm[b] and km[c] the
 * means of 64-row blocks of q and k (a short last block: the mean of its
 * rows), u[b, c] = sm_scale <qm[b], km[c]> for c <= b; query block b keeps its
 * min(topk_blocks, b+1) highest-scoring key blocks (exact ties to the lower
 * c), written as ascending key starts 64c.  column_count is set to 0.  block
 * must be 64; cap_blocks >= min(topk_blocks, ceil(N/64)).  Any seq_len below
 * 2^31 is accepted (the workspace grows as n_q_heads * ceil(N/64) *
 * min(ceil(N/64), 1024) * 4 bytes plus the pooled means).                   */
int msa_estimate_bs(const msa_problem *p, const void *q, const void *k, int32_t block,
                    int32_t topk_blocks, int32_t *block_count, int32_t *block_offset,
                    int32_t cap_blocks, int32_t *column_count, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Decode-side dynamic sparsity: one new query row per q head attends only to
 * the top-k cached keys by attention score, chosen anew at every call (talk
 * slides "System-Algorithm Co-design", slide "Dynamic sparsity in
 * attention", decoding panel: choosing the top-1000 keys of a 100K-token
 * cache dynamically keeps more of the attention mass than a static choice).
 *   p: seq_len = N cached keys; n_q_heads, n_kv_heads, dtype, sm_scale and
 *      seq_stride (rows between cache heads) as for prefill.  A batch of
 *      sequences is folded into the heads (n_q_heads = batch * Hq with the
 *      caches as batch * Hkv heads, Hq / Hkv per group as always).
 *   q [n_q_heads, 128] (one row per head, 16-byte aligned); k, v caches
 *      [n_kv_heads, stride, 128]; out [n_q_heads, 128] (dtype).
 *   topk in [1, N]; idx [n_q_heads, topk] int32: written with the selected
 *      keys, ascending, exact top-k of s[h, j] = sm_scale <q_h, k_j> (ties to
 *      the lower index) -- or, with flags = MSA_DECODE_GIVEN_KEYS, read as the
 *      caller's own selection (a static pattern, say; entries are clamped into
 *      [0, N), a key given twice counts twice).
 *   lse [n_q_heads] (optional): natural log-sum-exp of the selected scores;
 *   recovery [n_q_heads] (optional): the selected keys' share of the dense
 *      attention mass, sum over selected e^s / sum over all e^s.
 *   workspace: msa_decode_sparse_workspace(p) bytes, 16-byte aligned, no
 *      initial contents assumed.
 * Errors as for every call; topk out of range or unknown flags:
 * MSA_ERR_RANGE.                                                           */
#define MSA_DECODE_GIVEN_KEYS 1
size_t msa_decode_sparse_workspace(const msa_problem *p);
int msa_decode_sparse(const msa_problem *p, const void *q, const void *k, const void *v, int32_t topk,
                      int32_t *idx, int32_t flags, void *workspace, size_t workspace_bytes, void *out, float *lse,
                      float *recovery, void *stream);

/* msa_decode_sparse over caches of different lengths (a batch of sequences at
 * different positions, folded into the heads as above): kv head g holds the
 * keys 0 .. cache_lens[g] - 1 of its rows; seq_len is the capacity.  A
 * position past a cache's length holds no key and scores -inf (the same
 * slide: the decode step attends over the keys that exist): it is never read,
 * gets no weight and is outside the dense sum behind recovery.
 *   cache_lens [n_kv_heads] int32, device memory, 4-byte aligned; each value
 *     is clamped into [0, seq_len] on the device.
 *   idx: the top-k as above over those scores, so a cache holding fewer than
 *     topk keys gives all of them followed by the lowest positions past its
 *     end (no weight); given keys (MSA_DECODE_GIVEN_KEYS) at or past the end
 *     get no weight.
 *   A head whose cache is empty: out 0, lse -inf, recovery 0.
 * Workspace: msa_decode_sparse_workspace(p).  Errors as msa_decode_sparse;
 * cache_lens NULL: MSA_ERR_NULL.                                            */
int msa_decode_sparse_varlen(const msa_problem *p, const void *q, const void *k, const void *v,
                             const int32_t *cache_lens, int32_t topk, int32_t *idx, int32_t flags, void *workspace,
                             size_t workspace_bytes, void *out, float *lse, float *recovery, void *stream);

/* ---- Packed batches of sequences of different lengths ----
 * The pages' kernel-only interface takes a batch dimension ("MInference 1.0
 * README", kernel-only usage); these forms take a batch whose sequences have
 * different lengths as one problem (one launch chain instead of one per
 * sequence).  Sequence s holds rows cu_seqlens[s] .. cu_seqlens[s+1] - 1 of
 * every head of q, k, v, out and lse, which hold p->seq_len rows per head
 * (p->seq_stride apart; 0: seq_len).  Each sequence is computed exactly as the
 * one-sequence call on its own rows would compute it, except that a sequence
 * shorter than last_q = 64 takes all its rows as the estimate's window (the
 * one-sequence estimate refuses such a length).
 *   cu_seqlens: device int32 [n_seqs + 1], ascending from 0, at most seq_len,
 *     4-byte aligned; max_seqlen: a host value at least every length, at
 *     most seq_len.  The device clamps entries into [0, seq_len] and lengths
 *     to max_seqlen, so contents that break these rules give unspecified
 *     results (overlapping sequences overwrite each other's rows) but no
 *     access outside the buffers.
 *   n_seqs * n_q_heads at most 32767.
 *   Per-head arrays (index sets, work lists) hold n_seqs * n_q_heads heads:
 *     head h of sequence s is s * n_q_heads + h; each is sized for max_seqlen
 *     (index sets [heads, topk]; block_count [heads, ceil(max_seqlen / 64)],
 *     caps from msa_index_caps with seq_len = max_seqlen); the entries of
 *     query blocks past a sequence's end are not written.  A sequence whose
 *     length is at most a top-k selects all its keys and then the positions
 *     past its end, which msa_build_index_varlen ignores.
 *   Rows of q, k, v, out and lse outside every sequence are neither read nor
 *     written.
 *   The grouped walk's marks in a msa_sparse_prefill_varlen workspace are
 *     where msa_sparse_prefill_walk_marks puts them for a problem of
 *     n_seqs * n_q_heads q heads, n_seqs * n_kv_heads kv heads and seq_len =
 *     max_seqlen.
 * Errors as for the one-sequence calls; a NULL descriptor or cu_seqlens:
 * MSA_ERR_NULL; n_seqs, max_seqlen or the head count out of range:
 * MSA_ERR_SHAPE.                                                            */
typedef struct {
    const int32_t *cu_seqlens;
    int32_t n_seqs;
    int32_t max_seqlen;
} msa_varlen;

size_t msa_estimate_vs_varlen_workspace(const msa_problem *p, const msa_varlen *vl, int32_t last_q);
/* msa_estimate_vs per sequence (the same online estimate); top-k values in
 * [1, max_seqlen]. */
int msa_estimate_vs_varlen(const msa_problem *p, const msa_varlen *vl, const void *q, const void *k, int32_t last_q,
                           int32_t vertical_topk, int32_t slash_topk, int32_t *v_idx, int32_t *s_idx, void *workspace,
                           size_t workspace_bytes, void *stream);
/* msa_build_index per sequence (the same cover rule). */
int msa_build_index_varlen(const msa_problem *p, const msa_varlen *vl, const int32_t *v_idx, int32_t vertical_topk,
                           const int32_t *s_idx, int32_t slash_topk, int32_t block, int32_t *block_count,
                           int32_t *block_offset, int32_t cap_blocks, int32_t *column_count, int32_t *column_index,
                           int32_t cap_cols, void *stream);
size_t msa_sparse_prefill_varlen_workspace(const msa_problem *p, const msa_varlen *vl, int32_t phase_keys);
/* msa_sparse_prefill per sequence (the same attention over the lists, key
 * phases of the longest sequence's geometry). */
int msa_sparse_prefill_varlen(const msa_problem *p, const msa_varlen *vl, const void *q, const void *k, const void *v,
                              const int32_t *block_count, const int32_t *block_offset, int32_t cap_blocks,
                              const int32_t *column_count, const int32_t *column_index, int32_t cap_cols,
                              int32_t phase_keys, void *workspace, size_t workspace_bytes, void *out, float *lse,
                              void *stream);
size_t msa_estimate_bs_varlen_workspace(const msa_problem *p, const msa_varlen *vl, int32_t block);
/* msa_estimate_bs per sequence (the same block scores and selection): work
 * lists of n_seqs * n_q_heads heads, ceil(max_seqlen / 64) query blocks each;
 * cap_blocks at least min(topk_blocks, ceil(max_seqlen / 64)). */
int msa_estimate_bs_varlen(const msa_problem *p, const msa_varlen *vl, const void *q, const void *k, int32_t block,
                           int32_t topk_blocks, int32_t *block_count, int32_t *block_offset, int32_t cap_blocks,
                           int32_t *column_count, void *workspace, size_t workspace_bytes, void *stream);
/* msa_dense_prefill per sequence (the FlashAttention baseline the speedups
 * of the pages are quoted against, on a packed batch). */
int msa_dense_prefill_varlen(const msa_problem *p, const msa_varlen *vl, const void *q, const void *k, const void *v,
                             void *out, float *lse, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
