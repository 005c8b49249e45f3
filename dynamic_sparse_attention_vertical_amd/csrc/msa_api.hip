// C-ABI entry points: host-side validation, workspace layout and launches.
// Every argument is checked before anything is enqueued; no C++ exception
// leaves this file.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "msa.h"
#include "common.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = 0;
    return MSA_OK;
}

int launch_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(MSA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

int check_problem(const msa_problem *p) {
    if (!p) return fail(MSA_ERR_NULL, "problem descriptor is NULL");
    if (p->head_dim != 128) return fail(MSA_ERR_SHAPE, "head_dim must be 128 (got %d)", p->head_dim);
    if (p->n_q_heads <= 0 || p->n_kv_heads <= 0 || p->n_q_heads % p->n_kv_heads != 0)
        return fail(MSA_ERR_SHAPE, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                    p->n_q_heads, p->n_kv_heads);
    if (p->seq_len <= 0 || p->seq_len >= (int64_t(1) << 31))
        return fail(MSA_ERR_SHAPE, "seq_len must be positive and below 2^31 (got %lld)", (long long)p->seq_len);
    if (p->dtype != MSA_BF16 && p->dtype != MSA_F32)
        return fail(MSA_ERR_DTYPE, "unknown dtype %d", p->dtype);
    if (!(p->sm_scale >= 0.f) || isinf(p->sm_scale))
        return fail(MSA_ERR_RANGE, "sm_scale must be finite and >= 0");
    if (p->seq_stride != 0 && p->seq_stride < p->seq_len)
        return fail(MSA_ERR_SHAPE, "seq_stride (%lld) must be 0 or at least seq_len (%lld)",
                    (long long)p->seq_stride, (long long)p->seq_len);
    return MSA_OK;
}

// rows from one head's start to the next
int64_t stride_of(const msa_problem *p) { return p->seq_stride ? p->seq_stride : p->seq_len; }

float scale_of(const msa_problem *p) {
    return p->sm_scale > 0.f ? p->sm_scale : 1.0f / sqrtf((float)p->head_dim);
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Row data (q, k, v, out) and workspaces are read and written 16 bytes at a
// time; int32 and float arrays one element at a time.
bool off_align(const void *ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) != 0; }

int check_rows(const void *q, const void *k, const void *v, const void *out) {
    if (off_align(q, 16) || off_align(k, 16) || (v && off_align(v, 16)) || (out && off_align(out, 16)))
        return fail(MSA_ERR_RANGE, "q, k, v and out must be 16-byte aligned");
    return MSA_OK;
}

// Estimator work split: contiguous key ranges (256 .. 8192 keys) per workgroup,
// about 512 workgroups over the kv heads: long enough ranges to amortise each
// workgroup's set-up, enough workgroups for every CU.
struct EstLayout {
    int64_t range_keys;
    int32_t nranges;
    int32_t nslices;
    size_t off_part_m, off_part_l, off_row_norm, off_hi, off_lo, off_v, off_s;
    size_t off_hist, off_state, off_cnt, off_off, off_lens, total;
};

// hq_all, hkv_all: the heads of all sequences; n: keys of the longest one;
// nlens: sequences of a packed batch (their lengths for the top-k go to
// off_lens), 0 for one sequence
EstLayout est_layout_for(int64_t hq_all, int64_t hkv_all, int64_t n, int64_t nlens) {
    EstLayout L;
    const int64_t nv = (n + 63) / 64 * 64;            // keys tiled in 64s, ending at key n-1
    int64_t rk = (nv * hkv_all + 511) / 512;
    rk = ((rk + 63) / 64) * 64;
    if (rk < 256) rk = 256;
    if (rk > 8192) rk = 8192;
    if (rk > nv) rk = nv;
    L.range_keys = rk;
    L.nranges = (int32_t)((nv + rk - 1) / rk);
    L.nslices = (int32_t)((n + msa::kTopkSlice - 1) / msa::kTopkSlice);
    const size_t hq = (size_t)hq_all;
    size_t o = 0;
    L.off_part_m = o; o = align_up(o + hq * 64 * L.nranges * 4);
    L.off_part_l = o; o = align_up(o + hq * 64 * L.nranges * 4);
    L.off_row_norm = o; o = align_up(o + hq * 64 * 4);
    L.off_hi = o;     o = align_up(o + hq * L.nranges * 64 * 4);
    L.off_lo = o;     o = align_up(o + hq * L.nranges * 64 * 4);
    L.off_v = o;      o = align_up(o + hq * (size_t)n * 4);
    L.off_s = o;      o = align_up(o + hq * (size_t)n * 4);
    L.off_hist = o;   o = align_up(o + 2 * hq * 2048 * 4);
    L.off_state = o;  o = align_up(o + 2 * hq * 4 * 4);
    L.off_cnt = o;    o = align_up(o + 2 * hq * (size_t)L.nslices * 2 * 4);
    L.off_off = o;    o = align_up(o + 2 * hq * (size_t)L.nslices * 2 * 4);
    L.off_lens = o;   o = align_up(o + (size_t)nlens * 4);
    L.total = o;
    return L;
}

EstLayout est_layout(const msa_problem *p) { return est_layout_for(p->n_q_heads, p->n_kv_heads, p->seq_len, 0); }

template <typename T> T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off);
}

// Argument checks of msa_estimate_vs other than the workspace.
int check_estimate_vs(const msa_problem *p, const void *q, const void *k, int32_t last_q, int32_t vertical_topk,
                      int32_t slash_topk, const int32_t *v_idx, const int32_t *s_idx, const float *v_score,
                      const float *s_score) {
    int st = check_problem(p);
    if (st) return st;
    if (!q || !k || !v_idx || !s_idx) return fail(MSA_ERR_NULL, "a required pointer is NULL");
    if ((st = check_rows(q, k, nullptr, nullptr))) return st;
    if (off_align(v_idx, 4) || off_align(s_idx, 4) || off_align(v_score, 4) || off_align(s_score, 4))
        return fail(MSA_ERR_RANGE, "index and score arrays must be 4-byte aligned");
    if (last_q != 64) return fail(MSA_ERR_RANGE, "last_q must be 64 (got %d)", last_q);
    if (p->seq_len < 64)
        return fail(MSA_ERR_SHAPE, "seq_len must be at least last_q = 64 (got %lld)", (long long)p->seq_len);
    if (vertical_topk < 1 || vertical_topk > p->seq_len || slash_topk < 1 || slash_topk > p->seq_len)
        return fail(MSA_ERR_RANGE, "top-k values must lie in [1, seq_len]");
    return MSA_OK;
}

// The estimate's launches on a checked problem and a workspace of at least
// est_layout(p).total bytes.
int run_estimate_vs(const msa_problem *p, const void *q, const void *k, int32_t vertical_topk, int32_t slash_topk,
                    int32_t *v_idx, int32_t *s_idx, float *v_score, float *s_score, void *workspace,
                    void *stream, const msa::Varlen *vl = nullptr, int64_t max_len = 0) {
    const int64_t nseq = vl ? vl->nseq : 1, n = vl ? max_len : p->seq_len;
    const EstLayout L = est_layout_for(p->n_q_heads * nseq, p->n_kv_heads * nseq, n, vl ? nseq : 0);
    int st;
    msa::EstArgs e;
    e.q = q;
    e.k = k;
    e.n = n;
    e.stride = stride_of(p);
    e.nv = (n + 63) / 64 * 64;
    e.pad = (int32_t)(e.nv - e.n);
    e.hq = p->n_q_heads;
    e.hkv = p->n_kv_heads;
    e.scale_log2 = scale_of(p) * msa::kLog2e;
    e.range_keys = L.range_keys;
    e.nranges = L.nranges;
    e.part_m = at<float>(workspace, L.off_part_m);
    e.part_l = at<float>(workspace, L.off_part_l);
    e.row_norm = at<float>(workspace, L.off_row_norm);
    e.diag_hi = at<float>(workspace, L.off_hi);
    e.diag_lo = at<float>(workspace, L.off_lo);
    e.v_score = v_score ? v_score : at<float>(workspace, L.off_v);
    e.s_score = s_score ? s_score : at<float>(workspace, L.off_s);
    if (vl) e.vl = *vl;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    st = launch_status(msa::launch_estimate_scores(e, p->dtype, s), "estimate");
    if (st) return st;
    msa::TopkArgs t;
    t.src0 = e.v_score;
    t.src1 = e.s_score;
    t.dst0 = v_idx;
    t.dst1 = s_idx;
    t.k0 = vertical_topk;
    t.k1 = slash_topk;
    t.hq = (int32_t)(p->n_q_heads * nseq);
    t.n = n;
    t.nslices = L.nslices;
    t.hist = at<uint32_t>(workspace, L.off_hist);
    t.state = at<uint32_t>(workspace, L.off_state);
    t.cnt = at<uint32_t>(workspace, L.off_cnt);
    t.off = at<uint32_t>(workspace, L.off_off);
    t.rows = 0;
    if (!vl) return launch_status(msa::launch_topk(t, s), "top-k");
    // a packed batch: each row selects among its own sequence's keys (a row
    // with at most k of them takes 0 .. k-1, the ones past its end ignored by
    // the index builder), one workgroup per row
    int32_t *lens = at<int32_t>(workspace, L.off_lens);
    if ((st = launch_status(msa::launch_seq_lengths(*vl, n, lens, s), "sequence lengths"))) return st;
    t.row_len = lens;
    t.row_len_div = p->n_q_heads;
    return launch_status(msa::launch_topk_rows(t, s), "top-k");
}

// Workspace of msa_decode_sparse: score keys, chunk partials, dense lse, and
// the top-k select's histograms and counters.
struct DecodeLayout {
    int64_t chunk_keys;
    int32_t nchunks, nslices;
    size_t off_keys, off_part, off_lse, off_hist, off_state, off_cnt, off_off, total;
};

DecodeLayout decode_layout(const msa_problem *p) {
    DecodeLayout L;
    const int64_t n = p->seq_len;
    // about 24576 workgroups per pass over the caches (16 rounds of the ~1536
    // that fit on the chip at once): with a few large chunks per kv head the
    // last round runs a handful of workgroups alone (1600 chunks of 4096 keys:
    // 0.558 ms per 100K-key step against 0.484 with 24576 chunks of 261).
    // Chunks are whole multiples of the 256 rows a workgroup loads per step.
    int64_t ck = (n * p->n_kv_heads + 24575) / 24576;
    ck = (ck + 128) / 256 * 256;
    if (ck < 256) ck = 256;
    L.chunk_keys = ck;
    L.nchunks = (int32_t)((n + ck - 1) / ck);
    L.nslices = (int32_t)((n + msa::kTopkSlice - 1) / msa::kTopkSlice);
    const size_t hq = (size_t)p->n_q_heads;
    size_t o = 0;
    L.off_keys = o;  o = align_up(o + hq * (size_t)n * 4);
    L.off_part = o;  o = align_up(o + hq * (size_t)L.nchunks * 2 * 4);
    L.off_lse = o;   o = align_up(o + hq * 4);
    L.off_hist = o;  o = align_up(o + hq * 2048 * 4);
    L.off_state = o; o = align_up(o + hq * 4 * 4);
    L.off_cnt = o;   o = align_up(o + hq * (size_t)L.nslices * 2 * 4);
    L.off_off = o;   o = align_up(o + hq * (size_t)L.nslices * 2 * 4);
    L.total = o;
    return L;
}

// Scratch of msa_estimate_vs_noalloc: device memory of the library itself, one
// copy per GPU, held until the process ends, so that the call allocates
// nothing.  Host code reaches it only through the per-device address that
// hipGetSymbolAddress returns (the array's own name is a host-side stand-in).
constexpr size_t kNoAllocScratchBytes = size_t(80) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

// This device's scratch address, looked up once per device (with the device
// current) and kept.
int scratch_of_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MSA_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MSA_ERR_LAUNCH, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void *addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || addr == nullptr)
            return fail(MSA_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch[dev] = addr;
    }
    *ptr = g_scratch[dev];
    return MSA_OK;
}

}  // namespace

extern "C" {

const char *msa_status_str(int status) {
    switch (status) {
        case MSA_OK: return "MSA_OK";
        case MSA_ERR_NULL: return "MSA_ERR_NULL";
        case MSA_ERR_SHAPE: return "MSA_ERR_SHAPE";
        case MSA_ERR_DTYPE: return "MSA_ERR_DTYPE";
        case MSA_ERR_RANGE: return "MSA_ERR_RANGE";
        case MSA_ERR_CAPACITY: return "MSA_ERR_CAPACITY";
        case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE";
        case MSA_ERR_LAUNCH: return "MSA_ERR_LAUNCH";
        default: return "MSA_ERR_UNKNOWN";
    }
}

const char *msa_last_error(void) { return g_err; }

int msa_index_caps(const msa_problem *p, int32_t vertical_topk, int32_t slash_topk, int32_t block,
                   int32_t *cap_blocks, int32_t *cap_cols) {
    int st = check_problem(p);
    if (st) return st;
    if (!cap_blocks || !cap_cols) return fail(MSA_ERR_NULL, "cap outputs are NULL");
    if (block != 64) return fail(MSA_ERR_RANGE, "block must be 64 (got %d)", block);
    if (vertical_topk < 0 || vertical_topk > p->seq_len || slash_topk < 0 || slash_topk > p->seq_len)
        return fail(MSA_ERR_RANGE, "top-k values must lie in [0, seq_len]");
    const int64_t nqb = (p->seq_len + 63) / 64;
    *cap_blocks = (int32_t)(slash_topk < nqb ? slash_topk : nqb);
    *cap_cols = vertical_topk;
    return ok();
}


size_t msa_estimate_vs_workspace(const msa_problem *p, int32_t last_q, int32_t vertical_topk,
                                 int32_t slash_topk) {
    (void)vertical_topk;
    (void)slash_topk;
    if (check_problem(p) != MSA_OK || last_q != 64) return 0;
    return est_layout(p).total;
}

int msa_estimate_vs(const msa_problem *p, const void *q, const void *k, int32_t last_q,
                    int32_t vertical_topk, int32_t slash_topk, int32_t *v_idx, int32_t *s_idx,
                    float *v_score, float *s_score, void *workspace, size_t workspace_bytes,
                    void *stream) {
    int st = check_estimate_vs(p, q, k, last_q, vertical_topk, slash_topk, v_idx, s_idx, v_score, s_score);
    if (st) return st;
    if (!workspace) return fail(MSA_ERR_NULL, "a required pointer is NULL");
    if (off_align(workspace, 16)) return fail(MSA_ERR_RANGE, "workspace is not 16-byte aligned");
    const size_t need = est_layout(p).total;
    if (workspace_bytes < need)
        return fail(MSA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    return run_estimate_vs(p, q, k, vertical_topk, slash_topk, v_idx, s_idx, v_score, s_score, workspace, stream);
}

int msa_estimate_vs_noalloc(const msa_problem *p, const void *q, const void *k, int32_t last_q,
                            int32_t vertical_topk, int32_t slash_topk, int32_t *v_idx, int32_t *s_idx,
                            float *v_score, float *s_score, void *stream) {
    int st = check_estimate_vs(p, q, k, last_q, vertical_topk, slash_topk, v_idx, s_idx, v_score, s_score);
    if (st) return st;
    const size_t need = est_layout(p).total;
    if (need > kNoAllocScratchBytes)
        return fail(MSA_ERR_WORKSPACE,
                    "msa_estimate_vs_noalloc: this problem needs %zu bytes of scratch, above the %zu bytes the "
                    "library holds per GPU; split the heads over several calls or use msa_estimate_vs",
                    need, kNoAllocScratchBytes);
    void *ws = nullptr;
    if ((st = scratch_of_current_device(&ws))) return st;
    return run_estimate_vs(p, q, k, vertical_topk, slash_topk, v_idx, s_idx, v_score, s_score, ws, stream);
}

int msa_build_index(const msa_problem *p, const int32_t *v_idx, int32_t vertical_topk,
                    const int32_t *s_idx, int32_t slash_topk, int32_t block,
                    int32_t *block_count, int32_t *block_offset, int32_t cap_blocks,
                    int32_t *column_count, int32_t *column_index, int32_t cap_cols, void *stream) {
    int32_t need_b, need_c;
    int st = msa_index_caps(p, vertical_topk, slash_topk, block, &need_b, &need_c);
    if (st) return st;
    if ((vertical_topk > 0 && !v_idx) || (slash_topk > 0 && !s_idx) || !block_count || !column_count ||
        (cap_blocks > 0 && !block_offset) || (cap_cols > 0 && !column_index))
        return fail(MSA_ERR_NULL, "a required pointer is NULL");
    if (cap_blocks < need_b || cap_cols < need_c)
        return fail(MSA_ERR_CAPACITY, "capacities (%d, %d) below required (%d, %d)", cap_blocks, cap_cols,
                    need_b, need_c);
    if (off_align(v_idx, 4) || off_align(s_idx, 4) || off_align(block_count, 4) || off_align(block_offset, 4) ||
        off_align(column_count, 4) || off_align(column_index, 4))
        return fail(MSA_ERR_RANGE, "index arrays must be 4-byte aligned");
    msa::IndexArgs a;
    a.v_idx = v_idx;
    a.s_idx = s_idx;
    a.kv = vertical_topk;
    a.ks = slash_topk;
    a.n = p->seq_len;
    a.hq = p->n_q_heads;
    a.block_count = block_count;
    a.block_offset = block_offset;
    a.column_count = column_count;
    a.column_index = column_index;
    a.cap_b = cap_blocks;
    a.cap_c = cap_cols;
    a.vec_rows = (cap_blocks & 3) == 0 && !off_align(block_offset, 16);
    return launch_status(msa::launch_build_index(a, reinterpret_cast<hipStream_t>(stream)), "build_index");
}

static int attn_common(const msa_problem *p, const void *q, const void *k, const void *v, void *out,
                       msa::AttnArgs &a) {
    int st = check_problem(p);
    if (st) return st;
    if (!q || !k || !v || !out) return fail(MSA_ERR_NULL, "a required pointer is NULL");
    if ((st = check_rows(q, k, v, out))) return st;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.hq = p->n_q_heads;
    a.hkv = p->n_kv_heads;
    a.n = p->seq_len;
    a.stride = stride_of(p);
    a.scale = scale_of(p);
    a.scale_log2 = a.scale * msa::kLog2e;
    a.phase_keys = 0;
    a.k_lo = INT32_MIN;
    a.k_hi = INT32_MAX;
    a.qb_lo = 0;
    a.ws = nullptr;
    a.grp = nullptr;
    a.grp_kh = 1;
    a.v_idx = a.s_idx = nullptr;
    a.kv = a.ks = 0;
    a.fused_cov = nullptr;
    a.fused_cols = nullptr;
    a.fused_cw = 0;
    a.ex_s = a.ex_v = nullptr;
    a.ex_words = 0;
    return MSA_OK;
}

static int64_t phase_keys_of(int32_t phase_keys) {
    return phase_keys == 0 ? MSA_DEFAULT_PHASE_KEYS : phase_keys;
}

size_t msa_sparse_prefill_workspace(const msa_problem *p, int32_t phase_keys) {
    if (check_problem(p) != MSA_OK || phase_keys < 0 || phase_keys % 64 != 0) return 0;
    return msa::sparse_state_bytes(p->n_q_heads, p->seq_len, phase_keys_of(phase_keys));
}

int msa_sparse_prefill(const msa_problem *p, const void *q, const void *k, const void *v,
                       const int32_t *block_count, const int32_t *block_offset, int32_t cap_blocks,
                       const int32_t *column_count, const int32_t *column_index, int32_t cap_cols,
                       int32_t phase_keys, void *workspace, size_t workspace_bytes, void *out, float *lse,
                       void *stream) {
    msa::AttnArgs a;
    int st = attn_common(p, q, k, v, out, a);
    if (st) return st;
    if (!block_count || !column_count || (cap_blocks > 0 && !block_offset) || (cap_cols > 0 && !column_index))
        return fail(MSA_ERR_NULL, "an index pointer is NULL");
    if (cap_blocks < 0 || cap_cols < 0) return fail(MSA_ERR_CAPACITY, "negative capacity");
    if (off_align(block_count, 4) || off_align(block_offset, 4) || off_align(column_count, 4) ||
        off_align(column_index, 4) || off_align(lse, 4))
        return fail(MSA_ERR_RANGE, "index and lse arrays must be 4-byte aligned");
    a.block_count = block_count;
    a.block_offset = block_offset;
    a.column_count = column_count;
    a.column_index = column_index;
    a.cap_b = cap_blocks;
    a.cap_c = cap_cols;
    a.lse = lse;
    if (phase_keys < 0 || phase_keys % 64 != 0)
        return fail(MSA_ERR_RANGE, "phase_keys %d is not a non-negative multiple of 64", phase_keys);
    a.phase_keys = (int32_t)phase_keys_of(phase_keys);
    const size_t need = msa::sparse_state_bytes(p->n_q_heads, p->seq_len, a.phase_keys);
    if (need > 0) {
        if (!workspace) return fail(MSA_ERR_NULL, "workspace is NULL (%zu bytes needed)", need);
        if (workspace_bytes < need)
            return fail(MSA_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", workspace_bytes, need);
        if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
            return fail(MSA_ERR_RANGE, "workspace is not 16-byte aligned");
        a.ws = static_cast<float *>(workspace);
    }
    return launch_status(msa::launch_sparse_prefill(a, p->dtype, reinterpret_cast<hipStream_t>(stream)),
                         "sparse_prefill");
}

size_t msa_sparse_prefill_fused_workspace(const msa_problem *p, int32_t vertical_topk, int32_t phase_keys,
                                          int32_t flags) {
    if (check_problem(p) != MSA_OK || phase_keys < 0 || phase_keys % 64 != 0 || vertical_topk < 0 ||
        vertical_topk > msa::fused_max_columns() || (flags & ~MSA_FUSED_EXACT) != 0)
        return 0;
    return msa::fused_state_bytes(p->n_q_heads, p->seq_len, phase_keys_of(phase_keys), vertical_topk,
                                  (flags & MSA_FUSED_EXACT) != 0);
}

int msa_sparse_prefill_fused(const msa_problem *p, const void *q, const void *k, const void *v,
                             const int32_t *v_idx, int32_t vertical_topk, const int32_t *s_idx, int32_t slash_topk,
                             int32_t phase_keys, int32_t flags, void *workspace, size_t workspace_bytes, void *out,
                             float *lse, void *stream) {
    msa::AttnArgs a;
    int st = attn_common(p, q, k, v, out, a);
    if (st) return st;
    if ((vertical_topk > 0 && !v_idx) || (slash_topk > 0 && !s_idx))
        return fail(MSA_ERR_NULL, "an index set pointer is NULL");
    if (vertical_topk < 0 || slash_topk < 0 || vertical_topk > p->seq_len || slash_topk > p->seq_len)
        return fail(MSA_ERR_RANGE, "top-k values must lie in [0, seq_len]");
    if (vertical_topk > msa::fused_max_columns())
        return fail(MSA_ERR_RANGE, "the fused mode holds at most %d columns per head (got %d)",
                    msa::fused_max_columns(), vertical_topk);
    if (off_align(v_idx, 4) || off_align(s_idx, 4) || off_align(lse, 4))
        return fail(MSA_ERR_RANGE, "index sets and lse must be 4-byte aligned");
    if (phase_keys < 0 || phase_keys % 64 != 0)
        return fail(MSA_ERR_RANGE, "phase_keys %d is not a non-negative multiple of 64", phase_keys);
    if ((flags & ~MSA_FUSED_EXACT) != 0) return fail(MSA_ERR_RANGE, "unknown flags 0x%x", (unsigned)flags);
    const bool exact = (flags & MSA_FUSED_EXACT) != 0;
    a.phase_keys = (int32_t)phase_keys_of(phase_keys);
    if (a.phase_keys > msa::fused_max_phase_keys())
        return fail(MSA_ERR_RANGE, "the fused mode takes phases of at most %d keys (got %d)",
                    msa::fused_max_phase_keys(), a.phase_keys);
    a.block_count = a.block_offset = a.column_count = a.column_index = nullptr;
    a.cap_b = a.cap_c = 0;
    a.lse = lse;
    a.v_idx = v_idx;
    a.s_idx = s_idx;
    a.kv = vertical_topk;
    a.ks = slash_topk;
    const size_t need = msa::fused_state_bytes(p->n_q_heads, p->seq_len, a.phase_keys, vertical_topk, exact);
    if (need > 0) {
        if (!workspace) return fail(MSA_ERR_NULL, "workspace is NULL (%zu bytes needed)", need);
        if (workspace_bytes < need)
            return fail(MSA_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", workspace_bytes, need);
        if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
            return fail(MSA_ERR_RANGE, "workspace is not 16-byte aligned");
        a.ws = static_cast<float *>(workspace);
    }
    return launch_status(msa::launch_sparse_prefill_fused(a, p->dtype, exact, reinterpret_cast<hipStream_t>(stream)),
                         "sparse_prefill_fused");
}

size_t msa_decode_sparse_workspace(const msa_problem *p) {
    if (check_problem(p) != MSA_OK) return 0;
    return decode_layout(p).total;
}

static int run_decode_sparse(const msa_problem *p, const void *q, const void *k, const void *v,
                             const int32_t *cache_lens, int32_t topk, int32_t *idx, int32_t flags, void *workspace,
                             size_t workspace_bytes, void *out, float *lse, float *recovery, void *stream) {
    int st = check_problem(p);
    if (st) return st;
    if (!q || !k || !v || !out || !idx) return fail(MSA_ERR_NULL, "a required pointer is NULL");
    if ((st = check_rows(q, k, v, out))) return st;
    if ((flags & ~MSA_DECODE_GIVEN_KEYS) != 0) return fail(MSA_ERR_RANGE, "unknown flags 0x%x", (unsigned)flags);
    if (topk < 1 || topk > p->seq_len) return fail(MSA_ERR_RANGE, "topk must lie in [1, seq_len] (got %d)", topk);
    if (off_align(idx, 4) || off_align(lse, 4) || off_align(recovery, 4) || off_align(cache_lens, 4))
        return fail(MSA_ERR_RANGE, "idx, lse, recovery and cache_lens must be 4-byte aligned");
    const DecodeLayout L = decode_layout(p);
    if (!workspace) return fail(MSA_ERR_NULL, "workspace is NULL (%zu bytes needed)", L.total);
    if (workspace_bytes < L.total) return fail(MSA_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", workspace_bytes, L.total);
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return fail(MSA_ERR_RANGE, "workspace is not 16-byte aligned");
    msa::DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.recovery = recovery;
    a.hq = p->n_q_heads;
    a.hkv = p->n_kv_heads;
    a.n = p->seq_len;
    a.stride = stride_of(p);
    a.scale_log2 = scale_of(p) * msa::kLog2e;
    a.topk = topk;
    a.idx = idx;
    a.keys = at<uint32_t>(workspace, L.off_keys);
    a.part = at<float>(workspace, L.off_part);
    a.lse2_all = at<float>(workspace, L.off_lse);
    a.chunk_keys = L.chunk_keys;
    a.nchunks = L.nchunks;
    a.lens = cache_lens;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if ((st = launch_status(msa::launch_decode_scores(a, p->dtype, s), "decode scores"))) return st;
    if ((flags & MSA_DECODE_GIVEN_KEYS) == 0) {
        msa::TopkArgs t;
        t.src0 = t.src1 = reinterpret_cast<const float *>(a.keys);
        t.dst0 = t.dst1 = idx;
        t.k0 = t.k1 = topk;
        t.hq = p->n_q_heads;
        t.rows = p->n_q_heads;
        t.n = p->seq_len;
        t.nslices = L.nslices;
        t.hist = at<uint32_t>(workspace, L.off_hist);
        t.state = at<uint32_t>(workspace, L.off_state);
        t.cnt = at<uint32_t>(workspace, L.off_cnt);
        t.off = at<uint32_t>(workspace, L.off_off);
        t.row_len = cache_lens;                      // q head h reads kv head h / G's cache
        t.row_len_div = p->n_q_heads / p->n_kv_heads;
        // one workgroup per row once there are rows for half the chip; fewer
        // rows are split into slices across the chip
        const hipError_t e = t.rows >= 128 ? msa::launch_topk_rows(t, s) : msa::launch_topk(t, s);
        if ((st = launch_status(e, "decode top-k"))) return st;
    }
    return launch_status(msa::launch_decode_attend(a, p->dtype, s), "decode attend");
}

int msa_decode_sparse(const msa_problem *p, const void *q, const void *k, const void *v, int32_t topk,
                      int32_t *idx, int32_t flags, void *workspace, size_t workspace_bytes, void *out, float *lse,
                      float *recovery, void *stream) {
    return run_decode_sparse(p, q, k, v, nullptr, topk, idx, flags, workspace, workspace_bytes, out, lse, recovery,
                             stream);
}

int msa_decode_sparse_varlen(const msa_problem *p, const void *q, const void *k, const void *v,
                             const int32_t *cache_lens, int32_t topk, int32_t *idx, int32_t flags, void *workspace,
                             size_t workspace_bytes, void *out, float *lse, float *recovery, void *stream) {
    if (!cache_lens) return fail(MSA_ERR_NULL, "cache_lens is NULL");
    return run_decode_sparse(p, q, k, v, cache_lens, topk, idx, flags, workspace, workspace_bytes, out, lse,
                             recovery, stream);
}

int msa_sparse_prefill_walk_marks(const msa_problem *p, int32_t phase_keys, size_t *offset,
                                  int32_t *heads_per_unit) {
    int st = check_problem(p);
    if (st) return st;
    if (!offset || !heads_per_unit) return fail(MSA_ERR_NULL, "outputs are NULL");
    if (phase_keys < 0 || phase_keys % 64 != 0)
        return fail(MSA_ERR_RANGE, "phase_keys %d is not a non-negative multiple of 64", phase_keys);
    if (msa::sparse_state_bytes(p->n_q_heads, p->seq_len, phase_keys_of(phase_keys)) == 0) {
        *offset = 0;
        *heads_per_unit = 0;
    } else {
        *offset = msa::sparse_walk_marks_offset(p->n_q_heads, p->seq_len);
        *heads_per_unit = msa::walk_heads_per_unit(p->n_q_heads, p->n_kv_heads);
    }
    return ok();
}

int msa_dense_prefill(const msa_problem *p, const void *q, const void *k, const void *v, void *out,
                      float *lse, void *stream) {
    msa::AttnArgs a;
    int st = attn_common(p, q, k, v, out, a);
    if (st) return st;
    if (off_align(lse, 4)) return fail(MSA_ERR_RANGE, "lse must be 4-byte aligned");
    a.block_count = a.block_offset = a.column_count = a.column_index = nullptr;
    a.cap_b = a.cap_c = 0;
    a.lse = lse;
    return launch_status(msa::launch_dense_prefill(a, p->dtype, reinterpret_cast<hipStream_t>(stream)),
                         "dense_prefill");
}

// ---- Packed batches of sequences of different lengths ----

// heads of all sequences together: the kernels' grids index them in their
// second dimension (the top-k's rows are twice this many)
constexpr int64_t kMaxVarlenHeads = 32767;

static int check_varlen(const msa_problem *p, const msa_varlen *vl, msa::Varlen &out) {
    int st = check_problem(p);
    if (st) return st;
    if (!vl || !vl->cu_seqlens) return fail(MSA_ERR_NULL, "the varlen descriptor or its cu_seqlens is NULL");
    if (off_align(vl->cu_seqlens, 4)) return fail(MSA_ERR_RANGE, "cu_seqlens must be 4-byte aligned");
    if (vl->n_seqs < 1) return fail(MSA_ERR_SHAPE, "n_seqs must be at least 1 (got %d)", vl->n_seqs);
    if ((int64_t)vl->n_seqs * p->n_q_heads > kMaxVarlenHeads)
        return fail(MSA_ERR_SHAPE, "n_seqs * n_q_heads must be at most %lld (got %lld)", (long long)kMaxVarlenHeads,
                    (long long)vl->n_seqs * p->n_q_heads);
    if (vl->max_seqlen < 1 || vl->max_seqlen > p->seq_len)
        return fail(MSA_ERR_SHAPE, "max_seqlen must lie in [1, seq_len] (got %d)", vl->max_seqlen);
    out.cu = vl->cu_seqlens;
    out.nseq = vl->n_seqs;
    out.rows = p->seq_len;
    return MSA_OK;
}

size_t msa_estimate_vs_varlen_workspace(const msa_problem *p, const msa_varlen *vl, int32_t last_q) {
    msa::Varlen V;
    if (check_varlen(p, vl, V) != MSA_OK || last_q != 64) return 0;
    return est_layout_for((int64_t)p->n_q_heads * V.nseq, (int64_t)p->n_kv_heads * V.nseq, vl->max_seqlen, V.nseq)
        .total;
}

int msa_estimate_vs_varlen(const msa_problem *p, const msa_varlen *vl, const void *q, const void *k, int32_t last_q,
                           int32_t vertical_topk, int32_t slash_topk, int32_t *v_idx, int32_t *s_idx, void *workspace,
                           size_t workspace_bytes, void *stream) {
    msa::Varlen V;
    int st = check_varlen(p, vl, V);
    if (st) return st;
    if (!q || !k || !v_idx || !s_idx || !workspace) return fail(MSA_ERR_NULL, "a required pointer is NULL");
    if ((st = check_rows(q, k, nullptr, nullptr))) return st;
    if (off_align(v_idx, 4) || off_align(s_idx, 4)) return fail(MSA_ERR_RANGE, "index arrays must be 4-byte aligned");
    if (off_align(workspace, 16)) return fail(MSA_ERR_RANGE, "workspace is not 16-byte aligned");
    if (last_q != 64) return fail(MSA_ERR_RANGE, "last_q must be 64 (got %d)", last_q);
    if (vertical_topk < 1 || vertical_topk > vl->max_seqlen || slash_topk < 1 || slash_topk > vl->max_seqlen)
        return fail(MSA_ERR_RANGE, "top-k values must lie in [1, max_seqlen]");
    const size_t need = msa_estimate_vs_varlen_workspace(p, vl, last_q);
    if (workspace_bytes < need)
        return fail(MSA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    return run_estimate_vs(p, q, k, vertical_topk, slash_topk, v_idx, s_idx, nullptr, nullptr, workspace, stream, &V,
                           vl->max_seqlen);
}

int msa_build_index_varlen(const msa_problem *p, const msa_varlen *vl, const int32_t *v_idx, int32_t vertical_topk,
                           const int32_t *s_idx, int32_t slash_topk, int32_t block, int32_t *block_count,
                           int32_t *block_offset, int32_t cap_blocks, int32_t *column_count, int32_t *column_index,
                           int32_t cap_cols, void *stream) {
    msa::Varlen V;
    int st = check_varlen(p, vl, V);
    if (st) return st;
    msa_problem one = *p;                          // the per-head arrays' geometry: the longest sequence
    one.seq_len = vl->max_seqlen;
    one.seq_stride = 0;
    int32_t need_b, need_c;
    if ((st = msa_index_caps(&one, vertical_topk, slash_topk, block, &need_b, &need_c))) return st;
    if ((vertical_topk > 0 && !v_idx) || (slash_topk > 0 && !s_idx) || !block_count || !column_count ||
        (cap_blocks > 0 && !block_offset) || (cap_cols > 0 && !column_index))
        return fail(MSA_ERR_NULL, "a required pointer is NULL");
    if (cap_blocks < need_b || cap_cols < need_c)
        return fail(MSA_ERR_CAPACITY, "capacities (%d, %d) below required (%d, %d)", cap_blocks, cap_cols,
                    need_b, need_c);
    if (off_align(v_idx, 4) || off_align(s_idx, 4) || off_align(block_count, 4) || off_align(block_offset, 4) ||
        off_align(column_count, 4) || off_align(column_index, 4))
        return fail(MSA_ERR_RANGE, "index arrays must be 4-byte aligned");
    msa::IndexArgs a;
    a.v_idx = v_idx;
    a.s_idx = s_idx;
    a.kv = vertical_topk;
    a.ks = slash_topk;
    a.n = vl->max_seqlen;
    a.hq = p->n_q_heads;
    a.block_count = block_count;
    a.block_offset = block_offset;
    a.column_count = column_count;
    a.column_index = column_index;
    a.cap_b = cap_blocks;
    a.cap_c = cap_cols;
    a.vec_rows = (cap_blocks & 3) == 0 && !off_align(block_offset, 16);
    a.vl = V;
    return launch_status(msa::launch_build_index(a, reinterpret_cast<hipStream_t>(stream)), "build_index_varlen");
}

size_t msa_sparse_prefill_varlen_workspace(const msa_problem *p, const msa_varlen *vl, int32_t phase_keys) {
    msa::Varlen V;
    if (check_varlen(p, vl, V) != MSA_OK || phase_keys < 0 || phase_keys % 64 != 0) return 0;
    return msa::sparse_state_bytes((int64_t)p->n_q_heads * V.nseq, vl->max_seqlen, phase_keys_of(phase_keys));
}

int msa_sparse_prefill_varlen(const msa_problem *p, const msa_varlen *vl, const void *q, const void *k, const void *v,
                              const int32_t *block_count, const int32_t *block_offset, int32_t cap_blocks,
                              const int32_t *column_count, const int32_t *column_index, int32_t cap_cols,
                              int32_t phase_keys, void *workspace, size_t workspace_bytes, void *out, float *lse,
                              void *stream) {
    msa::Varlen V;
    int st = check_varlen(p, vl, V);
    if (st) return st;
    msa::AttnArgs a;
    if ((st = attn_common(p, q, k, v, out, a))) return st;
    if (!block_count || !column_count || (cap_blocks > 0 && !block_offset) || (cap_cols > 0 && !column_index))
        return fail(MSA_ERR_NULL, "an index pointer is NULL");
    if (cap_blocks < 0 || cap_cols < 0) return fail(MSA_ERR_CAPACITY, "negative capacity");
    if (off_align(block_count, 4) || off_align(block_offset, 4) || off_align(column_count, 4) ||
        off_align(column_index, 4) || off_align(lse, 4))
        return fail(MSA_ERR_RANGE, "index and lse arrays must be 4-byte aligned");
    if (phase_keys < 0 || phase_keys % 64 != 0)
        return fail(MSA_ERR_RANGE, "phase_keys %d is not a non-negative multiple of 64", phase_keys);
    a.n = vl->max_seqlen;
    a.vl = V;
    a.block_count = block_count;
    a.block_offset = block_offset;
    a.column_count = column_count;
    a.column_index = column_index;
    a.cap_b = cap_blocks;
    a.cap_c = cap_cols;
    a.lse = lse;
    a.phase_keys = (int32_t)phase_keys_of(phase_keys);
    const size_t need = msa::sparse_state_bytes((int64_t)p->n_q_heads * V.nseq, a.n, a.phase_keys);
    if (need > 0) {
        if (!workspace) return fail(MSA_ERR_NULL, "workspace is NULL (%zu bytes needed)", need);
        if (workspace_bytes < need)
            return fail(MSA_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", workspace_bytes, need);
        if (off_align(workspace, 16)) return fail(MSA_ERR_RANGE, "workspace is not 16-byte aligned");
        a.ws = static_cast<float *>(workspace);
    }
    return launch_status(msa::launch_sparse_prefill(a, p->dtype, reinterpret_cast<hipStream_t>(stream)),
                         "sparse_prefill_varlen");
}

int msa_dense_prefill_varlen(const msa_problem *p, const msa_varlen *vl, const void *q, const void *k, const void *v,
                             void *out, float *lse, void *stream) {
    msa::Varlen V;
    int st = check_varlen(p, vl, V);
    if (st) return st;
    msa::AttnArgs a;
    if ((st = attn_common(p, q, k, v, out, a))) return st;
    if (off_align(lse, 4)) return fail(MSA_ERR_RANGE, "lse must be 4-byte aligned");
    a.n = vl->max_seqlen;
    a.vl = V;
    a.block_count = a.block_offset = a.column_count = a.column_index = nullptr;
    a.cap_b = a.cap_c = 0;
    a.lse = lse;
    return launch_status(msa::launch_dense_prefill(a, p->dtype, reinterpret_cast<hipStream_t>(stream)),
                         "dense_prefill_varlen");
}

// block-sparse workspace: pooled q and k means, then the score keys of one
// chunk of query blocks
static size_t bs_chunk_rows(int64_t nb) { return (size_t)(nb < msa::kBsChunkRows ? nb : msa::kBsChunkRows); }

// hq, hkv: heads of all sequences; n: the longest sequence
static size_t bs_workspace(int64_t hq, int64_t hkv, int64_t n) {
    const size_t nb = (size_t)((n + 63) / 64);
    return align_up((size_t)hq * nb * 128 * 4) + align_up((size_t)hkv * nb * 128 * 4) +
           align_up((size_t)hq * bs_chunk_rows((int64_t)nb) * nb * 4);
}

size_t msa_estimate_bs_workspace(const msa_problem *p, int32_t block) {
    if (check_problem(p) != MSA_OK || block != 64) return 0;
    return bs_workspace(p->n_q_heads, p->n_kv_heads, p->seq_len);
}

static int run_estimate_bs(const msa_problem *p, const msa::Varlen *vl, int64_t n, const void *q, const void *k,
                           int32_t block, int32_t topk_blocks, int32_t *block_count, int32_t *block_offset,
                           int32_t cap_blocks, int32_t *column_count, void *workspace, size_t workspace_bytes,
                           void *stream) {
    int st;
    if (!q || !k || !block_count || !block_offset || !column_count || !workspace)
        return fail(MSA_ERR_NULL, "a required pointer is NULL");
    if ((st = check_rows(q, k, nullptr, nullptr))) return st;
    if (off_align(block_count, 4) || off_align(block_offset, 4) || off_align(column_count, 4))
        return fail(MSA_ERR_RANGE, "index arrays must be 4-byte aligned");
    if (off_align(workspace, 16)) return fail(MSA_ERR_RANGE, "workspace is not 16-byte aligned");
    if (block != 64) return fail(MSA_ERR_RANGE, "block must be 64 (got %d)", block);
    const int64_t nb = (n + 63) / 64;
    if (topk_blocks < 1) return fail(MSA_ERR_RANGE, "topk_blocks must be >= 1");
    const int64_t need = topk_blocks < nb ? topk_blocks : nb;
    if (cap_blocks < need) return fail(MSA_ERR_CAPACITY, "cap_blocks %d below %lld", cap_blocks, (long long)need);
    const int64_t nseq = vl ? vl->nseq : 1;
    const size_t ws = bs_workspace(p->n_q_heads * nseq, p->n_kv_heads * nseq, n);
    if (workspace_bytes < ws) return fail(MSA_ERR_WORKSPACE, "workspace too small: %zu < %zu", workspace_bytes, ws);
    msa::BsArgs a;
    a.q = q;
    a.k = k;
    a.n = n;
    a.stride = stride_of(p);
    a.hq = p->n_q_heads;
    a.hkv = p->n_kv_heads;
    if (vl) a.vl = *vl;
    a.scale = scale_of(p);
    a.topk = topk_blocks;
    a.qm = at<float>(workspace, 0);
    a.km = at<float>(workspace, align_up((size_t)(p->n_q_heads * nseq) * nb * 128 * 4));
    a.keys = at<uint32_t>(workspace, align_up((size_t)(p->n_q_heads * nseq) * nb * 128 * 4) +
                                         align_up((size_t)(p->n_kv_heads * nseq) * nb * 128 * 4));
    a.chunk_rows = (int32_t)bs_chunk_rows(nb);    // the workspace holds this many rows of keys
    a.row0 = 0;
    a.block_count = block_count;
    a.block_offset = block_offset;
    a.column_count = column_count;
    a.cap_b = cap_blocks;
    return launch_status(msa::launch_estimate_bs(a, p->dtype, reinterpret_cast<hipStream_t>(stream)),
                         "estimate_bs");
}

int msa_estimate_bs(const msa_problem *p, const void *q, const void *k, int32_t block, int32_t topk_blocks,
                    int32_t *block_count, int32_t *block_offset, int32_t cap_blocks, int32_t *column_count,
                    void *workspace, size_t workspace_bytes, void *stream) {
    const int st = check_problem(p);
    if (st) return st;
    return run_estimate_bs(p, nullptr, p->seq_len, q, k, block, topk_blocks, block_count, block_offset, cap_blocks,
                           column_count, workspace, workspace_bytes, stream);
}

size_t msa_estimate_bs_varlen_workspace(const msa_problem *p, const msa_varlen *vl, int32_t block) {
    msa::Varlen V;
    if (check_varlen(p, vl, V) != MSA_OK || block != 64) return 0;
    return bs_workspace((int64_t)p->n_q_heads * V.nseq, (int64_t)p->n_kv_heads * V.nseq, vl->max_seqlen);
}

int msa_estimate_bs_varlen(const msa_problem *p, const msa_varlen *vl, const void *q, const void *k, int32_t block,
                           int32_t topk_blocks, int32_t *block_count, int32_t *block_offset, int32_t cap_blocks,
                           int32_t *column_count, void *workspace, size_t workspace_bytes, void *stream) {
    msa::Varlen V;
    const int st = check_varlen(p, vl, V);
    if (st) return st;
    return run_estimate_bs(p, &V, vl->max_seqlen, q, k, block, topk_blocks, block_count, block_offset, cap_blocks,
                           column_count, workspace, workspace_bytes, stream);
}

}  // extern "C"
