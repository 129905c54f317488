// C ABI of libqsa: argument validation, error reporting and dispatch.
// Every entry point validates on the host before anything is enqueued; on
// error nothing is enqueued, outputs are untouched and qsa_last_error()
// names the offending argument and the limit.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <set>
#include <tuple>

#include "qsa_debug.hpp"
#include "qsa_internal.hpp"
#include "qsa_lists.hpp"

namespace qsa {

static thread_local char g_err[512] = "";

static qsa_status fail(qsa_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    if (trace_enabled()) fprintf(stderr, "[qsa] error %d: %s\n", (int)s, g_err);
    return s;
}

static qsa_status ok() {
    g_err[0] = '\0';
    return QSA_OK;
}

static qsa_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(QSA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

hipError_t enable_dyn_lds(const void *fn, int bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::mutex mu;
    static std::set<std::tuple<int, const void *, int>> done;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count(std::make_tuple(dev, fn, bytes))) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done.insert(std::make_tuple(dev, fn, bytes));
    return e;
}

bool trace_enabled() {
    static int v = -1;
    if (v < 0) {
        const char *s = getenv("QSA_TRACE");
        v = (s && s[0] && s[0] != '0') ? 1 : 0;
    }
    return v == 1;
}

void trace(const char *fmt, ...) {
    if (!trace_enabled()) return;
    va_list ap;
    va_start(ap, fmt);
    fprintf(stderr, "[qsa] ");
    vfprintf(stderr, fmt, ap);
    fprintf(stderr, "\n");
    va_end(ap);
}

static bool env_flag(const char *name) {
    const char *s = getenv(name);
    return s && s[0] && s[0] != '0';
}

// QSA_DEBUG=1: device-side argument contents are checked before every
// launch, and every call waits for its kernels (so that a fault is reported
// by the call that caused it).  Read on every call, so a process can switch
// it on and off; a call in debug mode synchronises and cannot be captured in
// a graph.
static bool debug_enabled() { return env_flag("QSA_DEBUG"); }

// QSA_TEST_FORCE_LAUNCH_ERROR=1: every entry point that passes host
// validation returns QSA_ERR_HIP without touching a device (a test hook for
// the error path of a failed launch).
static bool forced_launch_error() { return env_flag("QSA_TEST_FORCE_LAUNCH_ERROR"); }

static const char *debug_check_name(int32_t code) {
    switch (code) {
    case QSA_DBG_KV_OFFSETS: return "kv_offsets: offsets[0] != 0, a negative length or a length past max_kv_len";
    case QSA_DBG_BLK_OFFSETS: return "blk_offsets: not the prefix sums of floor(N_s/ratio)";
    case QSA_DBG_Q_OFFSETS:
        return "q_offsets: offsets[0] != 0, offsets[B] != total_q, or a query count below 0, above N_s or above "
               "max_q_per_seq";
    case QSA_DBG_IDX_RANGE: return "idx: a selected block id outside [-1, floor(L/ratio))";
    case QSA_DBG_PAGE_ID: return "block_table: a page id outside [0, num_pages)";
    default: return "unknown check";
    }
}

// What the debug check reads for a call on batch b (blk: the call reads
// blk_offsets; pg: the paging descriptor or NULL).
static DebugCheck batch_check(const qsa_batch &b, int32_t ratio, bool blk, const qsa_paged_kv *pg) {
    DebugCheck c;
    c.kv_off = b.kv_offsets;
    c.blk_off = blk ? b.blk_offsets : nullptr;
    c.q_off = b.q_offsets;
    c.num_seqs = b.num_seqs;
    c.max_q_per_seq = b.q_offsets ? b.max_q_per_seq : 1;
    c.total_q = b.total_q;
    c.max_kv_len = b.max_kv_len;
    c.log2r = ratio > 0 ? __builtin_ctz((unsigned)ratio) : 0;
    if (pg) {
        c.table = pg->block_table;
        c.max_pages = pg->max_pages;
        c.num_pages = pg->num_pages;
        c.page_size = pg->page_size;
    }
    return c;
}

// Run one validated call's launches: the forced-error hook, the debug check
// of device contents (nothing of the call is launched on a violation), the
// launch itself and, in debug mode, a wait for it.
template <typename F>
static qsa_status launch_checked(const char *what, const DebugCheck &dc, void *stream, F &&launch) {
    if (forced_launch_error())
        return fail(QSA_ERR_HIP, "%s: launch failed (forced by QSA_TEST_FORCE_LAUNCH_ERROR)", what);
    hipStream_t st = (hipStream_t)stream;
    const bool dbg = debug_enabled();
    if (dbg) {
        int32_t code = 0;
        int64_t where = 0, value = 0;
        hipError_t e = launch_debug_check(dc, st);
        if (e == hipSuccess) e = read_debug_status(st, code, where, value);
        if (e != hipSuccess) return hip_status(e, what);
        if (code != 0)
            return fail(QSA_ERR_DEVICE_ASSERT,
                        "%s: debug check failed: %s (sequence or query %lld, value %lld); nothing was launched",
                        what, debug_check_name(code), (long long)where, (long long)value);
        trace("%s: debug check passed", what);
    }
    hipError_t e = launch(st);
    if (e == hipSuccess && dbg) e = hipStreamSynchronize(st);
    return hip_status(e, what);
}

static bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Largest number of complete blocks one row may hold (top-k keeps at most
// 128 per thread of a 1024-thread workgroup).
static constexpr int64_t kMaxBlocksPerRow = 131072;

static qsa_status check_batch(const qsa_batch *b, bool need_blk) {
    if (!b) return fail(QSA_ERR_INVALID_ARGUMENT, "batch is NULL");
    if (b->num_seqs < 1) return fail(QSA_ERR_INVALID_ARGUMENT, "batch.num_seqs=%d must be >= 1", b->num_seqs);
    if (b->num_seqs > 65535)
        return fail(QSA_ERR_UNSUPPORTED, "batch.num_seqs=%d exceeds 65535", b->num_seqs);
    if (!b->kv_offsets) return fail(QSA_ERR_INVALID_ARGUMENT, "batch.kv_offsets is NULL");
    if (need_blk && !b->blk_offsets) return fail(QSA_ERR_INVALID_ARGUMENT, "batch.blk_offsets is NULL");
    if (b->max_kv_len < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "batch.max_kv_len=%lld < 0", (long long)b->max_kv_len);
    if (b->total_q < 0) return fail(QSA_ERR_INVALID_ARGUMENT, "batch.total_q=%lld < 0", (long long)b->total_q);
    if (b->q_offsets == nullptr && b->total_q != b->num_seqs)
        return fail(QSA_ERR_INVALID_ARGUMENT,
                    "batch.q_offsets is NULL (one query per sequence) but total_q=%lld != num_seqs=%d",
                    (long long)b->total_q, b->num_seqs);
    if (b->q_offsets != nullptr && b->max_q_per_seq < 1 && b->total_q > 0)
        return fail(QSA_ERR_INVALID_ARGUMENT, "batch.max_q_per_seq=%d must be >= 1", b->max_q_per_seq);
    if (b->total_q > 0x7fffffffLL)
        return fail(QSA_ERR_UNSUPPORTED, "batch.total_q=%lld exceeds 2^31-1", (long long)b->total_q);
    return ok();
}

static qsa_status check_ratio(int32_t ratio) {
    if (!is_pow2(ratio) || ratio > 64)
        return fail(QSA_ERR_UNSUPPORTED, "ratio=%d must be a power of two in [1, 64]", ratio);
    return ok();
}

static qsa_status check_budget(int32_t budget, int32_t ratio) {
    qsa_status s = check_ratio(ratio);
    if (s != QSA_OK) return s;
    if (budget <= 0 || budget % ratio != 0)
        return fail(QSA_ERR_UNSUPPORTED, "budget=%d must be a positive multiple of ratio=%d", budget, ratio);
    const int32_t K = budget / ratio;
    if (K < 1 || K > 2048)
        return fail(QSA_ERR_UNSUPPORTED, "budget/ratio=%d must be in [1, 2048]", K);
    return ok();
}

static qsa_status check_rows(const qsa_batch *b, int32_t ratio) {
    const int64_t max_nb = b->max_kv_len / ratio;
    if (max_nb > kMaxBlocksPerRow)
        return fail(QSA_ERR_UNSUPPORTED,
                    "max_kv_len/ratio=%lld exceeds %lld complete blocks per sequence",
                    (long long)max_nb, (long long)kMaxBlocksPerRow);
    return ok();
}

static qsa_status check_indexer(const qsa_indexer *ix, bool mfma) {
    if (!ix) return fail(QSA_ERR_INVALID_ARGUMENT, "indexer is NULL");
    if (!ix->q_idx) return fail(QSA_ERR_INVALID_ARGUMENT, "indexer.q_idx is NULL");
    if (!ix->w) return fail(QSA_ERR_INVALID_ARGUMENT, "indexer.w is NULL");
    if (!ix->kc) return fail(QSA_ERR_INVALID_ARGUMENT, "indexer.kc is NULL");
    if (ix->q_dtype != QSA_F32 && ix->q_dtype != QSA_BF16)
        return fail(QSA_ERR_UNSUPPORTED, "indexer.q_dtype=%d must be QSA_F32 or QSA_BF16", ix->q_dtype);
    if (ix->kc_dtype != QSA_F32 && ix->kc_dtype != QSA_BF16 && ix->kc_dtype != QSA_FP8_E4M3 &&
        ix->kc_dtype != QSA_FP4_E2M1)
        return fail(QSA_ERR_UNSUPPORTED, "indexer.kc_dtype=%d is not a qsa_dtype", ix->kc_dtype);
    const bool scaled = ix->kc_dtype == QSA_FP8_E4M3 || ix->kc_dtype == QSA_FP4_E2M1;
    if (scaled && !ix->kc_scale)
        return fail(QSA_ERR_INVALID_ARGUMENT, "indexer.kc_scale is NULL but kc_dtype=%d needs scales",
                    ix->kc_dtype);
    if (!scaled && ix->kc_scale)
        return fail(QSA_ERR_INVALID_ARGUMENT,
                    "indexer.kc_scale must be NULL unless kc_dtype is QSA_FP8_E4M3 or QSA_FP4_E2M1");
    if (ix->kc_dtype == QSA_FP4_E2M1 && ix->q_dtype != QSA_BF16)
        return fail(QSA_ERR_UNSUPPORTED, "fp4 compressed keys need a bf16 q_idx (q_dtype=%d)", ix->q_dtype);
    if (ix->h_idx != 1 && ix->h_idx != 2 && ix->h_idx != 4 && ix->h_idx != 8 && ix->h_idx != 16)
        return fail(QSA_ERR_UNSUPPORTED, "indexer.h_idx=%d must be 1, 2, 4, 8 or 16", ix->h_idx);
    if (ix->d_idx != 64 && ix->d_idx != 128)
        return fail(QSA_ERR_UNSUPPORTED, "indexer.d_idx=%d must be 64 or 128", ix->d_idx);
    if (mfma && (ix->q_dtype != QSA_BF16 || ix->kc_dtype != QSA_BF16))
        return fail(QSA_ERR_UNSUPPORTED, "QSA_SCORE_MFMA needs bf16 q_idx and bf16 kc");
    return ok();
}

static qsa_status check_attn(const qsa_attn *a) {
    if (!a) return fail(QSA_ERR_INVALID_ARGUMENT, "attn is NULL");
    if (!a->q || !a->k || !a->v) return fail(QSA_ERR_INVALID_ARGUMENT, "attn.q/k/v must not be NULL");
    if (a->dtype != QSA_F32 && a->dtype != QSA_BF16)
        return fail(QSA_ERR_UNSUPPORTED, "attn.dtype=%d must be QSA_F32 or QSA_BF16", a->dtype);
    if (a->hq < 1 || a->hkv < 1 || a->hq % a->hkv != 0)
        return fail(QSA_ERR_INVALID_ARGUMENT, "attn.hq=%d must be a positive multiple of attn.hkv=%d", a->hq, a->hkv);
    const int G = a->hq / a->hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
        return fail(QSA_ERR_UNSUPPORTED, "attn.hq/attn.hkv=%d must be 1, 2, 4, 8 or 16", G);
    if (a->d != 128) return fail(QSA_ERR_UNSUPPORTED, "attn.d=%d must be 128", a->d);
    if (!(a->softmax_scale > 0.0f) || a->softmax_scale > 1e30f)
        return fail(QSA_ERR_INVALID_ARGUMENT, "attn.softmax_scale must be finite and > 0");
    return ok();
}

// Paged caches: the descriptor and the batch it must cover.  Pool rows stay
// below 2^31 (the kernels index rows with 32-bit integers).
static qsa_status check_paging(const qsa_paged_kv *pg, const qsa_batch *b, int32_t ratio) {
    if (!pg) return fail(QSA_ERR_INVALID_ARGUMENT, "paging descriptor is NULL");
    if (!pg->block_table) return fail(QSA_ERR_INVALID_ARGUMENT, "paging.block_table is NULL");
    if (!is_pow2(pg->page_size) || pg->page_size < ratio)
        return fail(QSA_ERR_INVALID_ARGUMENT,
                    "paging.page_size=%d must be a power of two and a multiple of ratio=%d", pg->page_size, ratio);
    if (pg->num_pages < 1) return fail(QSA_ERR_INVALID_ARGUMENT, "paging.num_pages=%lld must be >= 1",
                                       (long long)pg->num_pages);
    if (pg->num_pages > (0x7fffffffLL / pg->page_size))
        return fail(QSA_ERR_UNSUPPORTED, "paging: num_pages*page_size=%lld exceeds 2^31-1 pool rows",
                    (long long)(pg->num_pages * pg->page_size));
    const int64_t need = (b->max_kv_len + pg->page_size - 1) / pg->page_size;
    if (pg->max_pages < need || pg->max_pages < 1)
        return fail(QSA_ERR_INVALID_ARGUMENT, "paging.max_pages=%lld must be >= ceil(max_kv_len/page_size)=%lld",
                    (long long)pg->max_pages, (long long)need);
    return ok();
}

// Host validation of an attention call, workspace excluded.
static qsa_status attn_validate(const qsa_attn *a, const int32_t *idx, int32_t budget, int32_t ratio,
                                const qsa_batch *b, void *out, bool decode, const qsa_paged_kv *pg) {
    qsa_status s = check_attn(a);
    if (s == QSA_OK) s = check_batch(b, false);
    if (s == QSA_OK && pg) s = check_paging(pg, b, ratio);
    if (s == QSA_OK) s = check_budget(budget, ratio);
    if (s != QSA_OK) return s;
    if (!idx) return fail(QSA_ERR_INVALID_ARGUMENT, "idx is NULL");
    if (!out) return fail(QSA_ERR_INVALID_ARGUMENT, "out is NULL");
    if (decode && b->q_offsets != nullptr && b->max_q_per_seq != 1)
        return fail(QSA_ERR_INVALID_ARGUMENT,
                    "decode takes one query per sequence (q_offsets NULL or max_q_per_seq == 1); "
                    "use qsa_sparse_attn_prefill for max_q_per_seq=%d", b->max_q_per_seq);
    return ok();
}

// Launch a validated attention call (ws: at least attn_workspace_bytes for decode).
static qsa_status attn_launch(const qsa_attn *a, const int32_t *idx, int32_t budget, int32_t ratio,
                              const qsa_batch *b, void *out, void *ws, bool decode, const qsa_paged_kv *pg,
                              void *st) {
    DebugCheck dc = batch_check(*b, ratio, false, pg);
    dc.idx = idx;
    dc.ldi = budget / ratio;
    return launch_checked(decode ? "qsa_sparse_attn_decode" : "qsa_sparse_attn_prefill", dc, st,
                          [&](hipStream_t s_) { return launch_attn(*a, idx, budget, ratio, *b, out, ws, decode, pg, s_); });
}

static qsa_status attn_common(const qsa_attn *a, const int32_t *idx, int32_t budget, int32_t ratio,
                              const qsa_batch *b, void *out, void *ws, size_t ws_bytes, bool decode,
                              const qsa_paged_kv *pg, hipStream_t st) {
    qsa_status s = attn_validate(a, idx, budget, ratio, b, out, decode, pg);
    if (s != QSA_OK) return s;
    const size_t need = decode ? attn_workspace_bytes(*b, *a, budget, ratio) : 0;
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return fail(QSA_ERR_WORKSPACE, "attention workspace of %zu bytes is smaller than the %zu required "
                    "(qsa_attn_workspace_size)", ws == nullptr ? (size_t)0 : ws_bytes, need);
    return attn_launch(a, idx, budget, ratio, b, out, ws, decode, pg, st);
}


}  // namespace qsa

using namespace qsa;

extern "C" {

int32_t qsa_inert_bound(int32_t budget, int32_t ratio) {
    if (budget <= 0 || ratio <= 0) return -1;
    return budget + ratio - 1;
}

const char *qsa_last_error(void) { return g_err; }

const char *qsa_version(void) { return "qsa 0.5.0 (abi 3, gfx950)"; }

int32_t qsa_abi_version(void) { return QSA_ABI_VERSION; }

static qsa_status compress_common(const void *k_idx, int32_t k_dtype, int32_t d_idx, int32_t ratio,
                                  const qsa_batch *b, const int64_t *first_block, void *kc,
                                  int32_t kc_dtype, void *kc_scale, const qsa_paged_kv *pg,
                                  void *stream) {
    qsa_status s = check_batch(b, pg == nullptr);
    if (s == QSA_OK && pg) s = check_paging(pg, b, ratio);
    if (s != QSA_OK) return s;
    if (!k_idx) return fail(QSA_ERR_INVALID_ARGUMENT, "k_idx is NULL");
    if (!kc) return fail(QSA_ERR_INVALID_ARGUMENT, "kc is NULL");
    s = check_ratio(ratio);
    if (s != QSA_OK) return s;
    if (k_dtype != QSA_F32 && k_dtype != QSA_BF16)
        return fail(QSA_ERR_UNSUPPORTED, "k_dtype=%d must be QSA_F32 or QSA_BF16", k_dtype);
    if (kc_dtype != QSA_F32 && kc_dtype != QSA_BF16 && kc_dtype != QSA_FP8_E4M3 && kc_dtype != QSA_FP4_E2M1)
        return fail(QSA_ERR_UNSUPPORTED, "kc_dtype=%d is not a qsa_dtype", kc_dtype);
    if ((kc_dtype == QSA_FP8_E4M3 || kc_dtype == QSA_FP4_E2M1) && !kc_scale)
        return fail(QSA_ERR_INVALID_ARGUMENT, "kc_scale is NULL but kc_dtype=%d needs scales", kc_dtype);
    if (d_idx != 64 && d_idx != 128) return fail(QSA_ERR_UNSUPPORTED, "d_idx=%d must be 64 or 128", d_idx);
    if ((b->max_kv_len / ratio) > 0xffffffffLL * 16)
        return fail(QSA_ERR_UNSUPPORTED, "max_kv_len=%lld is too large", (long long)b->max_kv_len);
    return launch_checked("qsa_compress_keys", batch_check(*b, ratio, pg == nullptr, pg), stream, [&](hipStream_t st) {
        return launch_compress(k_idx, k_dtype, d_idx, ratio, *b, first_block, kc, kc_dtype, kc_scale, pg, st);
    });
}

qsa_status qsa_compress_keys(const void *k_idx, int32_t k_dtype, int32_t d_idx, int32_t ratio,
                             const qsa_batch *b, const int64_t *first_block, void *kc,
                             int32_t kc_dtype, void *kc_scale, void *stream) {
    return compress_common(k_idx, k_dtype, d_idx, ratio, b, first_block, kc, kc_dtype, kc_scale,
                           nullptr, stream);
}

qsa_status qsa_compress_keys_paged(const void *k_idx, int32_t k_dtype, int32_t d_idx, int32_t ratio,
                                   const qsa_batch *b, const int64_t *first_block, void *kc,
                                   int32_t kc_dtype, void *kc_scale, const qsa_paged_kv *pg,
                                   void *stream) {
    if (!pg) return fail(QSA_ERR_INVALID_ARGUMENT, "paging descriptor is NULL");
    return compress_common(k_idx, k_dtype, d_idx, ratio, b, first_block, kc, kc_dtype, kc_scale, pg,
                           stream);
}

static qsa_status score_common(const qsa_indexer *ix, int32_t ratio, const qsa_batch *b, float *scores,
                               int64_t ld_scores, uint32_t flags, const qsa_paged_kv *pg, void *stream) {
    if (flags != QSA_SCORE_CANONICAL && flags != QSA_SCORE_MFMA)
        return fail(QSA_ERR_INVALID_ARGUMENT, "flags=%u must be QSA_SCORE_CANONICAL or QSA_SCORE_MFMA", flags);
    const bool mfma = flags == QSA_SCORE_MFMA;
    if (mfma && pg)
        return fail(QSA_ERR_UNSUPPORTED, "QSA_SCORE_MFMA does not read paged caches; use QSA_SCORE_CANONICAL");
    qsa_status s = check_indexer(ix, mfma);
    if (s == QSA_OK) s = check_batch(b, pg == nullptr);
    if (s == QSA_OK && pg) s = check_paging(pg, b, ratio);
    if (s == QSA_OK) s = check_ratio(ratio);
    if (s == QSA_OK) s = check_rows(b, ratio);
    if (s != QSA_OK) return s;
    if (!scores) return fail(QSA_ERR_INVALID_ARGUMENT, "scores is NULL");
    const int64_t need_ld = (b->max_kv_len + ratio - 1) / ratio;
    if (ld_scores < need_ld || ld_scores < 1)
        return fail(QSA_ERR_INVALID_ARGUMENT, "ld_scores=%lld must be >= ceil(max_kv_len/ratio)=%lld",
                    (long long)ld_scores, (long long)need_ld);
    return launch_checked("qsa_index_score", batch_check(*b, ratio, pg == nullptr, pg), stream, [&](hipStream_t st) {
        return mfma ? launch_score_mfma(*ix, ratio, *b, scores, ld_scores, st)
                    : launch_score_canonical(*ix, ratio, *b, scores, ld_scores, pg, st, ListArgs{});
    });
}

qsa_status qsa_index_score(const qsa_indexer *ix, int32_t ratio, const qsa_batch *b, float *scores,
                           int64_t ld_scores, uint32_t flags, void *stream) {
    return score_common(ix, ratio, b, scores, ld_scores, flags, nullptr, stream);
}

qsa_status qsa_index_score_paged(const qsa_indexer *ix, int32_t ratio, const qsa_batch *b, float *scores,
                                 int64_t ld_scores, uint32_t flags, const qsa_paged_kv *pg, void *stream) {
    if (!pg) return fail(QSA_ERR_INVALID_ARGUMENT, "paging descriptor is NULL");
    return score_common(ix, ratio, b, scores, ld_scores, flags, pg, stream);
}

size_t qsa_score_topk_workspace_size(const qsa_batch *b, int32_t budget, int32_t ratio) {
    if (!b || check_budget(budget, ratio) != QSA_OK) return 0;
    return score_topk_workspace_bytes(*b, budget, ratio);
}

qsa_status qsa_index_score_topk(const qsa_indexer *ix, int32_t budget, int32_t ratio, const qsa_batch *b,
                                float *scores, int64_t ld_scores, int32_t *idx, void *ws, size_t ws_bytes,
                                const qsa_paged_kv *pg, void *stream) {
    qsa_status s = check_indexer(ix, false);
    if (s == QSA_OK) s = check_batch(b, pg == nullptr);
    if (s == QSA_OK && pg) s = check_paging(pg, b, ratio);
    if (s == QSA_OK) s = check_budget(budget, ratio);
    if (s == QSA_OK) s = check_rows(b, ratio);
    if (s != QSA_OK) return s;
    if (!scores) return fail(QSA_ERR_INVALID_ARGUMENT, "scores is NULL");
    if (!idx) return fail(QSA_ERR_INVALID_ARGUMENT, "idx is NULL");
    const int64_t need_ld = (b->max_kv_len + ratio - 1) / ratio;
    if (ld_scores < need_ld || ld_scores < 1)
        return fail(QSA_ERR_INVALID_ARGUMENT, "ld_scores=%lld must be >= ceil(max_kv_len/ratio)=%lld",
                    (long long)ld_scores, (long long)need_ld);
    const size_t need = score_topk_workspace_bytes(*b, budget, ratio);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return fail(QSA_ERR_WORKSPACE, "score + top-k workspace of %zu bytes is smaller than the %zu required "
                    "(qsa_score_topk_workspace_size)", ws == nullptr ? (size_t)0 : ws_bytes, need);
    return launch_checked("qsa_index_score_topk", batch_check(*b, ratio, pg == nullptr, pg), stream,
                          [&](hipStream_t st) {
                              return launch_score_topk(*ix, budget, ratio, *b, scores, ld_scores, idx, ws, pg, st);
                          });
}

// Workspace of qsa_decode_step: the candidate lists, then the attention
// partials (each 256-byte aligned).
static size_t decode_step_lists_bytes(const qsa_batch &b, int32_t budget, int32_t ratio) {
    return (score_topk_workspace_bytes(b, budget, ratio) + 255) & ~(size_t)255;
}

size_t qsa_decode_step_workspace_size(const qsa_batch *b, const qsa_attn *a, int32_t budget, int32_t ratio) {
    if (!b || !a || check_budget(budget, ratio) != QSA_OK || a->hkv < 1) return 0;
    return decode_step_lists_bytes(*b, budget, ratio) + attn_workspace_bytes(*b, *a, budget, ratio);
}

// Shared validation of the decode-step calls.
static qsa_status decode_step_check(const qsa_indexer *ix, const qsa_attn *a, int32_t budget, int32_t ratio,
                                    const qsa_batch *b, const float *scores, int64_t ld_scores, int32_t *idx,
                                    void *out, void *ws, size_t ws_bytes, const qsa_paged_kv *pg) {
    qsa_status s = ix ? check_indexer(ix, false) : ok();
    if (s == QSA_OK) s = attn_validate(a, idx, budget, ratio, b, out, true, pg);
    if (s == QSA_OK) s = check_batch(b, ix != nullptr && pg == nullptr);   // the scorer reads blk_offsets
    if (s == QSA_OK) s = check_rows(b, ratio);
    if (s != QSA_OK) return s;
    if (!scores) return fail(QSA_ERR_INVALID_ARGUMENT, "scores is NULL");
    const int64_t need_ld = (b->max_kv_len + ratio - 1) / ratio;
    if (ld_scores < need_ld || ld_scores < 1)
        return fail(QSA_ERR_INVALID_ARGUMENT, "ld_scores=%lld must be >= ceil(max_kv_len/ratio)=%lld",
                    (long long)ld_scores, (long long)need_ld);
    const size_t need = decode_step_lists_bytes(*b, budget, ratio) + attn_workspace_bytes(*b, *a, budget, ratio);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return fail(QSA_ERR_WORKSPACE, "decode step workspace of %zu bytes is smaller than the %zu required "
                    "(qsa_decode_step_workspace_size)", ws == nullptr ? (size_t)0 : ws_bytes, need);
    if (ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 15u) != 0)
        return fail(QSA_ERR_INVALID_ARGUMENT, "decode step workspace %p is not 16-byte aligned (the candidate "
                    "lists are read 16 bytes at a time)", ws);
    return ok();
}

// The scorer half: scores, and the candidate lists when the batch has them.
static hipError_t decode_step_score(const qsa_indexer &ix, int32_t budget, int32_t ratio, const qsa_batch &b,
                                    float *scores, int64_t ld, void *ws, const qsa_paged_kv *pg, hipStream_t st) {
    if (!score_topk_uses_lists(b)) return launch_score_canonical(ix, ratio, b, scores, ld, pg, st, ListArgs{});
    return launch_score_canonical(ix, ratio, b, scores, ld, pg, st, list_args(b, budget, ratio, ws));
}

// The attention half: the selection (in the attention kernel when it can
// make it, else the list finish or the plain top-k) and the attention.
static hipError_t decode_step_attend(const qsa_attn &a, int32_t budget, int32_t ratio, const qsa_batch &b,
                                     const float *scores, int64_t ld, int32_t *idx, void *out, void *ws,
                                     const qsa_paged_kv *pg, hipStream_t st) {
    void *attn_ws = ws ? static_cast<uint8_t *>(ws) + decode_step_lists_bytes(b, budget, ratio) : nullptr;
    if (!score_topk_uses_lists(b)) {
        hipError_t e = launch_topk(scores, ld, nullptr, budget, ratio, b, idx, budget / ratio, ws, st);
        if (e != hipSuccess) return e;
        return launch_attn(a, idx, budget, ratio, b, out, attn_ws, true, pg, st);
    }
    const ListArgs la = list_args(b, budget, ratio, ws);
    if (attn_select_supported(b, a, pg))
        return launch_attn_select(a, budget, ratio, b, la, scores, ld, idx, out, attn_ws, pg, st);
    hipError_t e = launch_topk_from_lists(scores, ld, budget, ratio, b, idx, la, st);
    if (e != hipSuccess) return e;
    return launch_attn(a, idx, budget, ratio, b, out, attn_ws, true, pg, st);
}

qsa_status qsa_decode_step(const qsa_indexer *ix, const qsa_attn *a, int32_t budget, int32_t ratio,
                           const qsa_batch *b, float *scores, int64_t ld_scores, int32_t *idx, void *out, void *ws,
                           size_t ws_bytes, const qsa_paged_kv *pg, void *stream) {
    if (!ix) return fail(QSA_ERR_INVALID_ARGUMENT, "indexer is NULL");
    qsa_status s = decode_step_check(ix, a, budget, ratio, b, scores, ld_scores, idx, out, ws, ws_bytes, pg);
    if (s != QSA_OK) return s;
    return launch_checked("qsa_decode_step", batch_check(*b, ratio, pg == nullptr, pg), stream, [&](hipStream_t st) {
        hipError_t e = decode_step_score(*ix, budget, ratio, *b, scores, ld_scores, ws, pg, st);
        if (e != hipSuccess) return e;
        return decode_step_attend(*a, budget, ratio, *b, scores, ld_scores, idx, out, ws, pg, st);
    });
}

qsa_status qsa_index_score_lists(const qsa_indexer *ix, const qsa_attn *a, int32_t budget, int32_t ratio,
                                 const qsa_batch *b, float *scores, int64_t ld_scores, void *ws, size_t ws_bytes,
                                 const qsa_paged_kv *pg, void *stream) {
    if (!ix) return fail(QSA_ERR_INVALID_ARGUMENT, "indexer is NULL");
    // idx and out are not touched by this half: validate with stand-ins
    int32_t dummy_idx = 0;
    qsa_status s = decode_step_check(ix, a, budget, ratio, b, scores, ld_scores, &dummy_idx, &dummy_idx, ws,
                                     ws_bytes, pg);
    if (s != QSA_OK) return s;
    return launch_checked("qsa_index_score_lists", batch_check(*b, ratio, pg == nullptr, pg), stream,
                          [&](hipStream_t st) {
                              return decode_step_score(*ix, budget, ratio, *b, scores, ld_scores, ws, pg, st);
                          });
}

qsa_status qsa_sparse_attn_decode_lists(const qsa_attn *a, int32_t budget, int32_t ratio, const qsa_batch *b,
                                        const float *scores, int64_t ld_scores, int32_t *idx, void *out, void *ws,
                                        size_t ws_bytes, const qsa_paged_kv *pg, void *stream) {
    qsa_status s = decode_step_check(nullptr, a, budget, ratio, b, scores, ld_scores, idx, out, ws, ws_bytes, pg);
    if (s != QSA_OK) return s;
    return launch_checked("qsa_sparse_attn_decode_lists", batch_check(*b, ratio, false, pg), stream,
                          [&](hipStream_t st) {
                              return decode_step_attend(*a, budget, ratio, *b, scores, ld_scores, idx, out, ws, pg,
                                                        st);
                          });
}

size_t qsa_topk_workspace_size(const qsa_batch *b, int32_t budget, int32_t ratio,
                               const qsa_indexer *recheck) {
    if (!b || check_budget(budget, ratio) != QSA_OK) return 0;
    return topk_workspace_bytes(*b, budget, ratio, recheck);
}

static qsa_status topk_common(const float *scores, int64_t ld_scores, const qsa_indexer *recheck,
                              int32_t budget, int32_t ratio, int32_t local_blocks, const qsa_batch *b,
                              int32_t *idx, void *ws, size_t ws_bytes, void *stream) {
    qsa_status s = check_batch(b, recheck != nullptr);
    if (s == QSA_OK) s = check_budget(budget, ratio);
    if (s == QSA_OK) s = check_rows(b, ratio);
    if (s == QSA_OK && recheck) s = check_indexer(recheck, false);
    if (s == QSA_OK && recheck && recheck->kc_dtype == QSA_FP4_E2M1)
        return fail(QSA_ERR_UNSUPPORTED, "recheck: fp4 compressed keys are scored canonically only");
    if (s != QSA_OK) return s;
    if (local_blocks < 0 || budget / ratio + local_blocks > 2048)
        return fail(QSA_ERR_UNSUPPORTED, "local_blocks=%d: budget/ratio + local_blocks must be in [K, 2048]",
                    local_blocks);
    if (recheck && b->max_kv_len / ratio > kTopkRecheckMaxBlocks)
        return fail(QSA_ERR_UNSUPPORTED,
                    "re-checked top-k supports at most %lld blocks per row (max_kv_len/ratio=%lld)",
                    (long long)kTopkRecheckMaxBlocks, (long long)(b->max_kv_len / ratio));
    if (!scores) return fail(QSA_ERR_INVALID_ARGUMENT, "scores is NULL");
    if (!idx) return fail(QSA_ERR_INVALID_ARGUMENT, "idx is NULL");
    const int64_t need_ld = (b->max_kv_len + ratio - 1) / ratio;
    if (ld_scores < need_ld || ld_scores < 1)
        return fail(QSA_ERR_INVALID_ARGUMENT, "ld_scores=%lld must be >= ceil(max_kv_len/ratio)=%lld",
                    (long long)ld_scores, (long long)need_ld);
    const size_t need = topk_workspace_bytes(*b, budget, ratio, recheck);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return fail(QSA_ERR_WORKSPACE, "top-k workspace of %zu bytes is smaller than the %zu required "
                    "(qsa_topk_workspace_size)", ws == nullptr ? (size_t)0 : ws_bytes, need);
    const int ldi = budget / ratio + local_blocks;
    return launch_checked("qsa_topk_blocks", batch_check(*b, ratio, recheck != nullptr, nullptr), stream,
                          [&](hipStream_t st) {
                              hipError_t e = launch_topk(scores, ld_scores, recheck, budget, ratio, *b, idx, ldi, ws, st);
                              if (e == hipSuccess && local_blocks > 0)
                                  e = launch_topk_local(budget, ratio, local_blocks, *b, idx, ldi, st);
                              return e;
                          });
}

qsa_status qsa_topk_blocks(const float *scores, int64_t ld_scores, const qsa_indexer *recheck,
                           int32_t budget, int32_t ratio, const qsa_batch *b, int32_t *idx,
                           void *ws, size_t ws_bytes, void *stream) {
    return topk_common(scores, ld_scores, recheck, budget, ratio, 0, b, idx, ws, ws_bytes, stream);
}

qsa_status qsa_topk_blocks_local(const float *scores, int64_t ld_scores, const qsa_indexer *recheck,
                                 int32_t budget, int32_t ratio, int32_t local_blocks, const qsa_batch *b,
                                 int32_t *idx, void *ws, size_t ws_bytes, void *stream) {
    return topk_common(scores, ld_scores, recheck, budget, ratio, local_blocks, b, idx, ws, ws_bytes,
                       stream);
}

size_t qsa_attn_workspace_size(const qsa_batch *b, const qsa_attn *a, int32_t budget, int32_t ratio) {
    if (!b || !a || check_budget(budget, ratio) != QSA_OK || a->hkv < 1) return 0;
    return attn_workspace_bytes(*b, *a, budget, ratio);
}

qsa_status qsa_sparse_attn_decode(const qsa_attn *a, const int32_t *idx, int32_t budget, int32_t ratio,
                                  const qsa_batch *b, void *out, void *ws, size_t ws_bytes, void *stream) {
    return attn_common(a, idx, budget, ratio, b, out, ws, ws_bytes, true, nullptr, (hipStream_t)stream);
}

qsa_status qsa_sparse_attn_decode_static(const qsa_attn *a, const int32_t *idx, int32_t budget, int32_t ratio,
                                         const qsa_batch *b, void *out, void *stream) {
    qsa_status s = attn_validate(a, idx, budget, ratio, b, out, true, nullptr);
    if (s != QSA_OK) return s;
    const size_t need = attn_workspace_bytes(*b, *a, budget, ratio);
    if (need > kAttnStaticScratchBytes)
        return fail(QSA_ERR_WORKSPACE,
                    "qsa_sparse_attn_decode_static: this batch needs %zu bytes of scratch (total_q x hq x parts "
                    "x 130 floats), more than the %zu bytes of the static array; use qsa_sparse_attn_decode "
                    "with a workspace", need, kAttnStaticScratchBytes);
    if (forced_launch_error())
        return fail(QSA_ERR_HIP, "qsa_sparse_attn_decode_static: launch failed (forced by "
                    "QSA_TEST_FORCE_LAUNCH_ERROR)");
    void *ws = nullptr;
    if (need > 0) {
        const hipError_t e = attn_static_scratch(&ws);
        if (e != hipSuccess) return hip_status(e, "qsa_sparse_attn_decode_static: scratch address");
    }
    return attn_launch(a, idx, budget, ratio, b, out, ws, true, nullptr, stream);
}

qsa_status qsa_sparse_attn_prefill(const qsa_attn *a, const int32_t *idx, int32_t budget, int32_t ratio,
                                   const qsa_batch *b, void *out, void *ws, size_t ws_bytes, void *stream) {
    return attn_common(a, idx, budget, ratio, b, out, ws, ws_bytes, false, nullptr, (hipStream_t)stream);
}

qsa_status qsa_sparse_attn_decode_paged(const qsa_attn *a, const int32_t *idx, int32_t budget,
                                        int32_t ratio, const qsa_batch *b, void *out, void *ws,
                                        size_t ws_bytes, const qsa_paged_kv *pg, void *stream) {
    if (!pg) return fail(QSA_ERR_INVALID_ARGUMENT, "paging descriptor is NULL");
    return attn_common(a, idx, budget, ratio, b, out, ws, ws_bytes, true, pg, (hipStream_t)stream);
}

size_t qsa_attn_layers_workspace_size(const qsa_batch *b, const qsa_attn *a, int32_t n_layers, int32_t budget,
                                      int32_t ratio) {
    if (!b || !a || check_budget(budget, ratio) != QSA_OK || a->hkv < 1 || n_layers < 1 ||
        n_layers > QSA_MAX_LAYERS)
        return 0;
    return (size_t)n_layers * attn_layer_stride_bytes(*b, *a, budget, ratio);
}

qsa_status qsa_sparse_attn_decode_layers(const qsa_attn *layers, int32_t n_layers, const int32_t *idx,
                                         int32_t budget, int32_t ratio, const qsa_batch *b, void *const *outs,
                                         void *ws, size_t ws_bytes, const qsa_paged_kv *pg, void *stream) {
    if (!layers) return fail(QSA_ERR_INVALID_ARGUMENT, "layers is NULL");
    if (n_layers < 1 || n_layers > QSA_MAX_LAYERS)
        return fail(QSA_ERR_INVALID_ARGUMENT, "n_layers=%d must be in [1, %d]", n_layers, QSA_MAX_LAYERS);
    if (!outs) return fail(QSA_ERR_INVALID_ARGUMENT, "outs is NULL");
    for (int l = 0; l < n_layers; ++l) {
        qsa_status s = check_attn(&layers[l]);
        if (s != QSA_OK) return s;
        if (!outs[l]) return fail(QSA_ERR_INVALID_ARGUMENT, "outs[%d] is NULL", l);
        if (layers[l].dtype != layers[0].dtype || layers[l].hq != layers[0].hq ||
            layers[l].hkv != layers[0].hkv || layers[l].d != layers[0].d)
            return fail(QSA_ERR_INVALID_ARGUMENT, "layers[%d] differs from layers[0] in dtype, hq, hkv or d", l);
    }
    qsa_status s = check_batch(b, false);
    if (s == QSA_OK && pg) s = check_paging(pg, b, ratio);
    if (s == QSA_OK) s = check_budget(budget, ratio);
    if (s != QSA_OK) return s;
    if (!idx) return fail(QSA_ERR_INVALID_ARGUMENT, "idx is NULL");
    if (b->q_offsets != nullptr && b->max_q_per_seq != 1)
        return fail(QSA_ERR_INVALID_ARGUMENT,
                    "decode takes one query per sequence (q_offsets NULL or max_q_per_seq == 1)");
    const size_t need = (size_t)n_layers * attn_layer_stride_bytes(*b, layers[0], budget, ratio);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return fail(QSA_ERR_WORKSPACE, "attention workspace of %zu bytes is smaller than the %zu required "
                    "(qsa_attn_layers_workspace_size)", ws == nullptr ? (size_t)0 : ws_bytes, need);
    DebugCheck dc = batch_check(*b, ratio, false, pg);
    dc.idx = idx;
    dc.ldi = budget / ratio;
    return launch_checked("qsa_sparse_attn_decode_layers", dc, stream, [&](hipStream_t st) {
        return launch_attn_layers(layers, n_layers, idx, budget, ratio, *b, outs, ws, pg, st);
    });
}

qsa_status qsa_sparse_attn_prefill_paged(const qsa_attn *a, const int32_t *idx, int32_t budget,
                                         int32_t ratio, const qsa_batch *b, void *out, void *ws,
                                         size_t ws_bytes, const qsa_paged_kv *pg, void *stream) {
    if (!pg) return fail(QSA_ERR_INVALID_ARGUMENT, "paging descriptor is NULL");
    return attn_common(a, idx, budget, ratio, b, out, ws, ws_bytes, false, pg, (hipStream_t)stream);
}

static qsa_status check_ring(const qsa_key_ring *ring, const qsa_batch *b, int32_t ratio) {
    if (!ring) return fail(QSA_ERR_INVALID_ARGUMENT, "ring is NULL");
    if (!ring->keys) return fail(QSA_ERR_INVALID_ARGUMENT, "ring.keys is NULL");
    if (!ring->window) return fail(QSA_ERR_INVALID_ARGUMENT, "ring.window is NULL");
    if (ring->capacity < ratio || ring->capacity % ratio != 0)
        return fail(QSA_ERR_INVALID_ARGUMENT, "ring.capacity=%d must be a positive multiple of ratio=%d",
                    ring->capacity, ratio);
    if (ring->num_slots < 1 || (!ring->slots && ring->num_slots < b->num_seqs))
        return fail(QSA_ERR_INVALID_ARGUMENT,
                    "ring.num_slots=%lld must be >= 1 (>= num_seqs=%d when ring.slots is NULL)",
                    (long long)ring->num_slots, b->num_seqs);
    if (ring->num_slots > 0x7fffffffLL)
        return fail(QSA_ERR_UNSUPPORTED, "ring.num_slots=%lld exceeds 2^31-1", (long long)ring->num_slots);
    return ok();
}

static qsa_status check_kv_append(const qsa_kv_append *kv) {
    if (!kv) return ok();
    if (!kv->k_new || !kv->v_new || !kv->k || !kv->v)
        return fail(QSA_ERR_INVALID_ARGUMENT, "kv.k_new/v_new/k/v must not be NULL");
    if (kv->dtype != QSA_F32 && kv->dtype != QSA_BF16)
        return fail(QSA_ERR_UNSUPPORTED, "kv.dtype=%d must be QSA_F32 or QSA_BF16", kv->dtype);
    if (kv->hkv < 1 || kv->hkv > 64)
        return fail(QSA_ERR_UNSUPPORTED, "kv.hkv=%d must be in [1, 64]", kv->hkv);
    if (kv->d != 128) return fail(QSA_ERR_UNSUPPORTED, "kv.d=%d must be 128", kv->d);
    return ok();
}

qsa_status qsa_ingest(const void *k_new, int32_t k_dtype, int32_t d_idx, int32_t ratio,
                      const qsa_batch *b, const qsa_key_ring *ring, void *kc, int32_t kc_dtype,
                      void *kc_scale, const qsa_kv_append *kv, int32_t *status,
                      const qsa_paged_kv *pg, void *stream) {
    qsa_status s = check_batch(b, pg == nullptr);
    if (s == QSA_OK) s = check_ratio(ratio);
    if (s == QSA_OK && pg) s = check_paging(pg, b, ratio);
    if (s == QSA_OK) s = check_ring(ring, b, ratio);
    if (s != QSA_OK) return s;
    if (!k_new) return fail(QSA_ERR_INVALID_ARGUMENT, "k_new is NULL");
    if (!kc) return fail(QSA_ERR_INVALID_ARGUMENT, "kc is NULL");
    if (k_dtype != QSA_F32 && k_dtype != QSA_BF16)
        return fail(QSA_ERR_UNSUPPORTED, "k_dtype=%d must be QSA_F32 or QSA_BF16", k_dtype);
    if (kc_dtype != QSA_F32 && kc_dtype != QSA_BF16 && kc_dtype != QSA_FP8_E4M3 && kc_dtype != QSA_FP4_E2M1)
        return fail(QSA_ERR_UNSUPPORTED, "kc_dtype=%d is not a qsa_dtype", kc_dtype);
    if ((kc_dtype == QSA_FP8_E4M3 || kc_dtype == QSA_FP4_E2M1) && !kc_scale)
        return fail(QSA_ERR_INVALID_ARGUMENT, "kc_scale is NULL but kc_dtype=%d needs scales", kc_dtype);
    if (d_idx != 64 && d_idx != 128) return fail(QSA_ERR_UNSUPPORTED, "d_idx=%d must be 64 or 128", d_idx);
    if (b->q_offsets && b->max_q_per_seq < 0)
        return fail(QSA_ERR_INVALID_ARGUMENT, "batch.max_q_per_seq=%d must be >= 0", b->max_q_per_seq);
    s = check_kv_append(kv);
    if (s != QSA_OK) return s;
    DebugCheck dc = batch_check(*b, ratio, pg == nullptr, pg);
    dc.strict_q = false;
    return launch_checked("qsa_ingest", dc, stream, [&](hipStream_t st) {
        return launch_ingest(k_new, k_dtype, d_idx, ratio, *b, *ring, kc, kc_dtype, kc_scale, kv, status, pg, st);
    });
}

// Shared validation of the append + score calls.
static qsa_status ingest_score_check(const void *k_new, int32_t k_dtype, int32_t ratio, const qsa_batch *b,
                                     const qsa_key_ring *ring, const qsa_kv_append *kv, const qsa_indexer *ix,
                                     const float *scores, int64_t ld_scores, const qsa_paged_kv *pg,
                                     const char *what) {
    qsa_status s = check_indexer(ix, false);
    if (s == QSA_OK) s = check_batch(b, pg == nullptr);
    if (s == QSA_OK) s = check_ratio(ratio);
    if (s == QSA_OK && pg) s = check_paging(pg, b, ratio);
    if (s == QSA_OK) s = check_rows(b, ratio);
    if (s == QSA_OK) s = check_ring(ring, b, ratio);
    if (s == QSA_OK) s = check_kv_append(kv);
    if (s != QSA_OK) return s;
    if (b->q_offsets)
        return fail(QSA_ERR_INVALID_ARGUMENT,
                    "%s takes one new token and one query per sequence "
                    "(batch.q_offsets must be NULL); use qsa_ingest and qsa_index_score", what);
    if (ix->q_dtype != QSA_BF16 || ix->kc_dtype == QSA_F32)
        return fail(QSA_ERR_UNSUPPORTED,
                    "%s needs a bf16 q_idx and bf16, e4m3 or fp4 compressed keys "
                    "(q_dtype=%d, kc_dtype=%d)", what, ix->q_dtype, ix->kc_dtype);
    if (!k_new) return fail(QSA_ERR_INVALID_ARGUMENT, "k_new is NULL");
    if (k_dtype != QSA_F32 && k_dtype != QSA_BF16)
        return fail(QSA_ERR_UNSUPPORTED, "k_dtype=%d must be QSA_F32 or QSA_BF16", k_dtype);
    if (!scores) return fail(QSA_ERR_INVALID_ARGUMENT, "scores is NULL");
    const int64_t need_ld = (b->max_kv_len + ratio - 1) / ratio;
    if (ld_scores < need_ld || ld_scores < 1)
        return fail(QSA_ERR_INVALID_ARGUMENT, "ld_scores=%lld must be >= ceil(max_kv_len/ratio)=%lld",
                    (long long)ld_scores, (long long)need_ld);
    return ok();
}

qsa_status qsa_ingest_index_score(const void *k_new, int32_t k_dtype, int32_t ratio, const qsa_batch *b,
                                  const qsa_key_ring *ring, const qsa_kv_append *kv, int32_t *status,
                                  const qsa_indexer *ix, float *scores, int64_t ld_scores,
                                  const qsa_paged_kv *pg, void *stream) {
    qsa_status s = ingest_score_check(k_new, k_dtype, ratio, b, ring, kv, ix, scores, ld_scores, pg,
                                      "qsa_ingest_index_score");
    if (s != QSA_OK) return s;
    return launch_checked("qsa_ingest_index_score", batch_check(*b, ratio, pg == nullptr, pg), stream,
                          [&](hipStream_t st) {
                              return launch_ingest_score(k_new, k_dtype, ratio, *b, *ring, kv, status, *ix, scores,
                                                         ld_scores, pg, st, ListArgs{});
                          });
}

qsa_status qsa_ingest_index_score_lists(const void *k_new, int32_t k_dtype, const qsa_key_ring *ring,
                                        const qsa_kv_append *kv, int32_t *status, const qsa_indexer *ix,
                                        const qsa_attn *a, int32_t budget, int32_t ratio, const qsa_batch *b,
                                        float *scores, int64_t ld_scores, void *ws, size_t ws_bytes,
                                        const qsa_paged_kv *pg, void *stream) {
    qsa_status s = ingest_score_check(k_new, k_dtype, ratio, b, ring, kv, ix, scores, ld_scores, pg,
                                      "qsa_ingest_index_score_lists");
    if (s != QSA_OK) return s;
    // idx and out are not touched by this half: validate with stand-ins
    int32_t dummy = 0;
    s = decode_step_check(ix, a, budget, ratio, b, scores, ld_scores, &dummy, &dummy, ws, ws_bytes, pg);
    if (s != QSA_OK) return s;
    return launch_checked("qsa_ingest_index_score_lists", batch_check(*b, ratio, pg == nullptr, pg), stream,
                          [&](hipStream_t st) {
                              const ListArgs la = score_topk_uses_lists(*b) ? list_args(*b, budget, ratio, ws)
                                                                            : ListArgs{};
                              return launch_ingest_score(k_new, k_dtype, ratio, *b, *ring, kv, status, *ix, scores,
                                                         ld_scores, pg, st, la);
                          });
}

qsa_status qsa_ring_rewind(const qsa_batch *b, int32_t ratio, const qsa_key_ring *ring, int32_t *status,
                           void *stream) {
    qsa_status s = check_batch(b, false);
    if (s == QSA_OK) s = check_ratio(ratio);
    if (s == QSA_OK) s = check_ring(ring, b, ratio);
    if (s != QSA_OK) return s;
    return launch_checked("qsa_ring_rewind", batch_check(*b, ratio, false, nullptr), stream,
                          [&](hipStream_t st) { return launch_ring_rewind(*b, ratio, *ring, status, st); });
}

qsa_status qsa_pool_scores(const float *tok, int64_t ld_tok, int32_t ratio, int32_t mode,
                           const qsa_batch *b, float *blk, int64_t ld_blk, void *stream) {
    qsa_status s = check_batch(b, false);
    if (s == QSA_OK) s = check_ratio(ratio);
    if (s == QSA_OK) s = check_rows(b, ratio);
    if (s != QSA_OK) return s;
    if (!tok || !blk) return fail(QSA_ERR_INVALID_ARGUMENT, "tok/blk must not be NULL");
    if (mode != QSA_POOL_MAX && mode != QSA_POOL_MEAN)
        return fail(QSA_ERR_INVALID_ARGUMENT, "mode=%d must be QSA_POOL_MAX or QSA_POOL_MEAN", mode);
    if (ld_tok < b->max_kv_len || ld_tok < 1)
        return fail(QSA_ERR_INVALID_ARGUMENT, "ld_tok=%lld must be >= max_kv_len=%lld", (long long)ld_tok,
                    (long long)b->max_kv_len);
    const int64_t need = (b->max_kv_len + ratio - 1) / ratio;
    if (ld_blk < need || ld_blk < 1)
        return fail(QSA_ERR_INVALID_ARGUMENT, "ld_blk=%lld must be >= ceil(max_kv_len/ratio)=%lld",
                    (long long)ld_blk, (long long)need);
    return launch_checked("qsa_pool_scores", batch_check(*b, ratio, false, nullptr), stream, [&](hipStream_t st) {
        return launch_pool_scores(tok, ld_tok, ratio, mode, *b, blk, ld_blk, st);
    });
}

}  // extern "C"
