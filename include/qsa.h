/*
 * qsa.h — C ABI of libqsa: indexer-selected ("QSA-style") sparse attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (per query): an indexer scores keys mean-pooled into blocks of
 * `ratio` tokens; a top-k keeps budget/ratio blocks; attention runs over the
 * tokens of those blocks plus the incomplete tail block.  While the visible
 * prefix L satisfies L <= budget + ratio - 1 (the inert bound) every complete
 * block is kept, which is exactly dense causal attention.
 *   Sources: "Agentic shootout — Atlas x Flash-Next research" page:
 *   gap analysis #1, plan item P1 (indexer, block top-k, gather attention);
 *   report "Flash-Next support: vLLM vs Atlas", section (a)6 (compressed keys
 *   per complete group, block top-k, group->token expansion of width
 *   budget + ratio - 1, -1 padded); "PR 16 review", section (a) (4Q+1K
 *   indexer, 4-token mean-pooled blocks, relu score, top-512 + tail, inert
 *   <= 2051 visible tokens); "llama.cpp vs Atlas", section (a)3 (the
 *   incomplete tail block is always visible).  "Atlas Flash-Next defect
 *   investigations" page, Defect 2 (inert_bound = budget + ratio - 1).
 *
 * Conventions shared by every call:
 *  - Memory: every tensor pointer is a DEVICE pointer owned by the caller.
 *    The library never allocates, frees or keeps a pointer after returning.
 *    Struct arguments are HOST structs read during the call only.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *    stream).  Work is enqueued asynchronously; inputs must stay valid and
 *    unmodified until the stream has passed it.  No call synchronises, copies
 *    device->host or allocates, so a sequence of calls can be captured in a
 *    HIP graph.
 *  - Errors: arguments are validated on the host BEFORE anything is
 *    enqueued; on any error nothing is enqueued and outputs are untouched.
 *    qsa_last_error() returns a thread-local message naming the argument and
 *    the limit.  A failed kernel launch returns QSA_ERR_HIP with the HIP
 *    error text.  Device-side contents (offset arrays) are not read by the
 *    host; they must satisfy the layout rules below (out-of-contract
 *    contents are undefined behaviour, and are caught in debug mode, below).
 *    NaN/Inf inputs are out of contract.
 *  - The library never substitutes dense attention for sparse attention past
 *    the inert bound: the regime is decided per query from its own L.
 *  - Debug mode (environment variable QSA_DEBUG=1, read on every call):
 *    before its own kernels each call runs a check of the device arrays it
 *    reads — kv_offsets[0] == 0 and 0 <= N_s <= max_kv_len; blk_offsets (when
 *    read) the prefix sums of floor(N_s/ratio); q_offsets[0] == 0,
 *    q_offsets[B] == total_q and 0 <= n_s <= min(N_s, max_q_per_seq); every
 *    idx entry read by attention in [-1, floor(L/ratio)); every block-table
 *    entry of a used page in [0, num_pages) — waits for it, and on a
 *    violation returns QSA_ERR_DEVICE_ASSERT (qsa_last_error() names the
 *    rule, the sequence or query and the value) without launching anything
 *    else.  Calls then also wait for their own kernels, so a debug-mode call
 *    synchronises its stream and cannot be captured in a graph.  ("Atlas
 *    Flash-Next defect investigations" page, Defect 4, proposed fix, items
 *    1-2, and fix plan PR-G: debug asserts on offsets and typed row offsets.)
 *  - Test hook: with QSA_TEST_FORCE_LAUNCH_ERROR=1 every call that passes
 *    host validation returns QSA_ERR_HIP without touching a device.
 *
 * Layouts (row-major, varlen-packed, int64 offsets [B+1] with offsets[0]=0):
 *  k_idx [sum N_s, d_idx]; K, V [sum N_s, hkv, d];
 *  kc [sum floor(N_s/ratio), d_idx] (+ kc_scale [same rows] f32 for e4m3;
 *  fp4: d_idx/2 bytes per row + kc_scale [same rows, d_idx/32] E8M0 bytes);
 *  q [total_q, hq, d]; q_idx [total_q, h_idx, d_idx]; w [total_q, h_idx] f32;
 *  scores [total_q, ld_scores] f32; idx [total_q, budget/ratio] int32;
 *  out [total_q, hq, d] (dtype of q).
 *  Sequence s holds N_s tokens (the queries' own keys already appended); its
 *  n_s queries are its LAST n_s tokens, so query j (0-based) of s sees
 *  L = N_s - n_s + j + 1 tokens.  Query head h uses KV head h / (hq/hkv).
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 3

typedef enum qsa_status {
    QSA_OK = 0,
    QSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, inconsistent sizes */
    QSA_ERR_UNSUPPORTED = 2,      /* valid but outside what the kernels implement */
    QSA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
    QSA_ERR_HIP = 4,              /* a HIP call or kernel launch failed */
    QSA_ERR_DEVICE_ASSERT = 5     /* debug mode only: the contents of a device argument broke
                                     the layout rules (see "Debug mode" above); nothing of the
                                     call was launched */
} qsa_status;

typedef enum qsa_dtype {
    QSA_F32 = 0,
    QSA_BF16 = 1,
    QSA_FP8_E4M3 = 2, /* OCP E4M3FN: bias 7, max finite 448, no infinities */
    QSA_FP4_E2M1 = 3  /* compressed keys only: OCP E2M1 codes, two per byte (dim 2j in
                         the low nibble of byte j), with one E8M0 scale byte 2^(e-127)
                         per 32 dims in a second plane (kc_scale) */
} qsa_dtype;

/* A varlen batch.  Offsets are DEVICE int64 arrays of num_seqs+1 entries. */
typedef struct qsa_batch {
    int32_t num_seqs;            /* B >= 1 */
    int32_t max_q_per_seq;       /* host upper bound on n_s (1 for decode) */
    int64_t total_q;             /* host copy of q_offsets[B] (B when q_offsets is NULL) */
    int64_t max_kv_len;          /* host upper bound on N_s (grid sizing only) */
    const int64_t *kv_offsets;   /* rows of sequence s in K, V, k_idx */
    const int64_t *blk_offsets;  /* rows of sequence s in kc: prefix sums of floor(N_s/ratio) */
    const int64_t *q_offsets;    /* rows of sequence s in q, q_idx, w, scores, idx, out;
                                    NULL => exactly one query per sequence (decode) */
} qsa_batch;

/* Indexer operands.  One key head (MQA), h_idx query heads. */
typedef struct qsa_indexer {
    const void *q_idx;           /* [total_q, h_idx, d_idx], dtype q_dtype */
    const float *w;              /* [total_q, h_idx] per-query head weights */
    const void *kc;              /* [sum nb, d_idx] compressed keys, dtype kc_dtype
                                    ([sum nb, d_idx/2] bytes for QSA_FP4_E2M1) */
    const void *kc_scale;        /* e4m3: f32 [sum nb]; fp4: E8M0 bytes [sum nb, d_idx/32];
                                    NULL for the other dtypes */
    int32_t q_dtype;             /* QSA_F32 | QSA_BF16 (QSA_BF16 with QSA_FP4_E2M1 keys) */
    int32_t kc_dtype;            /* QSA_F32 | QSA_BF16 | QSA_FP8_E4M3 | QSA_FP4_E2M1 */
    int32_t h_idx;               /* 1, 2, 4, 8 or 16 */
    int32_t d_idx;               /* 64 | 128 */
} qsa_indexer;

/* Attention operands; the output has the dtype of q. */
typedef struct qsa_attn {
    const void *q;               /* [total_q, hq, d] */
    const void *k;               /* [sum N_s, hkv, d] */
    const void *v;               /* [sum N_s, hkv, d] */
    int32_t dtype;               /* QSA_F32 | QSA_BF16 (q, k, v and out) */
    int32_t hq, hkv, d;          /* hq % hkv == 0, hq/hkv in {1,2,4,8,16}, d == 128 */
    float softmax_scale;         /* e.g. 1/sqrt(d) rounded to fp32 */
} qsa_attn;

/* budget + ratio - 1: the largest visible prefix L that is still served by
 * dense attention ("PR 16 review" (a): inert <= 2051 visible tokens for
 * budget 2048, ratio 4; defect investigations page, Defect 2).  Returns -1
 * for ratio <= 0 or budget <= 0. */
int32_t qsa_inert_bound(int32_t budget, int32_t ratio);

/* Thread-local text of the last error ("" if none). Never NULL. */
const char *qsa_last_error(void);
/* Library version string, e.g. "qsa 0.5.0 (abi 3, gfx950)". */
const char *qsa_version(void);
/* QSA_ABI_VERSION the library was built with. */
int32_t qsa_abi_version(void);

/* Key compression: kc[b] = mean of k_idx rows b*ratio .. b*ratio+ratio-1 for
 * every COMPLETE block b < floor(N_s/ratio) of every sequence (vLLM report
 * (a)6: one compressed key per complete group, mean-pooled; "PR 16 review"
 * (a): 4-token mean-pooled blocks).
 * Arithmetic: fp32 sum in row order, times 1/ratio (exact: ratio is a power
 * of two), then stored as fp32, bf16 (round to nearest even) or e4m3: with
 * amax = max_d |mean_d|, scale = amax/448 (fp32, correctly rounded) is written
 * to kc_scale[b] and code_d = e4m3_rne(clamp(mean_d/scale, +-448)); scale 0
 * gives all-zero codes.  (The e4m3 index plane with a per-block fp32 scale of
 * max|x|/448 is the long-context decode workload's definition.)  fp4 (the
 * E2M1 + E8M0 index plane of the "ATOM Model Support Guide" page,
 * DeepSeek-V4.1: values and scales in two planes): per group of 32 dims,
 * X = floor(log2(amax)) - 2 clamped to [-127, 127] (X = -127 when amax = 0;
 * 2 is E2M1's largest exponent, as in the OCP MX rule), kc_scale byte
 * X + 127, and code_d = the nearest E2M1 value of mean_d * 2^-X (ties to the
 * even mantissa, magnitudes past 6 give 6; the sign bit is kept).
 *  k_idx:  device [sum N_s, d_idx], k_dtype QSA_F32 | QSA_BF16.
 *  ratio:  power of two in [1, 64]; d_idx in {64, 128}.
 *  first_block: device int64 [B] or NULL; blocks b < first_block[s] are not
 *          rewritten (incremental ingest after appending tokens).
 *  kc:     device [sum nb, d_idx] of kc_dtype (any of the four; fp4 rows are
 *          d_idx/2 bytes).
 *  kc_scale: device f32 [sum nb] for QSA_FP8_E4M3, E8M0 bytes [sum nb, d_idx/32]
 *          for QSA_FP4_E2M1 (required for both), else ignored.
 * Errors: INVALID_ARGUMENT (null pointers, num_seqs < 1), UNSUPPORTED (ratio,
 * d_idx, dtype), HIP. */
qsa_status qsa_compress_keys(const void *k_idx, int32_t k_dtype, int32_t d_idx, int32_t ratio,
                             const qsa_batch *b, const int64_t *first_block, void *kc,
                             int32_t kc_dtype, void *kc_scale, void *stream);

/* Indexer scores.  For every query i and visible block b < floor(L_i/ratio)
 * of its sequence:  s_b = sum_h w_h * ReLU(q_idx[i,h,:] . kc_b)  ("PR 16
 * review" (a): relu score of a 4Q+1K indexer; one key head, vLLM report
 * (a)1 validator).  For e4m3 keys the dot is taken over the code values and
 * then multiplied by kc_scale[b].  For fp4 keys each key value is its code
 * value times its group's 2^(e-127), which is exact in fp32, and the dot runs
 * over those values (needs a bf16 q_idx).
 *  QSA_SCORE_CANONICAL: the fp32 result of one fixed evaluation order —
 *    dot = +0; for d ascending: dot = fl(dot + fl(q*k)); [dot = fl(dot*scale)];
 *    r = dot > 0 ? dot : +0; s = +0; for h ascending: s = fl(s + fl(w_h*r)).
 *    Bit-identical on every call and on any host that follows the same order.
 *  QSA_SCORE_MFMA: matrix-core scores for prefill (q_idx and kc bf16 only);
 *    within a certified bound of the canonical value but not bit-identical.
 *    They must be passed to qsa_topk_blocks together with `recheck`.
 *  scores: device [total_q, ld_scores]; entries b >= floor(L_i/ratio) of a row
 *    are left untouched.  ld_scores >= ceil(max_kv_len/ratio).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (dtype pair, h_idx, d_idx, ratio,
 * MFMA with non-bf16 operands), HIP. */
#define QSA_SCORE_CANONICAL 0u
#define QSA_SCORE_MFMA 1u
qsa_status qsa_index_score(const qsa_indexer *ix, int32_t ratio, const qsa_batch *b,
                           float *scores, int64_t ld_scores, uint32_t flags, void *stream);

/* Workspace bytes qsa_topk_blocks needs.  With recheck == NULL (canonical
 * scores) it is non-zero for batches of at most 256 query rows, which are
 * selected by a multi-workgroup method that keeps per-row, per-chunk lists in
 * the workspace (0 for larger batches).  With recheck it holds per-sequence
 * key-norm maxima.  The workspace needs no initialisation and carries no
 * state between calls. */
size_t qsa_topk_workspace_size(const qsa_batch *b, int32_t budget, int32_t ratio,
                               const qsa_indexer *recheck);

/* Block top-k per query (vLLM report (a)6: block top-k of budget/ratio groups;
 * "PR 16 review" (a): top-512 + tail).  With K = budget/ratio and
 * nb = floor(L_i/ratio):
 *   nb <= K (L_i <= inert bound, the dense regime): idx = 0,1,...,nb-1, -1...
 *   otherwise: the K blocks with the largest score, ties to the LOWER block
 *   index, written in ASCENDING block order.
 * scores: as written by qsa_index_score.  recheck: NULL when the scores are
 * canonical; when they are QSA_SCORE_MFMA scores, the same indexer operands,
 * which the kernel uses to bound every score's error and recompute the
 * undecided blocks canonically, so idx equals the canonical selection bit for
 * bit.  idx: device int32 [total_q, K].  ws: device workspace of at least
 * qsa_topk_workspace_size() bytes (may be NULL when that is 0).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (ratio not a power of two in [1,64],
 * budget % ratio != 0, K outside [1, 2048]), WORKSPACE, HIP. */
qsa_status qsa_topk_blocks(const float *scores, int64_t ld_scores, const qsa_indexer *recheck,
                           int32_t budget, int32_t ratio, const qsa_batch *b, int32_t *idx,
                           void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes qsa_sparse_attn_decode needs for this batch and shape
 * (qsa_sparse_attn_prefill needs none and ignores ws). */
size_t qsa_attn_workspace_size(const qsa_batch *b, const qsa_attn *a, int32_t budget,
                               int32_t ratio);

/* Sparse attention over T(L) = tokens of the selected blocks (idx >= 0) plus
 * the tail ratio*floor(L/ratio) .. L-1 (vLLM report (a)6: gather attention
 * over the expanded selection; "llama.cpp vs Atlas" (a)3: the tail block is
 * always visible).  For each query head h with KV head g = h/(hq/hkv):
 *   out_h = sum_{t in T} softmax_t(softmax_scale * q_h . K[t,g]) V[t,g]
 * with fp32 softmax and accumulation.  Because idx lists every complete block
 * in the dense regime, a query at or below the inert bound gets exactly dense
 * causal attention.  Queries with an empty T get zeros.
 *  idx: device int32 [total_q, budget/ratio] as written by qsa_topk_blocks.
 *  out: device [total_q, hq, d], dtype of q.
 *  ws:  decode: device workspace of at least qsa_attn_workspace_size()
 *       bytes; prefill: unused (may be NULL).
 * Prefill does not split a query's reduction, so its outputs do not depend
 * on the rest of the batch (chunked prefill equals single-shot prefill bit
 * for bit).  Decode splits each query's selected blocks into a number of
 * parts chosen from the batch size (to fill the GPU), so a decode output is
 * deterministic for a given batch size but may differ in the last bits
 * between batch sizes; the selection itself never does.
 * Decode requires one query per sequence (q_offsets NULL or
 * max_q_per_seq == 1), so L = N_s.  Prefill takes any n_s (chunked prefill or
 * speculative verify): each query uses its own causal L and its own regime
 * (defect investigations page, fix plan PR-G: two-chunk prefill must equal
 * single-chunk prefill, which per-query selection guarantees).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (dtype, d, group size), WORKSPACE,
 * HIP. */
qsa_status qsa_sparse_attn_decode(const qsa_attn *a, const int32_t *idx, int32_t budget,
                                  int32_t ratio, const qsa_batch *b, void *out, void *ws,
                                  size_t ws_bytes, void *stream);
qsa_status qsa_sparse_attn_prefill(const qsa_attn *a, const int32_t *idx, int32_t budget,
                                   int32_t ratio, const qsa_batch *b, void *out, void *ws,
                                   size_t ws_bytes, void *stream);

/* qsa_sparse_attn_decode for callers that cannot allocate (code under HIP
 * graph capture that may not call hipMalloc, tight serving loops, harnesses
 * that forbid allocation): the same computation and the same kernels, with
 * the split partials kept in a static device array of 16 MiB that the
 * library holds on every GPU it runs on until the process ends, instead of
 * a caller workspace.  Results equal qsa_sparse_attn_decode's bit for bit.
 * All calls on one GPU share that array and keep no state in it between
 * calls; calls that overlap on one GPU (concurrent streams or threads) race
 * and give undefined results.  Errors: as qsa_sparse_attn_decode, and
 * QSA_ERR_WORKSPACE when qsa_attn_workspace_size() of the batch exceeds
 * 16 MiB (e.g. more than 2048 query rows x 32 heads at K = 512); the call
 * never allocates. */
qsa_status qsa_sparse_attn_decode_static(const qsa_attn *a, const int32_t *idx, int32_t budget,
                                         int32_t ratio, const qsa_batch *b, void *out, void *stream);

/* Block top-k with a recent window always kept: the second "llama.cpp vs
 * Atlas" report's adoption plan (section (d), phase 3, item 6) keeps the
 * most recent tokens as a union with the top-k set, and the first one
 * (section (a)3) lists a count of local blocks among the indexer's
 * parameters.  The window is taken in whole blocks.  Row i of idx
 * (int32 [total_q, K + local_blocks], K = budget/ratio) is the ascending
 * union of the blocks qsa_topk_blocks selects and the last
 * min(local_blocks, nb) complete blocks, -1 padded.  In the dense regime it
 * equals qsa_topk_blocks' row.  Attend it by passing
 * budget + local_blocks*ratio to the attention call (same token set rule:
 * the listed blocks plus the incomplete tail).  Workspace as
 * qsa_topk_blocks(budget).  Errors: as qsa_topk_blocks, plus UNSUPPORTED
 * when local_blocks < 0 or K + local_blocks > 2048. */
qsa_status qsa_topk_blocks_local(const float *scores, int64_t ld_scores, const qsa_indexer *recheck,
                                 int32_t budget, int32_t ratio, int32_t local_blocks, const qsa_batch *b,
                                 int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/* Two-stage selection from token scores: the second "vLLM vs Atlas" report
 * (section (a)3, the block-pooling refinement) scores every token, reduces
 * each block of `ratio` tokens to one score and takes the block top-k on
 * those.  Token scores come from qsa_index_score with ratio 1 on the raw
 * indexer keys (pass k_idx as kc and kv_offsets as blk_offsets); this call
 * pools them, for every query i and complete block b < floor(L_i/ratio):
 *   QSA_POOL_MAX:  blk[i,b] = max_j tok[i, b*ratio + j]
 *   QSA_POOL_MEAN: blk[i,b] = (sum_j tok[i, b*ratio + j], fp32 left to right,
 *                  from +0) * (1/ratio)
 * then qsa_topk_blocks on blk selects as usual.  The report names no
 * reduction; max is the reading that keeps a block with one strong token.
 *  tok: device f32 [total_q, ld_tok], ld_tok >= max_kv_len; blk: device f32
 *  [total_q, ld_blk], ld_blk >= ceil(max_kv_len/ratio); entries past
 *  floor(L_i/ratio) are left untouched.
 * Errors: INVALID_ARGUMENT (pointers, leading dimensions, mode),
 * UNSUPPORTED (ratio), HIP. */
#define QSA_POOL_MAX 0
#define QSA_POOL_MEAN 1
qsa_status qsa_pool_scores(const float *tok, int64_t ld_tok, int32_t ratio, int32_t mode,
                           const qsa_batch *b, float *blk, int64_t ld_blk, void *stream);

/* ---- Paged caches.  The serving engines on the pages keep K/V and the
 * indexer cache in fixed-size pages addressed through a per-sequence block
 * table (vLLM report (a)1 and (a)6: the indexer K cache and the selection go
 * through the paged KV layout; "Agentic shootout", vLLM vs Atlas: paged
 * attention over the selected blocks).  Page j of sequence s holds its
 * logical token rows j*page_size .. j*page_size + page_size - 1 and its
 * compressed rows j*(page_size/ratio) .. ; physical page p holds pool rows
 * p*page_size .. of K, V and k_idx, and p*(page_size/ratio) .. of kc and
 * kc_scale.  The _paged entry points below compute exactly what their
 * contiguous counterparts compute on the same logical rows (bit for bit: only
 * addresses change); the batch's kv_offsets give lengths only (N_s =
 * kv_offsets[s+1] - kv_offsets[s]) and blk_offsets is not read (may be NULL).
 * Every page a sequence uses must be listed; other table entries are not read. */
typedef struct qsa_paged_kv {
    const int32_t *block_table;  /* device int32 [num_seqs, max_pages]: physical page of
                                    each logical page, in [0, num_pages) */
    int64_t max_pages;           /* entries per sequence row of block_table, >= ceil(N_s/page_size) */
    int64_t num_pages;           /* physical pages in each pool */
    int32_t page_size;           /* tokens per page: a power of two and a multiple of ratio */
} qsa_paged_kv;

/* qsa_compress_keys on paged k_idx / kc / kc_scale pools (same arithmetic).
 * Errors: as qsa_compress_keys, plus INVALID_ARGUMENT (pg, block table, page
 * size not a power-of-two multiple of ratio, num_pages < 1). */
qsa_status qsa_compress_keys_paged(const void *k_idx, int32_t k_dtype, int32_t d_idx, int32_t ratio,
                                   const qsa_batch *b, const int64_t *first_block, void *kc,
                                   int32_t kc_dtype, void *kc_scale, const qsa_paged_kv *pg,
                                   void *stream);

/* qsa_index_score reading kc / kc_scale from pools (QSA_SCORE_CANONICAL only;
 * QSA_SCORE_MFMA with paging returns UNSUPPORTED). */
qsa_status qsa_index_score_paged(const qsa_indexer *ix, int32_t ratio, const qsa_batch *b,
                                 float *scores, int64_t ld_scores, uint32_t flags,
                                 const qsa_paged_kv *pg, void *stream);

/* qsa_sparse_attn_decode / _prefill reading K and V from pools (same
 * workspace as the contiguous calls). */
qsa_status qsa_sparse_attn_decode_paged(const qsa_attn *a, const int32_t *idx, int32_t budget,
                                        int32_t ratio, const qsa_batch *b, void *out, void *ws,
                                        size_t ws_bytes, const qsa_paged_kv *pg, void *stream);
qsa_status qsa_sparse_attn_prefill_paged(const qsa_attn *a, const int32_t *idx, int32_t budget,
                                         int32_t ratio, const qsa_batch *b, void *out, void *ws,
                                         size_t ws_bytes, const qsa_paged_kv *pg, void *stream);

/* Canonical scores and their block top-k in one call: the same scores and
 * the same idx, bit for bit, as qsa_index_score(ix, ratio, b, scores,
 * ld_scores, QSA_SCORE_CANONICAL, [pg]) followed by qsa_topk_blocks(scores,
 * ld_scores, NULL, budget, ratio, b, idx, ...).  For batches of at most 256
 * query rows (decode) the scorer also writes, per chunk of 64 consecutive
 * blocks, the chunk's best few blocks (enough for the chunk's expected share
 * of the top K many times over) into the workspace, and the selection is
 * made from those lists when a certificate shows it equals the selection
 * from the whole row: T, the K-th largest listed score, exceeds every
 * chunk's last listed score, so every block scoring at least T is listed.
 * A row that fails the certificate is selected from its whole score row.
 * (The "PR 16 review" report on the "Agentic shootout" page, section (b),
 * names the host-side top-k as the v1 cliff; this keeps the selection on the
 * device and small.)
 *  pg:  NULL (contiguous kc) or the paging of kc / kc_scale.
 *  ws:  device workspace of at least qsa_score_topk_workspace_size() bytes;
 *       no initialisation, no state between calls.
 * Errors: those of qsa_index_score and qsa_topk_blocks. */
size_t qsa_score_topk_workspace_size(const qsa_batch *b, int32_t budget, int32_t ratio);
qsa_status qsa_index_score_topk(const qsa_indexer *ix, int32_t budget, int32_t ratio, const qsa_batch *b,
                                float *scores, int64_t ld_scores, int32_t *idx, void *ws, size_t ws_bytes,
                                const qsa_paged_kv *pg, void *stream);

/* The whole decode step in two launches (plus the split combine): the same
 * scores, idx and out, bit for bit, as qsa_index_score_topk followed by
 * qsa_sparse_attn_decode(_paged) on the same batch.  The scorer writes its
 * per-chunk candidate lists (see qsa_index_score_topk), and every workgroup
 * of the attention kernel — one per (query, KV head, part of the selected
 * blocks) — derives the block ids of its own part from those lists with the
 * same certificate, or exactly from the query's score row when the
 * certificate fails; the workgroups of KV head 0, part 0 write idx.  No
 * workgroup waits for another, and no separate top-k launch runs.  (The
 * second "vLLM vs Atlas" report on the "Agentic shootout" page, section
 * (a)6, runs indexer, KV update and sparse attention as one step; the
 * third "Flash-Next support" report, section (d), item 3, recommends
 * splitting the key work from the query work within one launch.)
 * Decode batches of one query per sequence.  Batches of more than 256
 * queries, and K/V the matrix-core kernel does not address (fp32, or rows
 * past 32-bit offsets), run qsa_index_score_topk and qsa_sparse_attn_decode
 * instead, with the same results.
 *  ix, a:  as for qsa_index_score and qsa_sparse_attn_decode.
 *  scores: device f32 [total_q, ld_scores] (written, canonical).
 *  idx:    device int32 [total_q, budget/ratio] (written).
 *  out:    device [total_q, hq, d] (dtype of q).
 *  ws:     device workspace of at least qsa_decode_step_workspace_size()
 *          bytes, 16-byte aligned (QSA_ERR_INVALID_ARGUMENT otherwise); no
 *          initialisation, no state between calls.
 *  pg:     NULL, or the paging of kc, kc_scale, K and V.
 * Errors: those of qsa_index_score_topk and qsa_sparse_attn_decode. */
size_t qsa_decode_step_workspace_size(const qsa_batch *b, const qsa_attn *a, int32_t budget, int32_t ratio);
qsa_status qsa_decode_step(const qsa_indexer *ix, const qsa_attn *a, int32_t budget, int32_t ratio,
                           const qsa_batch *b, float *scores, int64_t ld_scores, int32_t *idx, void *out, void *ws,
                           size_t ws_bytes, const qsa_paged_kv *pg, void *stream);

/* The two halves of qsa_decode_step as separate calls, in this order on one
 * stream, with the same workspace (for a caller that times them apart or
 * puts work between them): qsa_index_score_lists writes the scores and the
 * candidate lists (into ws; a reads only the attention shape, for the
 * workspace size); qsa_sparse_attn_decode_lists selects and attends, and
 * writes idx and out.  Together they equal qsa_decode_step bit for bit.
 * Errors: as qsa_decode_step. */
qsa_status qsa_index_score_lists(const qsa_indexer *ix, const qsa_attn *a, int32_t budget, int32_t ratio,
                                 const qsa_batch *b, float *scores, int64_t ld_scores, void *ws, size_t ws_bytes,
                                 const qsa_paged_kv *pg, void *stream);
qsa_status qsa_sparse_attn_decode_lists(const qsa_attn *a, int32_t budget, int32_t ratio, const qsa_batch *b,
                                        const float *scores, int64_t ld_scores, int32_t *idx, void *out, void *ws,
                                        size_t ws_bytes, const qsa_paged_kv *pg, void *stream);


/* ---- Layers that share one selection.  The first "llama.cpp vs Atlas"
 * report (section (a)3) lists indexers that are either full or shared: a
 * shared layer attends its own K/V with the top-k of the last full layer.
 * qsa_sparse_attn_decode_layers runs the decode attention of n_layers such
 * layers (the full one and the shared ones after it) as one launch over the
 * same idx: layer l's output equals, bit for bit, that of
 * qsa_sparse_attn_decode(_paged)(&layers[l], idx, ..., outs[l]) on its own.
 *  layers: host array of n_layers (1 .. QSA_MAX_LAYERS) descriptors with
 *          the same dtype, hq, hkv and d (q, k, v and softmax_scale may
 *          differ; with pg, k and v are each layer's pools, all addressed
 *          through the one block table).
 *  outs:   host array of n_layers device pointers, each [total_q, hq, d].
 *  ws:     device workspace of at least qsa_attn_layers_workspace_size()
 *          bytes (n_layers slices, one per layer).
 *  pg:     NULL for contiguous K/V, else the paging descriptor.
 * Errors: as qsa_sparse_attn_decode, plus INVALID_ARGUMENT when n_layers is
 * out of range, an outs entry is NULL or the layers' shapes differ. */
#define QSA_MAX_LAYERS 8
size_t qsa_attn_layers_workspace_size(const qsa_batch *b, const qsa_attn *a, int32_t n_layers,
                                      int32_t budget, int32_t ratio);
qsa_status qsa_sparse_attn_decode_layers(const qsa_attn *layers, int32_t n_layers, const int32_t *idx,
                                         int32_t budget, int32_t ratio, const qsa_batch *b,
                                         void *const *outs, void *ws, size_t ws_bytes,
                                         const qsa_paged_kv *pg, void *stream);

/* ---- Ingest and rewind.  Serving engines append each new token's raw
 * indexer key and compress every block it completes inside the decode step
 * (vLLM report (a)6: one compressor work item per completed group, with the
 * raw keys of the incomplete group kept in a per-request circular buffer
 * whose capacity is a whole number of groups; the second "vLLM vs Atlas"
 * report, section (a), QSA sparse attention + indexer: the fused
 * pre-indexer commits the raw-key suffix to a circular state cache).  A rollback lowers the sequence length and must rewind the
 * indexer state with it; the defect investigations page (Defect 1, fix plan
 * PR-F) traces a crash to an indexer cursor left behind by a rollback, and
 * asks that a rewind the state cannot follow be declined.
 *
 * Here the caller's sequence lengths are the only cursor: the batch passed
 * to qsa_ingest gives each sequence's length N_s AFTER the append and its
 * n_s new tokens (positions N_s - n_s .. N_s - 1), and the pooled count is
 * floor(N_s/ratio) by definition.  A rollback is just a shorter N_s on a
 * later call; nothing in the library has to be moved back.  The only state
 * is a ring of the last raw keys per sequence and, per ring slot, the
 * window of positions it still holds, which qsa_ingest checks before it
 * completes a block from old keys. */
typedef struct qsa_key_ring {
    void *keys;            /* device [num_slots, capacity, d_idx] of the raw keys' dtype;
                              position p of a sequence lives at row p % capacity of its slot */
    int64_t *window;       /* device int64 [num_slots, 2] = {lo, hi}: the slot holds the raw
                              keys of positions lo .. hi-1.  A fresh slot is {0, 0}. */
    const int32_t *slots;  /* device int32 [num_seqs]: slot of sequence s; NULL = slot s */
    int64_t num_slots;     /* >= 1 (>= num_seqs when slots is NULL) */
    int32_t capacity;      /* tokens per slot: a multiple of ratio, >= ratio */
} qsa_key_ring;

/* Optional K/V append done by the same launch (the engine's paged KV write
 * that precedes sparse attention, vLLM report (a)6 dataflow). */
typedef struct qsa_kv_append {
    const void *k_new;     /* device [total_q, hkv, d] rows of the new tokens */
    const void *v_new;     /* device [total_q, hkv, d] */
    void *k, *v;           /* caches laid out as qsa_attn.k / .v (or pools when paged) */
    int32_t dtype;         /* QSA_F32 | QSA_BF16 */
    int32_t hkv, d;        /* hkv >= 1, d == 128 */
} qsa_kv_append;

/* Per-sequence result codes written to status[s] (device int32 [num_seqs]). */
#define QSA_INGEST_OK 0
#define QSA_INGEST_LOST_KEYS 1    /* a block completed here needs a raw key the ring no
                                     longer holds (rollback deeper than the ring, or skipped
                                     positions); that block's compressed key is NOT written */
#define QSA_INGEST_BAD_SLOT 2     /* slots[s] outside [0, num_slots): nothing written */
#define QSA_INGEST_TOO_LONG 3     /* N_s beyond the block table (paged), n_s > N_s, or more
                                     new tokens than the launch was sized for (the caller
                                     must keep n_s <= batch.max_q_per_seq): nothing written */
#define QSA_REWIND_DECLINED 4     /* qsa_ring_rewind only: see there */

/* Append the n_s new tokens of every sequence.  For each new position p
 * (ascending): the raw key k_new[row] is stored in the ring when p >= N_s -
 * capacity, and K/V rows are written when kv != NULL; for every block b in
 * floor((N_s - n_s)/ratio) .. floor(N_s/ratio) - 1 (those this append
 * completes) kc[b] (+ kc_scale[b]) is written with exactly the arithmetic of
 * qsa_compress_keys over the block's raw keys, old ones read from the ring,
 * new ones from k_new.  Reads of the ring see it as it was before the call.
 * Afterwards the slot's window is {max(lo', N_s - capacity), N_s} with lo' =
 * min(lo, N_s - n_s) (or N_s - n_s when N_s - n_s > hi: skipped positions).
 *  k_new:  device [total_q, d_idx] (rows by q_offsets; NULL q_offsets = one
 *          new token per sequence), k_dtype QSA_F32 | QSA_BF16; the ring
 *          keys have the same dtype.
 *  b:      kv_offsets give N_s after the append (and the contiguous rows of
 *          K, V when not paged); blk_offsets the kc rows when not paged;
 *          max_q_per_seq >= max n_s; max_kv_len >= max N_s.
 *  kc, kc_dtype, kc_scale: as qsa_compress_keys (any of the four dtypes).
 *  kv:     NULL, or the K/V append.
 *  status: device int32 [num_seqs] or NULL: one QSA_INGEST_* code per sequence.
 *  pg:     NULL (contiguous rows) or the paging of kc, kc_scale, K and V.
 * Sequences sharing a ring slot in one call race (undefined).  Host errors:
 * INVALID_ARGUMENT (null pointers, capacity, num_slots), UNSUPPORTED (ratio,
 * d_idx, dtypes, kv->d), HIP. */
qsa_status qsa_ingest(const void *k_new, int32_t k_dtype, int32_t d_idx, int32_t ratio,
                      const qsa_batch *b, const qsa_key_ring *ring, void *kc, int32_t kc_dtype,
                      void *kc_scale, const qsa_kv_append *kv, int32_t *status,
                      const qsa_paged_kv *pg, void *stream);

/* The decode step's append and canonical scores in one launch: the same
 * results, bit for bit, as qsa_ingest(k_new, k_dtype, ix->d_idx, ratio, b,
 * ring, ix->kc, ix->kc_dtype, ix->kc_scale, kv, status, pg) followed by
 * qsa_index_score(_paged)(ix, ratio, b, scores, ld_scores,
 * QSA_SCORE_CANONICAL, pg).  vLLM report (a)6 has the compressor work item
 * run inside the step; here the block a sequence's new token completes is
 * scored by the wave that compresses it, and every other block by the usual
 * scorer, so the append needs no launch of its own.  One new token and one
 * query per sequence (batch.q_offsets NULL), a bf16 q_idx and bf16, e4m3 or
 * fp4 compressed keys; ix->kc and ix->kc_scale are written (the indexer's
 * const pointers notwithstanding).  Errors: those of the two calls, plus
 * INVALID_ARGUMENT for q_offsets != NULL and UNSUPPORTED for other dtypes. */
qsa_status qsa_ingest_index_score(const void *k_new, int32_t k_dtype, int32_t ratio, const qsa_batch *b,
                                  const qsa_key_ring *ring, const qsa_kv_append *kv, int32_t *status,
                                  const qsa_indexer *ix, float *scores, int64_t ld_scores,
                                  const qsa_paged_kv *pg, void *stream);

/* The first half of a decode step with the append inside the scoring launch:
 * qsa_ingest_index_score (one new token per sequence: ring commit, the block
 * it completes, optional K/V rows; the canonical scores) that also writes the
 * candidate lists of qsa_index_score_lists into ws.  The block a sequence's
 * new token completes is scored by the append, so its chunk lists one block
 * fewer and leaves its last slot, which the selection fills from the score
 * row (every unlisted block is still bounded by its chunk's cutoff).  Follow
 * it with qsa_sparse_attn_decode_lists on the same stream and workspace: the
 * two calls equal qsa_ingest followed by qsa_decode_step bit for bit (scores,
 * idx, out, compressed keys, ring, statuses, K/V).  ("Agentic shootout"
 * page, vLLM vs Atlas (a)6 — indexer, KV update and sparse attention as one
 * step — and the third "Flash-Next support" report, section (d), item 3.)
 *  k_new .. status: as for qsa_ingest_index_score.
 *  ix, a, budget, ratio, b, scores, ld_scores, ws, pg: as for
 *                   qsa_index_score_lists (ws of at least
 *                   qsa_decode_step_workspace_size() bytes, 16-byte aligned).
 * Errors: those of qsa_ingest_index_score and qsa_decode_step. */
qsa_status qsa_ingest_index_score_lists(const void *k_new, int32_t k_dtype, const qsa_key_ring *ring,
                                        const qsa_kv_append *kv, int32_t *status, const qsa_indexer *ix,
                                        const qsa_attn *a, int32_t budget, int32_t ratio, const qsa_batch *b,
                                        float *scores, int64_t ld_scores, void *ws, size_t ws_bytes,
                                        const qsa_paged_kv *pg, void *stream);

/* Explicit rollback gate (defect investigations page, fix plan PR-F: a
 * rewind the indexer state cannot follow is declined, not applied).  The
 * batch's kv_offsets give the lengths N_s after the rollback.  Per sequence:
 * if N_s <= hi and min(lo, N_s) <= ratio*floor(N_s/ratio) (the ring still
 * holds the raw keys of the incomplete block), the window becomes
 * {min(lo, N_s), N_s} and status[s] = QSA_INGEST_OK; otherwise nothing
 * changes and status[s] = QSA_REWIND_DECLINED (or QSA_INGEST_BAD_SLOT).
 * Calling it is optional: qsa_ingest applies the same rule to any shorter
 * length, but reports a lost key only when the block completes.
 * Errors: INVALID_ARGUMENT (null pointers), HIP. */
qsa_status qsa_ring_rewind(const qsa_batch *b, int32_t ratio, const qsa_key_ring *ring,
                           int32_t *status, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
