// Internal launcher declarations of libqsa (host side).  Every launcher is
// called only after the C-ABI layer has validated its arguments; launchers
// enqueue work on `st` and return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

// Paged pools (pg != nullptr) or the contiguous layout (pg == nullptr) for the
// launchers that take `pg`.

// Key compression (mean-pool of complete blocks).
hipError_t launch_compress(const void *k_idx, int k_dtype, int d_idx, int ratio, const qsa_batch &b,
                           const int64_t *first_block, void *kc, int kc_dtype, void *kc_scale,
                           const qsa_paged_kv *pg, hipStream_t st);

// Canonical (bit-defined) indexer scores, decode and prefill; with la.keys
// set, also the per-chunk candidate lists of qsa_lists.hpp.
struct ListArgs;
hipError_t launch_score_canonical(const qsa_indexer &ix, int ratio, const qsa_batch &b,
                                  float *scores, int64_t ld, const qsa_paged_kv *pg, hipStream_t st,
                                  const ListArgs &la);

// Block pooling of token scores (QSA_POOL_MAX / QSA_POOL_MEAN).
hipError_t launch_pool_scores(const float *tok, int64_t ld_tok, int ratio, int mode, const qsa_batch &b,
                              float *blk, int64_t ld_blk, hipStream_t st);

// Matrix-core indexer scores (bf16 only), prefill.
hipError_t launch_score_mfma(const qsa_indexer &ix, int ratio, const qsa_batch &b, float *scores,
                             int64_t ld, hipStream_t st);

// Block top-k.  recheck == nullptr: scores are canonical.  With recheck the
// rows are cached whole in LDS, which bounds the blocks per row.
constexpr int64_t kTopkRecheckMaxBlocks = 32768;
size_t topk_workspace_bytes(const qsa_batch &b, int budget, int ratio, const qsa_indexer *recheck);
hipError_t launch_topk(const float *scores, int64_t ld, const qsa_indexer *recheck, int budget,
                       int ratio, const qsa_batch &b, int32_t *idx, int ldi, void *ws, hipStream_t st);
// Canonical scores and their block top-k in one call (qsa_index_score_topk):
// few-row batches take the scorer's candidate lists (qsa_lists.hpp) and the
// list finish; larger batches the two plain launches.
bool score_topk_uses_lists(const qsa_batch &b);
size_t score_topk_workspace_bytes(const qsa_batch &b, int budget, int ratio);
hipError_t launch_score_topk(const qsa_indexer &ix, int budget, int ratio, const qsa_batch &b, float *scores,
                             int64_t ld, int32_t *idx, void *ws, const qsa_paged_kv *pg, hipStream_t st);
// In place: row i of idx (stride ldi) becomes the ascending union of its
// top-K selection and the last local_blocks complete blocks.
hipError_t launch_topk_local(int budget, int ratio, int local_blocks, const qsa_batch &b, int32_t *idx,
                             int ldi, hipStream_t st);

// Sparse gather attention (decode and prefill share the kernel).
int attn_num_splits(const qsa_batch &b, const qsa_attn &a, int budget, int ratio, bool decode);
// Workspace of the decode entry point (prefill needs none).
size_t attn_workspace_bytes(const qsa_batch &b, const qsa_attn &a, int budget, int ratio);
hipError_t launch_attn(const qsa_attn &a, const int32_t *idx, int budget, int ratio,
                       const qsa_batch &b, void *out, void *ws, bool decode, const qsa_paged_kv *pg,
                       hipStream_t st);

// Decode attention that selects its own blocks from the scorer's candidate
// lists (qsa_decode_step): bf16 K/V on the matrix-core path only.
bool attn_select_supported(const qsa_batch &b, const qsa_attn &a, const qsa_paged_kv *pg);
hipError_t launch_attn_select(const qsa_attn &a, int budget, int ratio, const qsa_batch &b, const ListArgs &la,
                              const float *scores, int64_t ld, int32_t *idx, void *out, void *ws,
                              const qsa_paged_kv *pg, hipStream_t st);
// The same for lists of more than 4096 entries per row (K = 2048 rows), in
// a translation unit of its own (qsa_attn_wide.hip).
hipError_t launch_attn_select_wide(const qsa_attn &a, int budget, int ratio, const qsa_batch &b, const ListArgs &la,
                                   const float *scores, int64_t ld, int32_t *idx, void *out, void *ws,
                                   const qsa_paged_kv *pg, hipStream_t st);
// The lists of a score + select call (workspace carve-up shared by the calls
// that take them), and the list finish alone.
ListArgs list_args(const qsa_batch &b, int budget, int ratio, void *ws);
hipError_t launch_topk_from_lists(const float *scores, int64_t ld, int budget, int ratio, const qsa_batch &b,
                                  int32_t *idx, const ListArgs &la, hipStream_t st);

// Decode attention with the split partials in a static device array (no
// caller workspace): its size, and its address on the current device
// (resolved with hipGetSymbolAddress on the first call per device).
constexpr size_t kAttnStaticScratchBytes = size_t(16) << 20;
constexpr int kMaxScratchDevices = 64;
hipError_t attn_static_scratch(void **ptr);

// Decode attention of several layers sharing one selection (one launch on
// the matrix-core path); workspace: n_layers slices of attn_layer_stride_bytes.
size_t attn_layer_stride_bytes(const qsa_batch &b, const qsa_attn &a, int budget, int ratio);
hipError_t launch_attn_layers(const qsa_attn *layers, int n_layers, const int32_t *idx, int budget, int ratio,
                              const qsa_batch &b, void *const *outs, void *ws, const qsa_paged_kv *pg,
                              hipStream_t st);

// Append of one new token per sequence and the canonical scores of a decode
// step in one launch (bf16 q_idx; bf16, e4m3 or fp4 compressed keys).
// With la.keys set, also the candidate lists (the chunk of the block each
// row's newest token completes leaves its last slot to the selection).
hipError_t launch_ingest_score(const void *k_new, int k_dtype, int ratio, const qsa_batch &b,
                               const qsa_key_ring &ring, const qsa_kv_append *kv, int32_t *status,
                               const qsa_indexer &ix, float *scores, int64_t ld, const qsa_paged_kv *pg,
                               hipStream_t st, const ListArgs &la);

// Ingest of new tokens (ring commit, completed-block compression, optional
// K/V append) and the ring's rollback gate.
hipError_t launch_ingest(const void *k_new, int k_dtype, int d_idx, int ratio, const qsa_batch &b,
                         const qsa_key_ring &ring, void *kc, int kc_dtype, void *kc_scale,
                         const qsa_kv_append *kv, int32_t *status, const qsa_paged_kv *pg,
                         hipStream_t st);
hipError_t launch_ring_rewind(const qsa_batch &b, int ratio, const qsa_key_ring &ring, int32_t *status,
                              hipStream_t st);

// Host tracing (QSA_TRACE=1): one line per launch on stderr.
// Allow a kernel `bytes` of dynamic LDS on the current device (once per
// kernel, size and device; later calls return at once).
hipError_t enable_dyn_lds(const void *fn, int bytes);
bool trace_enabled();
void trace(const char *fmt, ...);

}  // namespace qsa
