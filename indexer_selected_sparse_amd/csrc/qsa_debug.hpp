// Debug-mode checks of device-side argument contents (host interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

// Violation codes of the debug check (0 = none).
enum : int32_t {
    QSA_DBG_KV_OFFSETS = 1,   // kv_offsets[0] != 0, a negative length or N_s > max_kv_len
    QSA_DBG_BLK_OFFSETS = 2,  // blk_offsets not the prefix sums of floor(N_s / ratio)
    QSA_DBG_Q_OFFSETS = 3,    // q_offsets[0] != 0, q_offsets[B] != total_q, n_s < 0, n_s > N_s or > max_q_per_seq
    QSA_DBG_IDX_RANGE = 4,    // a selected block id outside [-1, floor(L / ratio))
    QSA_DBG_PAGE_ID = 5,      // a block-table entry of a used page outside [0, num_pages)
};

// What one call's check reads; null pointers are not checked.
struct DebugCheck {
    const int64_t *kv_off = nullptr, *blk_off = nullptr, *q_off = nullptr;
    int num_seqs = 0;
    int max_q_per_seq = 1;
    int64_t total_q = 0;
    int64_t max_kv_len = 0;
    int log2r = 0;
    const int32_t *idx = nullptr;     // selection rows [total_q, ldi]
    int ldi = 0;
    const int32_t *table = nullptr;   // block table [num_seqs, max_pages]
    int64_t max_pages = 0, num_pages = 0;
    int page_size = 1;
    bool strict_q = true;             // n_s > N_s and n_s > max_q_per_seq are violations
                                      // (ingest reports them per sequence instead)
};

// Clear the status word and enqueue the check on `st`.
hipError_t launch_debug_check(const DebugCheck &c, hipStream_t st);
// Wait for `st` and read the status word: code 0 = no violation; otherwise
// `where` is the sequence or query index and `value` the offending value.
hipError_t read_debug_status(hipStream_t st, int32_t &code, int64_t &where, int64_t &value);

}  // namespace qsa
