// Debug-mode checks of device-side argument contents (QSA_DEBUG=1).
//
// The host validates every argument it can see before a launch; the contents
// of device arrays (offsets, selections, block tables) it never reads.  In
// debug mode each entry point first runs this check kernel over them, waits
// for it and reads one status word: a violation is returned as
// QSA_ERR_DEVICE_ASSERT and the call's own kernels are not launched, so an
// offset past max_kv_len, a selected block id outside [-1, nb) or a page id
// outside the pools never reaches a gather.  ("Atlas Flash-Next defect
// investigations" page, Defect 4, proposed fix, items 1-2 — trace every
// launch and assert offsets under a debug flag — and fix plan PR-G — typed
// row offsets with debug asserts; "Agentic shootout" page, first "PR 16
// review" report, section (e), test 7 — a preflight check of arena bounds.)
//
// The check reads only what the call itself may read: B + 1 offsets per
// offset array, total_q rows of the selection and, per sequence, at most
// max_pages block-table entries.  The first violation recorded wins, with
// two numbers naming where it is; the word is cleared before each check.
#include "qsa_debug.hpp"
#include "qsa_device.hpp"

namespace qsa {

namespace {

struct DebugWord {
    int32_t code;
    int32_t pad;
    int64_t where;   // sequence or query index
    int64_t value;   // the offending value
};

__device__ DebugWord g_debug_word;

__device__ void report(int32_t code, int64_t where, int64_t value) {
    if (atomicCAS(&g_debug_word.code, 0, code) == 0) {
        g_debug_word.where = where;
        g_debug_word.value = value;
    }
}

__global__ void debug_clear_kernel() {
    if (threadIdx.x == 0) {
        g_debug_word.code = 0;
        g_debug_word.where = 0;
        g_debug_word.value = 0;
    }
}

constexpr int kDbgThreads = 256;

// Blocks [0, seq_blocks) check one sequence per thread; the rest check one
// selection entry per thread.
__global__ __launch_bounds__(kDbgThreads) void debug_check_kernel(DebugCheck c, int seq_blocks) {
    if ((int)blockIdx.x < seq_blocks) {
        const int s = blockIdx.x * kDbgThreads + threadIdx.x;
        if (s > c.num_seqs) return;
        if (s == 0) {
            if (c.kv_off[0] != 0) report(QSA_DBG_KV_OFFSETS, 0, c.kv_off[0]);
            if (c.blk_off && c.kv_off[0] == 0 && c.blk_off[0] != 0) report(QSA_DBG_BLK_OFFSETS, 0, c.blk_off[0]);
            if (c.q_off) {
                if (c.q_off[0] != 0) report(QSA_DBG_Q_OFFSETS, 0, c.q_off[0]);
                if (c.q_off[c.num_seqs] != c.total_q) report(QSA_DBG_Q_OFFSETS, c.num_seqs, c.q_off[c.num_seqs]);
            }
            return;
        }
        const int q = s - 1;                               // sequence q: rows kv_off[q] .. kv_off[q+1]
        const int64_t n = c.kv_off[q + 1] - c.kv_off[q];
        if (n < 0 || n > c.max_kv_len) {
            report(QSA_DBG_KV_OFFSETS, q, n);
            return;
        }
        if (c.blk_off) {
            const int64_t nb = c.blk_off[q + 1] - c.blk_off[q];
            if (nb != (n >> c.log2r)) report(QSA_DBG_BLK_OFFSETS, q, nb);
        }
        if (c.q_off) {
            const int64_t nq = c.q_off[q + 1] - c.q_off[q];
            if (nq < 0 || (c.strict_q && (nq > n || nq > c.max_q_per_seq))) report(QSA_DBG_Q_OFFSETS, q, nq);
        }
        if (c.table) {
            const int64_t pages = (n + c.page_size - 1) / c.page_size;
            for (int64_t j = 0; j < pages && j < c.max_pages; ++j) {
                const int32_t p = c.table[(int64_t)q * c.max_pages + j];
                if (p < 0 || p >= c.num_pages) {
                    report(QSA_DBG_PAGE_ID, q, p);
                    break;
                }
            }
        }
        return;
    }
    if (!c.idx) return;
    const int64_t e = (int64_t)(blockIdx.x - seq_blocks) * kDbgThreads + threadIdx.x;
    if (e >= c.total_q * c.ldi) return;
    const int64_t i = e / c.ldi;
    const int32_t b = c.idx[e];
    if (b == -1) return;
    // the query's visible blocks (offsets already checked by the other
    // blocks; a query of a malformed batch may see a wrong nb here, which
    // only changes which violation is reported first)
    int seq = (int)i;
    int64_t L;
    if (c.q_off == nullptr) {
        if (i >= c.num_seqs) return;
        L = c.kv_off[i + 1] - c.kv_off[i];
    } else {
        int lo = 0, hi = c.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (c.q_off[mid] <= i) lo = mid; else hi = mid - 1;
        }
        seq = lo;
        const int64_t n = c.kv_off[seq + 1] - c.kv_off[seq];
        const int64_t nq = c.q_off[seq + 1] - c.q_off[seq];
        L = n - nq + (i - c.q_off[seq]) + 1;
    }
    const int64_t nb = L >> c.log2r;
    if (b < -1 || (int64_t)b >= nb) report(QSA_DBG_IDX_RANGE, i, b);
}

}  // namespace

hipError_t launch_debug_check(const DebugCheck &c, hipStream_t st) {
    hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(64), 0, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int seq_blocks = (c.num_seqs + 1 + kDbgThreads - 1) / kDbgThreads;
    const int64_t entries = c.idx ? c.total_q * (int64_t)c.ldi : 0;
    const int64_t idx_blocks = (entries + kDbgThreads - 1) / kDbgThreads;
    hipLaunchKernelGGL(debug_check_kernel, dim3((unsigned)(seq_blocks + idx_blocks)), dim3(kDbgThreads), 0, st, c,
                       seq_blocks);
    return hipGetLastError();
}

hipError_t read_debug_status(hipStream_t st, int32_t &code, int64_t &where, int64_t &value) {
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return e;
    DebugWord w{};
    e = hipMemcpyFromSymbol(&w, HIP_SYMBOL(g_debug_word), sizeof(w), 0, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
    code = w.code;
    where = w.where;
    value = w.value;
    return hipSuccess;
}

}  // namespace qsa
