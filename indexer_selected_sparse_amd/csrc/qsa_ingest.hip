// Ingest of new tokens inside the decode step, and the rollback gate.
//
// Serving engines append each new token's raw indexer key and compress the
// blocks it completes as part of the step ("Agentic shootout" page,
// "Flash-Next support: vLLM vs Atlas", section (a)6: one compressor work
// item per completed group, raw keys of the open group kept in a
// per-request circular buffer of whole groups; the second "vLLM vs Atlas"
// report, section (a): the fused pre-indexer commits the raw-key suffix to
// that buffer).  The lengths the caller passes are the only cursor: the new
// tokens of sequence s are its positions N_s - n_s .. N_s - 1, so a rollback
// is a shorter N_s and cannot leave an indexer counter behind (the defect
// investigations page, Defect 1, traces a crash to exactly such a counter).
//
// One wave per touched block: a work item copies its new tokens' raw keys
// into the ring (and K/V rows when asked), then, if the block is complete,
// mean-pools it with the arithmetic of the batch compression pass
// (qsa_kc.hpp), reading old raw keys from the ring and new ones from the
// input.  Only the first block of a sequence can need old keys.  Ring
// writes that would land on a row that block still has to read (appends
// longer than the ring, after any number of laps) are done by that block's
// own wave after its reads; the same wave checks and moves the slot's window
// and writes the status.
#include "qsa_device.hpp"
#include "qsa_ingest.hpp"
#include "qsa_internal.hpp"
#include "qsa_kc.hpp"

namespace qsa {
namespace {

constexpr int kIngestMaxWaves = 4;
constexpr int kIngestBlocks = 4;     // blocks per wave of the compile-time-ratio prompt ingest

// One lane's DPL raw key values of a row, as stored (the ring holds raw
// keys), and their fp32 values (exact widening, as load_row gives them).
template <typename TIn, int DPL>
struct RawRow {
    TIn v[DPL];
};
template <typename TIn, int DPL>
__device__ __forceinline__ RawRow<TIn, DPL> raw_load(const TIn *__restrict__ p) {
    RawRow<TIn, DPL> r;
    if constexpr (std::is_same<TIn, uint16_t>::value && DPL == 2) {
        const uint32_t u = *reinterpret_cast<const uint32_t *>(p);
        r.v[0] = (uint16_t)(u & 0xffffu);
        r.v[1] = (uint16_t)(u >> 16);
    } else if constexpr (std::is_same<TIn, float>::value && DPL == 2) {
        const float2 f = *reinterpret_cast<const float2 *>(p);
        r.v[0] = f.x;
        r.v[1] = f.y;
    } else {
#pragma unroll
        for (int e = 0; e < DPL; ++e) r.v[e] = p[e];
    }
    return r;
}
template <typename TIn, int DPL>
__device__ __forceinline__ void raw_store(TIn *__restrict__ p, const RawRow<TIn, DPL> &r) {
    if constexpr (std::is_same<TIn, uint16_t>::value && DPL == 2) {
        *reinterpret_cast<uint32_t *>(p) = (uint32_t)r.v[0] | ((uint32_t)r.v[1] << 16);
    } else if constexpr (std::is_same<TIn, float>::value && DPL == 2) {
        *reinterpret_cast<float2 *>(p) = make_float2(r.v[0], r.v[1]);
    } else {
#pragma unroll
        for (int e = 0; e < DPL; ++e) p[e] = r.v[e];
    }
}
template <typename TIn, int DPL>
__device__ __forceinline__ void raw_widen(const RawRow<TIn, DPL> &r, float (&x)[DPL]) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
        if constexpr (std::is_same<TIn, uint16_t>::value) x[e] = bf16_to_f32(r.v[e]);
        else x[e] = r.v[e];
    }
}

template <typename TIn, int DPL, int KC>
__global__ __launch_bounds__(kIngestMaxWaves * kWave) void ingest_one_kernel(
    const TIn *__restrict__ k_new, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ blk_off, int num_seqs, int log2r, float inv_ratio, RingArgs ring,
    void *__restrict__ kc, void *__restrict__ kc_scale, KvArgs kv, int32_t *__restrict__ status,
    PageMap pm) {
    const int lane = threadIdx.x & (kWave - 1);
    const int s = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (s >= num_seqs) return;
    (void)append_one<TIn, DPL, KC>(k_new, kv_off, blk_off, s, log2r, inv_ratio, ring, kc, kc_scale, kv, status,
                                   pm, lane);
}

// R: the ratio when known at compile time (4), else 0.  With R a wave takes
// kIngestBlocks consecutive blocks in three phases: every key row of its
// blocks is loaded once (old keys from the ring, new ones from the input),
// then the new tokens' ring and K/V rows are stored, then the complete
// blocks are mean-pooled from the loaded rows.  With a runtime ratio a wave
// takes one block and its steps go one after another.
template <typename TIn, int DPL, int KC, int R>
__global__ __launch_bounds__(kIngestMaxWaves * kWave) void ingest_kernel(
    const TIn *__restrict__ k_new, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ blk_off, const int64_t *__restrict__ q_off, int log2r,
    float inv_ratio, RingArgs ring, void *__restrict__ kc, void *__restrict__ kc_scale, KvArgs kv,
    int32_t *__restrict__ status, PageMap pm, int items_per_seq) {
    constexpr int D = DPL * kWave;
    constexpr int kKeyBytes = D * (int)sizeof(TIn);
    const int s = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int kBlk = R > 0 ? kIngestBlocks : 1;   // blocks per wave
    const int wv = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int item = wv * kBlk;                       // the wave's first block (work item)

    const int64_t row0 = kv_off[s];
    const int64_t N = kv_off[s + 1] - row0;
    const int64_t q0 = q_off ? q_off[s] : s;
    const int64_t n = q_off ? q_off[s + 1] - q0 : 1;
    const int64_t start = N - n;
    const int slot = ring.slots ? ring.slots[s] : s;

    int code = QSA_INGEST_OK;
    int64_t g_first = 0, n_items = 0;
    if (slot < 0 || slot >= ring.num_slots) {
        code = QSA_INGEST_BAD_SLOT;
    } else if (n < 0 || start < 0 || (pm.table && N > (pm.stride << pm.log2_page))) {
        code = QSA_INGEST_TOO_LONG;
    } else {
        g_first = start >> log2r;
        n_items = n > 0 ? ((N - 1) >> log2r) - g_first + 1 : 0;
        if (n_items > items_per_seq) code = QSA_INGEST_TOO_LONG;
    }
    if (code != QSA_INGEST_OK) {
        if (item == 0 && lane == 0 && status) status[s] = code;
        return;
    }
    if (item >= n_items && item != 0) return;   // (item 0: the window and status below)

    const int64_t cap = ring.cap;
    TIn *const rkeys = static_cast<TIn *>(ring.keys) + (int64_t)slot * cap * D;
    int64_t *const win = ring.window + 2 * (int64_t)slot;
    // The ring keeps positions >= keep_lo.  The first block may read n_old old
    // keys (positions bf .. start-1); a kept new position whose ring row holds
    // one of them, (q - bf) % cap < n_old, at any number of laps around the
    // ring, is written by the first block's wave after its reads.
    const int64_t keep_lo = N - cap;
    const int64_t bf = g_first << log2r;
    const int64_t n_old = start - bf;
    bool lost = false;

    if constexpr (R > 0) {
        if (item < n_items) {
            // 1: every key row of the wave's blocks (rows past N, and blocks
            // past the append, read a row that exists and are not used)
            RawRow<TIn, DPL> raw[kBlk][R];
#pragma unroll
            for (int u = 0; u < kBlk; ++u) {
                const int64_t g = g_first + (item + u < n_items ? item + u : item);
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    const int64_t p0 = g * R + j;
                    const int64_t p = p0 < N ? p0 : N - 1;
                    const TIn *src = p < start ? rkeys + pos_mod(p, cap) * D : k_new + (q0 + p - start) * D;
                    raw[u][j] = raw_load<TIn, DPL>(src + lane * DPL);
                }
            }
            // 2: the new tokens' ring rows (those no old key of the first
            // block sits on) and K/V rows
#pragma unroll
            for (int u = 0; u < kBlk; ++u) {
                if (item + u >= n_items) break;                  // uniform
                const int64_t b0 = (g_first + item + u) * R;
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    const int64_t p = b0 + j;
                    if (p < start || p >= N) continue;           // uniform
                    if (p >= keep_lo && pos_mod(p - bf, cap) >= n_old)
                        raw_store<TIn, DPL>(rkeys + pos_mod(p, cap) * D + lane * DPL, raw[u][j]);
                    if (kv.row_bytes) {
                        const int64_t dst = pm.table ? paged_row(pm, s, p, pm.log2_page) : row0 + p;
                        const int64_t srow = q0 + p - start;
                        copy_row(kv.k + dst * kv.row_bytes, kv.k_new + srow * kv.row_bytes, kv.row_bytes, lane);
                        copy_row(kv.v + dst * kv.row_bytes, kv.v_new + srow * kv.row_bytes, kv.row_bytes, lane);
                    }
                }
            }
            // 3: the complete blocks' means, rows summed in token order
#pragma unroll
            for (int u = 0; u < kBlk; ++u) {
                if (item + u >= n_items) break;                  // uniform
                const int64_t g = g_first + item + u;
                const int64_t b0 = g * R;
                if (b0 + R > N) continue;                         // the append does not complete it
                if (b0 < start) {                                 // old keys came from the ring (g == g_first)
                    const int64_t lo = win[0], hi = win[1];
                    const int64_t lo_eff = start <= hi ? (lo < start ? lo : start) : start;
                    lost = lo_eff > b0;
                    if (lost) continue;
                }
                float acc[DPL];
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    float x[DPL];
                    raw_widen<TIn, DPL>(raw[u][j], x);
#pragma unroll
                    for (int e = 0; e < DPL; ++e) acc[e] = acc[e] + x[e];
                }
                float m[DPL];
#pragma unroll
                for (int e = 0; e < DPL; ++e) m[e] = acc[e] * inv_ratio;
                const int64_t out_row = pm.table ? paged_row(pm, s, g, pm.log2_page - log2r) : blk_off[s] + g;
                store_kc<KC, DPL>(m, kc, kc_scale, out_row, lane);
            }
        }
    } else if (item < n_items) {
        const int64_t g = g_first + item;
        const int64_t b0 = g << log2r;
        const int64_t t0 = b0 > start ? b0 : start;
        const int64_t t1 = b0 + (int64_t(1) << log2r) < N ? b0 + (int64_t(1) << log2r) : N;
        for (int64_t p = t0; p < t1; ++p) {
            const TIn *src = k_new + (q0 + p - start) * D;
            if (p >= keep_lo && pos_mod(p - bf, cap) >= n_old)
                copy_row(reinterpret_cast<uint8_t *>(rkeys + pos_mod(p, cap) * D),
                         reinterpret_cast<const uint8_t *>(src), kKeyBytes, lane);
            if (kv.row_bytes) {
                const int64_t dst = pm.table ? paged_row(pm, s, p, pm.log2_page) : row0 + p;
                const int64_t srow = q0 + p - start;
                copy_row(kv.k + dst * kv.row_bytes, kv.k_new + srow * kv.row_bytes, kv.row_bytes, lane);
                copy_row(kv.v + dst * kv.row_bytes, kv.v_new + srow * kv.row_bytes, kv.row_bytes, lane);
            }
        }
        if (b0 + (int64_t(1) << log2r) <= N) {   // the append completes block g
            if (b0 < start) {                    // old keys come from the ring (g == g_first)
                const int64_t lo = win[0], hi = win[1];
                const int64_t lo_eff = start <= hi ? (lo < start ? lo : start) : start;
                lost = lo_eff > b0;
            }
            if (!lost) {
                float acc[DPL];
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
                for (int j = 0; j < (1 << log2r); ++j) {
                    const int64_t p = b0 + j;
                    const TIn *src = p < start ? rkeys + pos_mod(p, cap) * D : k_new + (q0 + p - start) * D;
                    float x[DPL];
                    load_row<TIn, DPL>(src + lane * DPL, x);
#pragma unroll
                    for (int e = 0; e < DPL; ++e) acc[e] = acc[e] + x[e];
                }
                float m[DPL];
#pragma unroll
                for (int e = 0; e < DPL; ++e) m[e] = acc[e] * inv_ratio;
                const int64_t out_row = pm.table ? paged_row(pm, s, g, pm.log2_page - log2r) : blk_off[s] + g;
                store_kc<KC, DPL>(m, kc, kc_scale, out_row, lane);
            }
        }
    }
    if (item != 0) return;

    // First block's wave: the ring rows it has just read may now be replaced,
    // each by the one kept position (in keep_lo .. N-1) that maps to it, if
    // that position is new.
    if (n_old > 0 && n > 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        for (int64_t j = 0; j < n_old; ++j) {
            const int64_t p = bf + j;
            const int64_t q = keep_lo + (((p - keep_lo) % cap) + cap) % cap;
            if (q >= start && q < N)
                copy_row(reinterpret_cast<uint8_t *>(rkeys + pos_mod(q, cap) * D),
                         reinterpret_cast<const uint8_t *>(k_new + (q0 + q - start) * D), kKeyBytes, lane);
        }
    }
    if (lane == 0) {
        const int64_t lo = win[0], hi = win[1];
        const int64_t lo_eff = start <= hi ? (lo < start ? lo : start) : start;
        win[0] = lo_eff > keep_lo ? lo_eff : keep_lo;
        win[1] = N;
        if (status) status[s] = lost ? QSA_INGEST_LOST_KEYS : QSA_INGEST_OK;
    }
}

__global__ __launch_bounds__(256) void ring_rewind_kernel(const int64_t *__restrict__ kv_off, int num_seqs,
                                                          int log2r, RingArgs ring,
                                                          int32_t *__restrict__ status) {
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= num_seqs) return;
    const int64_t N = kv_off[s + 1] - kv_off[s];
    const int slot = ring.slots ? ring.slots[s] : s;
    if (slot < 0 || slot >= ring.num_slots) {
        if (status) status[s] = QSA_INGEST_BAD_SLOT;
        return;
    }
    int64_t *const win = ring.window + 2 * (int64_t)slot;
    const int64_t lo = win[0], hi = win[1];
    const int64_t lo2 = lo < N ? lo : N;
    const bool ok = N >= 0 && N <= hi && lo2 <= ((N >> log2r) << log2r);
    if (ok) {
        win[0] = lo2;
        win[1] = N;
    }
    if (status) status[s] = ok ? QSA_INGEST_OK : QSA_REWIND_DECLINED;
}

template <typename TIn, int DPL>
hipError_t dispatch_ingest(const void *k_new, const qsa_batch &b, int log2r, const RingArgs &ring,
                           void *kc, int kc_dtype, void *kc_scale, const KvArgs &kv, int32_t *status,
                           const PageMap &pm, dim3 grid, dim3 block, int items, hipStream_t st) {
    const float inv = 1.0f / (float)(1 << log2r);
    const TIn *x = static_cast<const TIn *>(k_new);
#define QSA_INGEST_LAUNCH(KC)                                                                       \
    if (b.q_offsets == nullptr)                                                                     \
        hipLaunchKernelGGL((ingest_one_kernel<TIn, DPL, KC>), grid, block, 0, st, x, b.kv_offsets,  \
                           b.blk_offsets, b.num_seqs, log2r, inv, ring, kc, kc_scale, kv, status,  \
                           pm);                                                                     \
    else if (log2r == 2)                                                                            \
        hipLaunchKernelGGL((ingest_kernel<TIn, DPL, KC, 4>), grid, block, 0, st, x, b.kv_offsets,   \
                           b.blk_offsets, b.q_offsets, log2r, inv, ring, kc, kc_scale, kv, status, \
                           pm, items);                                                              \
    else                                                                                            \
        hipLaunchKernelGGL((ingest_kernel<TIn, DPL, KC, 0>), grid, block, 0, st, x, b.kv_offsets,   \
                           b.blk_offsets, b.q_offsets, log2r, inv, ring, kc, kc_scale, kv, status, \
                           pm, items)
    switch (kc_dtype) {
    case QSA_F32: QSA_INGEST_LAUNCH(0); break;
    case QSA_BF16: QSA_INGEST_LAUNCH(1); break;
    case QSA_FP8_E4M3: QSA_INGEST_LAUNCH(2); break;
    default: QSA_INGEST_LAUNCH(3); break;
    }
#undef QSA_INGEST_LAUNCH
    return hipGetLastError();
}

RingArgs ring_args(const qsa_key_ring &r) {
    return RingArgs{r.keys, r.window, r.slots, r.num_slots, (int64_t)r.capacity};
}

}  // namespace

hipError_t launch_ingest(const void *k_new, int k_dtype, int d_idx, int ratio, const qsa_batch &b,
                         const qsa_key_ring &ring, void *kc, int kc_dtype, void *kc_scale,
                         const qsa_kv_append *kv, int32_t *status, const qsa_paged_kv *pg,
                         hipStream_t st) {
    const PageMap pm = page_map(pg);
    const int log2r = __builtin_ctz((unsigned)ratio);
    const int64_t max_n = b.q_offsets ? (int64_t)b.max_q_per_seq : 1;
    // blocks one sequence's append touches: at most floor((n + ratio - 2)/ratio) + 1
    const int64_t items = max_n > 0 ? (max_n + ratio - 2) / ratio + 1 : 1;
    // blocks per wave: kIngestBlocks on the compile-time ratio-4 path
    const int64_t kb = (log2r == 2) ? kIngestBlocks : 1;
    const int64_t wave_items = (items + kb - 1) / kb;
    int waves = (int)(wave_items < kIngestMaxWaves ? wave_items : kIngestMaxWaves);
    dim3 grid((unsigned)((wave_items + waves - 1) / waves), (unsigned)b.num_seqs);
    const int cap_items = (int)(grid.x * waves * kb);
    if (b.q_offsets == nullptr) {   // one token per sequence: one wave per sequence
        waves = kIngestMaxWaves;
        grid = dim3((unsigned)((b.num_seqs + waves - 1) / waves));
    }
    dim3 block(waves * kWave);
    KvArgs kva{nullptr, nullptr, nullptr, nullptr, 0};
    if (kv) {
        kva.k_new = static_cast<const uint8_t *>(kv->k_new);
        kva.v_new = static_cast<const uint8_t *>(kv->v_new);
        kva.k = static_cast<uint8_t *>(kv->k);
        kva.v = static_cast<uint8_t *>(kv->v);
        kva.row_bytes = kv->hkv * kv->d * (kv->dtype == QSA_BF16 ? 2 : 4);
    }
    const RingArgs ra = ring_args(ring);
    trace("ingest grid=(%u,%u) waves=%d d_idx=%d ratio=%d cap=%d kv=%d", grid.x, grid.y, waves, d_idx,
          ratio, ring.capacity, kva.row_bytes);
    const bool bf = (k_dtype == QSA_BF16);
    if (d_idx == 64)
        return bf ? dispatch_ingest<uint16_t, 1>(k_new, b, log2r, ra, kc, kc_dtype, kc_scale, kva, status,
                                                 pm, grid, block, cap_items, st)
                  : dispatch_ingest<float, 1>(k_new, b, log2r, ra, kc, kc_dtype, kc_scale, kva, status,
                                              pm, grid, block, cap_items, st);
    return bf ? dispatch_ingest<uint16_t, 2>(k_new, b, log2r, ra, kc, kc_dtype, kc_scale, kva, status, pm,
                                             grid, block, cap_items, st)
              : dispatch_ingest<float, 2>(k_new, b, log2r, ra, kc, kc_dtype, kc_scale, kva, status, pm,
                                          grid, block, cap_items, st);
}

hipError_t launch_ring_rewind(const qsa_batch &b, int ratio, const qsa_key_ring &ring, int32_t *status,
                              hipStream_t st) {
    const int log2r = __builtin_ctz((unsigned)ratio);
    const int threads = 256;
    dim3 grid((unsigned)((b.num_seqs + threads - 1) / threads));
    trace("ring_rewind grid=%u seqs=%d", grid.x, b.num_seqs);
    hipLaunchKernelGGL(ring_rewind_kernel, grid, dim3(threads), 0, st, b.kv_offsets, b.num_seqs, log2r,
                       ring_args(ring), status);
    return hipGetLastError();
}

}  // namespace qsa
