// Key compression: one mean-pooled indexer key per complete block of `ratio`
// tokens ("Agentic shootout" page, report "Flash-Next support: vLLM vs Atlas",
// section (a)6: one compressed key per complete group; "PR 16 review",
// section (a): 4-token mean-pooled blocks), stored as fp32, bf16 or OCP e4m3
// with one fp32 scale max|x|/448 per block (the e4m3 index plane of the
// long-context decode workload), or as fp4 E2M1 codes with one E8M0 scale
// per 32 dims ("ATOM Model Support Guide" page, DeepSeek-V4.1 index plane).
//
// A streaming HBM pass: each wave owns whole blocks; a lane owns DPL
// consecutive dims of the d_idx-wide row, so every row load of the wave is one
// contiguous, coalesced 128..512-byte segment.  Sum in row order in fp32, then
// times 1/ratio (exact for a power-of-two ratio, identical to dividing).
#include "qsa_device.hpp"
#include "qsa_internal.hpp"
#include "qsa_kc.hpp"

namespace qsa {
namespace {

constexpr int kCompressWaves = 4;        // waves per workgroup
constexpr int kBlocksPerWave = 4;        // blocks a wave handles (loads issued together)

// KC: 0 = fp32, 1 = bf16, 2 = e4m3 (+ scale), 3 = fp4 (+ scales).  R: the
// ratio when known at compile time (4), else 0.  With R, all R rows of the
// wave's blocks are requested before any is summed; with a runtime ratio
// the rows of one block are summed before the next block's are requested,
// and each block's loads wait behind the previous block's reduction and store.
template <typename TIn, int DPL, int KC, int R>
__global__ __launch_bounds__(kCompressWaves * kWave) void compress_kernel(
    const TIn *__restrict__ k_idx, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ blk_off, const int64_t *__restrict__ first_block, int log2_ratio,
    float inv_ratio, void *__restrict__ kc, void *__restrict__ kc_scale, PageMap pm) {
    constexpr int D = DPL * kWave;
    const int s = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int ratio = 1 << log2_ratio;
    const int64_t row0 = kv_off[s];
    const int64_t nb = (kv_off[s + 1] - row0) >> log2_ratio;
    const int64_t fb = first_block ? first_block[s] : 0;
    const int64_t out0 = pm.table ? 0 : blk_off[s];
    const int64_t b_base =
        ((int64_t)blockIdx.x * kCompressWaves + wave) * kBlocksPerWave;

    if constexpr (R > 0) {
        // the wave's blocks b_base .. b_base+3 that exist and are not before
        // the first block to compress (uniform over the wave)
        const int64_t b_lo = b_base > fb ? b_base : fb;
        if (b_lo >= nb || b_lo >= b_base + kBlocksPerWave) return;
        // rows first (page lookups), then every row load, then the sums: a
        // lookup issued behind row loads would wait for all of them
        int64_t in_row[kBlocksPerWave], out_row[kBlocksPerWave];
        if (pm.table) {
#pragma unroll
            for (int u = 0; u < kBlocksPerWave; ++u) {
                const int64_t b = b_base + u;
                const int64_t bb = (b < nb && b >= fb) ? b : b_lo;   // a block that exists
                in_row[u] = paged_row(pm, s, bb << log2_ratio, pm.log2_page);
                out_row[u] = paged_row(pm, s, bb, pm.log2_page - log2_ratio);
            }
        } else {
#pragma unroll
            for (int u = 0; u < kBlocksPerWave; ++u) {
                const int64_t b = b_base + u;
                const int64_t bb = (b < nb && b >= fb) ? b : b_lo;
                in_row[u] = row0 + (bb << log2_ratio);
                out_row[u] = out0 + bb;
            }
        }
        float x[kBlocksPerWave][R][DPL];
#pragma unroll
        for (int u = 0; u < kBlocksPerWave; ++u) {
            const TIn *src = k_idx + in_row[u] * D + lane * DPL;
#pragma unroll
            for (int j = 0; j < R; ++j) load_row<TIn, DPL>(src + (int64_t)j * D, x[u][j]);
        }
#pragma unroll
        for (int u = 0; u < kBlocksPerWave; ++u) {
            const int64_t b = b_base + u;
            if (b >= nb || b < fb) continue;
            float m[DPL];
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < R; ++j) acc = acc + x[u][j][e];
                m[e] = acc * inv_ratio;
            }
            store_kc<KC, DPL>(m, kc, kc_scale, out_row[u], lane);
        }
        return;
    }
    for (int u = 0; u < kBlocksPerWave; ++u) {
        const int64_t b = b_base + u;
        if (b >= nb || b < fb) continue;
        // the block's first token row (a page holds whole blocks) and its output row
        const int64_t in_row = pm.table ? paged_row(pm, s, b << log2_ratio, pm.log2_page)
                                        : row0 + (b << log2_ratio);
        const int64_t out_row = pm.table ? paged_row(pm, s, b, pm.log2_page - log2_ratio) : out0 + b;
        const TIn *src = k_idx + in_row * D + lane * DPL;
        float acc[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
        for (int j = 0; j < ratio; ++j) {
            float x[DPL];
            load_row<TIn, DPL>(src + (int64_t)j * D, x);
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[e] = acc[e] + x[e];
        }
        float m[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) m[e] = acc[e] * inv_ratio;
        store_kc<KC, DPL>(m, kc, kc_scale, out_row, lane);
    }
}

template <typename TIn, int DPL, int R>
hipError_t dispatch_kc(const void *k_idx, const qsa_batch &b, const int64_t *fb, int log2r,
                       void *kc, int kc_dtype, void *kc_scale, const PageMap &pm, dim3 grid,
                       hipStream_t st) {
    const float inv = 1.0f / (float)(1 << log2r);
    const TIn *x = static_cast<const TIn *>(k_idx);
    dim3 block(kCompressWaves * kWave);
#define QSA_COMPRESS_LAUNCH(KC)                                                                   \
    hipLaunchKernelGGL((compress_kernel<TIn, DPL, KC, R>), grid, block, 0, st, x, b.kv_offsets,  \
                       b.blk_offsets, fb, log2r, inv, kc, kc_scale, pm)
    switch (kc_dtype) {
    case QSA_F32: QSA_COMPRESS_LAUNCH(0); break;
    case QSA_BF16: QSA_COMPRESS_LAUNCH(1); break;
    case QSA_FP8_E4M3: QSA_COMPRESS_LAUNCH(2); break;
    default: QSA_COMPRESS_LAUNCH(3); break;
    }
#undef QSA_COMPRESS_LAUNCH
    return hipGetLastError();
}

template <typename TIn, int DPL>
hipError_t dispatch_r(const void *k_idx, const qsa_batch &b, const int64_t *fb, int log2r,
                      void *kc, int kc_dtype, void *kc_scale, const PageMap &pm, dim3 grid,
                      hipStream_t st) {
    return log2r == 2 ? dispatch_kc<TIn, DPL, 4>(k_idx, b, fb, log2r, kc, kc_dtype, kc_scale, pm, grid, st)
                      : dispatch_kc<TIn, DPL, 0>(k_idx, b, fb, log2r, kc, kc_dtype, kc_scale, pm, grid, st);
}

}  // namespace

hipError_t launch_compress(const void *k_idx, int k_dtype, int d_idx, int ratio, const qsa_batch &b,
                           const int64_t *first_block, void *kc, int kc_dtype, void *kc_scale,
                           const qsa_paged_kv *pg, hipStream_t st) {
    const PageMap pm = page_map(pg);
    const int log2r = __builtin_ctz((unsigned)ratio);
    const int64_t max_nb = b.max_kv_len >> log2r;
    const int64_t per_wg = (int64_t)kCompressWaves * kBlocksPerWave;
    if (max_nb <= 0) return hipSuccess;
    dim3 grid((unsigned)((max_nb + per_wg - 1) / per_wg), (unsigned)b.num_seqs);
    trace("compress grid=(%u,%u) d_idx=%d ratio=%d k_dtype=%d kc_dtype=%d", grid.x, grid.y, d_idx,
          ratio, k_dtype, kc_dtype);
    const bool bf = (k_dtype == QSA_BF16);
    if (d_idx == 64)
        return bf ? dispatch_r<uint16_t, 1>(k_idx, b, first_block, log2r, kc, kc_dtype, kc_scale, pm, grid, st)
                  : dispatch_r<float, 1>(k_idx, b, first_block, log2r, kc, kc_dtype, kc_scale, pm, grid, st);
    return bf ? dispatch_r<uint16_t, 2>(k_idx, b, first_block, log2r, kc, kc_dtype, kc_scale, pm, grid, st)
              : dispatch_r<float, 2>(k_idx, b, first_block, log2r, kc, kc_dtype, kc_scale, pm, grid, st);
}

}  // namespace qsa
