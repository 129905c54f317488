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

// KC: 0 = fp32, 1 = bf16, 2 = e4m3 (+ scale)
template <typename TIn, int DPL, int KC>
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

template <typename TIn, int DPL>
hipError_t dispatch_kc(const void *k_idx, const qsa_batch &b, const int64_t *fb, int log2r,
                       void *kc, int kc_dtype, void *kc_scale, const PageMap &pm, dim3 grid,
                       hipStream_t st) {
    const float inv = 1.0f / (float)(1 << log2r);
    const TIn *x = static_cast<const TIn *>(k_idx);
    dim3 block(kCompressWaves * kWave);
    switch (kc_dtype) {
    case QSA_F32:
        hipLaunchKernelGGL((compress_kernel<TIn, DPL, 0>), grid, block, 0, st, x, b.kv_offsets,
                           b.blk_offsets, fb, log2r, inv, kc, kc_scale, pm);
        break;
    case QSA_BF16:
        hipLaunchKernelGGL((compress_kernel<TIn, DPL, 1>), grid, block, 0, st, x, b.kv_offsets,
                           b.blk_offsets, fb, log2r, inv, kc, kc_scale, pm);
        break;
    case QSA_FP8_E4M3:
        hipLaunchKernelGGL((compress_kernel<TIn, DPL, 2>), grid, block, 0, st, x, b.kv_offsets,
                           b.blk_offsets, fb, log2r, inv, kc, kc_scale, pm);
        break;
    default:
        hipLaunchKernelGGL((compress_kernel<TIn, DPL, 3>), grid, block, 0, st, x, b.kv_offsets,
                           b.blk_offsets, fb, log2r, inv, kc, kc_scale, pm);
        break;
    }
    return hipGetLastError();
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
        return bf ? dispatch_kc<uint16_t, 1>(k_idx, b, first_block, log2r, kc, kc_dtype, kc_scale, pm, grid, st)
                  : dispatch_kc<float, 1>(k_idx, b, first_block, log2r, kc, kc_dtype, kc_scale, pm, grid, st);
    return bf ? dispatch_kc<uint16_t, 2>(k_idx, b, first_block, log2r, kc, kc_dtype, kc_scale, pm, grid, st)
              : dispatch_kc<float, 2>(k_idx, b, first_block, log2r, kc, kc_dtype, kc_scale, pm, grid, st);
}

}  // namespace qsa
