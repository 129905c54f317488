// Indexer scores for prefill on the matrix cores.
//
// With many queries per sequence the score s[i,b] = sum_h w[i,h] *
// ReLU(q_idx[i,h,:] . kc[b,:]) is a dense contraction: rows (query, head)
// of Q_idx times the compressed keys, followed by a ReLU and a w-weighted
// sum over the head rows of each query.  The relu score is the one of the
// "Agentic shootout" page, "PR 16 review" section (a); only blocks visible
// to a query, (b+1)*ratio <= L, are written (vLLM report section (a)6:
// complete groups only, causal within the chunk).
//
// MFMA sums the D products of a dot in an order the hardware chooses, so
// these scores are not the canonical ones; they lie within the bound that
// the certifying top-k uses (bf16 products are exact, every fp32 addition
// of a D-term sum has relative error at most 2^-23, see qsa_topk.hip), and
// the top-k restores the canonical selection.
//
// Tiling (v_mfma_f32_16x16x32_bf16, wave64): a 16x16 tile takes rows
// (query, head) as M and 16 blocks as N, D in steps of 32.  Operand A (one
// row per lane%16, 8 consecutive d per lane/16) and operand B (one block per
// lane%16, same d) are both row-major in d, so they load as 16-byte vectors.
// The result tile gives lane l the rows 4*(l/16) .. +3 of block l%16, i.e.
// up to four heads of one query, so the head sum is in-lane plus at most two
// lane swaps (gfx950 permlane16/32 swap) for 8 or 16 heads.
//
// A workgroup of 4 waves owns 256 rows (256/H queries) of one sequence and a
// chunk of kChunk blocks.  Each wave keeps its 64 rows of Q_idx in registers
// for the whole chunk; the blocks stream through LDS in slabs of 64 (double
// buffered, the next slab's global loads in flight while the current one is
// multiplied).  Chunks past the last visible block of the workgroup's
// queries are skipped (causal prefill leaves a triangle of empty tiles).
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaThreads = 256;
constexpr int kRowTiles = 4;          // 16-row tiles per wave
constexpr int kSlab = 64;             // blocks per LDS slab
constexpr int kChunk = 1024;          // blocks per workgroup

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float swap16_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Three workgroups per CU (168 registers, the LDS slabs fit three times):
// 203 us against 218 us at two for the 8193-query prefill chunk.
template <int H, int D>
__global__ __launch_bounds__(kMfmaThreads, 3) void score_mfma_kernel(
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w,
    const uint16_t *__restrict__ kc, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ blk_off, const int64_t *__restrict__ q_off, int log2r,
    int n_chunks, float *__restrict__ scores, int64_t ld) {
    constexpr int KS = D / 32;                     // MFMA k-steps
    constexpr int QPW = 64 / H;                    // queries per wave
    constexpr int QW = 4 * QPW;                    // queries per workgroup
    constexpr int LROW = D + 8;                    // LDS row (bf16), 16-byte pad
    constexpr int VPR = D / 8;                     // 16-byte vectors per key row
    constexpr int LOADS = kSlab * VPR / kMfmaThreads;
    static_assert(LOADS * kMfmaThreads == kSlab * VPR, "slab load split");
    __shared__ __attribute__((aligned(16))) uint16_t slab[2][kSlab * LROW];

    const int s = blockIdx.y;
    const int qg = blockIdx.x / n_chunks;
    const int ch = blockIdx.x - qg * n_chunks;
    const int64_t kv0 = kv_off[s];
    const int64_t N = kv_off[s + 1] - kv0;
    const int64_t q0 = q_off ? q_off[s] : s;
    const int64_t nq = q_off ? q_off[s + 1] - q0 : 1;
    const int64_t kb0 = blk_off[s];
    const int64_t qa = (int64_t)qg * QW;
    if (qa >= nq) return;
    const int64_t first_L = N - nq + 1;            // visible length of query 0
    const int64_t nb_last = (first_L + imin64(qa + QW, nq) - 1) >> log2r;
    const int64_t c0 = (int64_t)ch * kChunk;
    if (c0 >= nb_last) return;
    const int64_t c1 = imin64(c0 + kChunk, nb_last);

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane >> 4;
    const int col = lane & 15;

    // This wave's rows: r = wave*64 + rt*16 + (lane%16) -> query r/H, head r%H.
    bf16x8 A[kRowTiles][KS];
    float wv[kRowTiles][4];
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
        const int r = wave * 64 + rt * 16 + col;
        const int64_t qq = qa + r / H;
        const uint4 *src = reinterpret_cast<const uint4 *>(
            q_idx + ((q0 + qq) * H + (r % H)) * (int64_t)D + 8 * g);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            A[rt][ks] = as_bf16x8(qq < nq ? src[4 * ks] : make_uint4(0, 0, 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ro = wave * 64 + rt * 16 + 4 * g + i;
            const int64_t qo = qa + ro / H;
            wv[rt][i] = qo < nq ? w[(q0 + qo) * H + (ro % H)] : 0.0f;
        }
    }
    const int64_t wq_last = imin64(qa + (int64_t)(wave + 1) * QPW, nq) - 1;
    const int64_t nb_wave = qa + (int64_t)wave * QPW < nq ? (first_L + wq_last) >> log2r : 0;

    // slab prefetch: vector e = j*256 + tid -> block e / VPR, vector e % VPR
    uint4 pf[LOADS];
    auto prefetch = [&](int64_t base) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int e = j * kMfmaThreads + threadIdx.x;
            const int64_t blk = base + e / VPR;
            pf[j] = blk < c1 ? reinterpret_cast<const uint4 *>(kc + (kb0 + blk) * D)[e % VPR]
                             : make_uint4(0, 0, 0, 0);
        }
    };
    prefetch(c0);
    const int n_slabs = (int)((c1 - c0 + kSlab - 1) / kSlab);
    for (int sl = 0; sl < n_slabs; ++sl) {
        uint16_t *buf = slab[sl & 1];
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int e = j * kMfmaThreads + threadIdx.x;
            *reinterpret_cast<uint4 *>(buf + (e / VPR) * LROW + (e % VPR) * 8) = pf[j];
        }
        __syncthreads();
        const int64_t base = c0 + (int64_t)sl * kSlab;
        if (sl + 1 < n_slabs) prefetch(base + kSlab);
#pragma unroll
        for (int bt = 0; bt < kSlab / 16; ++bt) {
            const int64_t b0 = base + bt * 16;
            if (b0 >= nb_wave) break;
            f32x4 acc[kRowTiles];
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) acc[rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            const uint16_t *brow = buf + (bt * 16 + col) * LROW + 8 * g;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 B = as_bf16x8(*reinterpret_cast<const uint4 *>(brow + 32 * ks));
#pragma unroll
                for (int rt = 0; rt < kRowTiles; ++rt)
                    acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rt][ks], B, acc[rt], 0, 0, 0);
            }
            // epilogue: ReLU, w-weighted head sum, masked store
            const int64_t b = b0 + col;
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) {
                const int row0 = wave * 64 + rt * 16 + 4 * g;   // first of the lane's 4 rows
                float r[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] = fmaxf(acc[rt][i], 0.0f);
                if constexpr (H >= 4) {
                    float sc = wv[rt][0] * r[0];
                    sc = __builtin_fmaf(wv[rt][1], r[1], sc);
                    sc = __builtin_fmaf(wv[rt][2], r[2], sc);
                    sc = __builtin_fmaf(wv[rt][3], r[3], sc);
                    if constexpr (H >= 8) sc = swap16_sum(sc);
                    if constexpr (H >= 16) sc = swap32_sum(sc);
                    const bool writer = (H == 4) || (H == 8 && (g & 1) == 0) || (H == 16 && g == 0);
                    const int64_t qq = qa + row0 / H;
                    if (writer && qq < nq && b < ((first_L + qq) >> log2r))
                        scores[(q0 + qq) * ld + b] = sc;
                } else if constexpr (H == 2) {
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        const float sc = __builtin_fmaf(wv[rt][2 * p + 1], r[2 * p + 1],
                                                        wv[rt][2 * p] * r[2 * p]);
                        const int64_t qq = qa + (row0 + 2 * p) / 2;
                        if (qq < nq && b < ((first_L + qq) >> log2r)) scores[(q0 + qq) * ld + b] = sc;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t qq = qa + row0 + i;
                        if (qq < nq && b < ((first_L + qq) >> log2r))
                            scores[(q0 + qq) * ld + b] = wv[rt][i] * r[i];
                    }
                }
            }
        }
    }
}

template <int H, int D>
hipError_t launch_hd(const qsa_indexer &ix, int ratio, const qsa_batch &b, float *scores,
                     int64_t ld, hipStream_t st) {
    constexpr int QW = 4 * (64 / H);
    const int log2r = __builtin_ctz((unsigned)ratio);
    const int64_t max_nb = b.max_kv_len >> log2r;
    const int64_t max_q = b.q_offsets ? b.max_q_per_seq : 1;
    if (max_nb == 0 || max_q == 0 || b.total_q == 0) return hipSuccess;
    const int64_t n_chunks = (max_nb + kChunk - 1) / kChunk;
    const int64_t q_groups = (max_q + QW - 1) / QW;
    if (n_chunks * q_groups > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 grid((unsigned)(n_chunks * q_groups), (unsigned)b.num_seqs);
    trace("score_mfma grid=%ux%u H=%d D=%d chunks=%lld", grid.x, grid.y, H, D, (long long)n_chunks);
    hipLaunchKernelGGL((score_mfma_kernel<H, D>), grid, dim3(kMfmaThreads), 0, st,
                       static_cast<const uint16_t *>(ix.q_idx), ix.w,
                       static_cast<const uint16_t *>(ix.kc), b.kv_offsets, b.blk_offsets,
                       b.q_offsets, log2r, (int)n_chunks, scores, ld);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const qsa_indexer &ix, int ratio, const qsa_batch &b, float *scores,
                    int64_t ld, hipStream_t st) {
    switch (ix.h_idx) {
        case 1: return launch_hd<1, D>(ix, ratio, b, scores, ld, st);
        case 2: return launch_hd<2, D>(ix, ratio, b, scores, ld, st);
        case 4: return launch_hd<4, D>(ix, ratio, b, scores, ld, st);
        case 8: return launch_hd<8, D>(ix, ratio, b, scores, ld, st);
        case 16: return launch_hd<16, D>(ix, ratio, b, scores, ld, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_score_mfma(const qsa_indexer &ix, int ratio, const qsa_batch &b, float *scores,
                             int64_t ld, hipStream_t st) {
    if (ix.q_dtype != QSA_BF16 || ix.kc_dtype != QSA_BF16) return hipErrorNotSupported;
    return ix.d_idx == 128 ? launch_d<128>(ix, ratio, b, scores, ld, st)
                           : launch_d<64>(ix, ratio, b, scores, ld, st);
}

}  // namespace qsa
