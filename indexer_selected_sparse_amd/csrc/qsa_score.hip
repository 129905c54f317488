// Indexer scores, canonical (bit-defined) form.
//
// s_b = sum_h w_h * ReLU(q_idx[h] . kc_b)  — "Agentic shootout" page, "PR 16
// review" section (a): a 4Q+1K indexer with a relu score over 4-token
// mean-pooled blocks; the single key head is the vLLM report's validator
// (indexer kv heads == 1, section (a)1).  For e4m3 keys the dot runs over the
// code values and is then multiplied by the block's fp32 scale.
//
// The score decides an integer (the selection), so it is evaluated in one
// fixed fp32 order that the CPU oracle follows too: for each head, a
// left-to-right sum over d of rounded products; ReLU; then a left-to-right
// sum over heads of rounded w_h * r_h.  A product of bf16 by bf16 (or by an
// e4m3 code) is exact in fp32, so a fused multiply-add there gives the same
// bits as multiply-then-add; fp32 inputs use a separate multiply and add.
//
// Decode is a GEMV per query and bound by HBM bandwidth (and, for e4m3 keys,
// by VALU issue): one lane owns one block and keeps its whole key row in
// registers (all row loads of the wave are in flight together, so the L1
// keeps each line for the burst); the query's H x D values are wave-uniform,
// read through the scalar unit.  Workgroup = 256 blocks of one query; blocks
// that are not yet visible to the query (b >= floor(L/ratio)) are skipped.
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {
namespace {

constexpr int kScoreThreads = 256;

template <typename KT, int D>
struct KRow;

// bf16 row: D/2 dwords
template <int D>
struct KRow<uint16_t, D> {
    uint32_t u[D / 2];
    __device__ __forceinline__ void load(const uint16_t *__restrict__ p) {
        const uint4 *v = reinterpret_cast<const uint4 *>(p);
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
            uint4 x = v[c];
            u[4 * c + 0] = x.x; u[4 * c + 1] = x.y; u[4 * c + 2] = x.z; u[4 * c + 3] = x.w;
        }
    }
    __device__ __forceinline__ float get(int d) const {
        return (d & 1) ? bf16hi(u[d >> 1]) : bf16lo(u[d >> 1]);
    }
};

// e4m3 codes: D/4 dwords
template <int D>
struct KRow<uint8_t, D> {
    uint32_t u[D / 4];
    __device__ __forceinline__ void load(const uint8_t *__restrict__ p) {
        const uint4 *v = reinterpret_cast<const uint4 *>(p);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            uint4 x = v[c];
            u[4 * c + 0] = x.x; u[4 * c + 1] = x.y; u[4 * c + 2] = x.z; u[4 * c + 3] = x.w;
        }
    }
};

// fp32 row
template <int D>
struct KRow<float, D> {
    float f[D];
    __device__ __forceinline__ void load(const float *__restrict__ p) {
        const float4 *v = reinterpret_cast<const float4 *>(p);
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
            float4 x = v[c];
            f[4 * c + 0] = x.x; f[4 * c + 1] = x.y; f[4 * c + 2] = x.z; f[4 * c + 3] = x.w;
        }
    }
    __device__ __forceinline__ float get(int d) const { return f[d]; }
};

// Wave-uniform query values for dims d0..d0+N-1 of one head, widened to fp32.
// Loaded as whole dwords from a uniform address, so they come through the
// scalar unit into SGPRs and feed the FMAs as scalar operands.
template <typename QT, int N>
__device__ __forceinline__ void load_q(const QT *__restrict__ q, int off, float (&v)[N]);
template <int N>
__device__ __forceinline__ void load_q(const uint16_t *__restrict__ q, int off, float (&v)[N]) {
    const uint32_t *p = reinterpret_cast<const uint32_t *>(q + off);
#pragma unroll
    for (int e = 0; e < N / 2; ++e) {
        const uint32_t u = p[e];
        v[2 * e] = bf16lo(u);
        v[2 * e + 1] = bf16hi(u);
    }
}
template <int N>
__device__ __forceinline__ void load_q(const float *__restrict__ q, int off, float (&v)[N]) {
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] = q[off + e];
}

// acc + q*k with the canonical rounding: fused only when q*k is exact.
template <bool EXACT>
__device__ __forceinline__ float mac(float acc, float q, float k) {
    if constexpr (EXACT) {
        return __builtin_fmaf(q, k, acc);
    } else {
        float p = q * k;
        return acc + p;
    }
}

template <typename QT, typename KT, int D, int H>
__global__ __launch_bounds__(kScoreThreads) void score_canonical_kernel(
    const QT *__restrict__ q_idx, const float *__restrict__ w, const KT *__restrict__ kc,
    const float *__restrict__ kc_scale, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ blk_off, const int64_t *__restrict__ q_off, int num_seqs,
    int log2r, float *__restrict__ scores, int64_t ld) {
    constexpr bool kExact = std::is_same<QT, uint16_t>::value && !std::is_same<KT, float>::value;
    constexpr bool kE4M3 = std::is_same<KT, uint8_t>::value;
    const int64_t i = blockIdx.x;
    const QueryPos qp = query_pos(kv_off, blk_off, q_off, num_seqs, i);
    const int64_t nb = qp.L >> log2r;
    const int64_t b = (int64_t)blockIdx.y * kScoreThreads + threadIdx.x;
    if ((int64_t)blockIdx.y * kScoreThreads >= nb) return;   // whole workgroup invisible
    const bool active = b < nb;
    const int64_t row = qp.blk_row0 + (active ? b : 0);

    const float sc = kE4M3 ? kc_scale[row] : 1.0f;
    const float *__restrict__ wi = w + i * (int64_t)H;
    float s = 0.0f;

    if constexpr (kExact) {
        // bf16 query x (bf16 | e4m3) key: every product is exact in fp32, so
        // the canonical step acc = fl(acc + q*k) is one IEEE fused
        // multiply-add.  The query pair (q_d, q_d+1) arrives as one dword in
        // an SGPR and is widened by two scalar ops (shift / mask); the
        // scheduling groups below interleave each scalar widening with its
        // FMA so that only a few widened values are live at a time (scalar
        // and vector ops of different waves issue in the same cycle).
        float kf[D];
        {
            KRow<KT, D> k;
            k.load(kc + row * D);
            if constexpr (kE4M3) {
#pragma unroll
                for (int c = 0; c < D / 4; ++c) {
                    const float2 a = e4m3x2_to_f32<false>(k.u[c]);
                    const float2 bb = e4m3x2_to_f32<true>(k.u[c]);
                    kf[4 * c] = a.x; kf[4 * c + 1] = a.y; kf[4 * c + 2] = bb.x; kf[4 * c + 3] = bb.y;
                }
            } else {
#pragma unroll
                for (int d = 0; d < D; ++d) kf[d] = k.get(d);
            }
        }
        const uint32_t *__restrict__ q32 =
            reinterpret_cast<const uint32_t *>(q_idx) + i * (int64_t)(H * D / 2);
#pragma unroll 1
        for (int h = 0; h < H; ++h) {
            float dot = 0.0f;
#pragma unroll
            for (int j = 0; j < D / 2; ++j) {
                const uint32_t u = q32[h * (D / 2) + j];
                dot = __builtin_fmaf(bf16lo(u), kf[2 * j], dot);
                dot = __builtin_fmaf(bf16hi(u), kf[2 * j + 1], dot);
            }
#pragma unroll
            for (int j = 0; j < D; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x004, 1, 0);   // one SALU op
                __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // one VALU op
            }
            if constexpr (kE4M3) dot = dot * sc;
            const float r = dot > 0.0f ? dot : 0.0f;
            const float t = wi[h] * r;
            s = s + t;
        }
    } else {
        // fp32 on either side: products are rounded, so multiply and add are
        // separate operations.  The key row is widened once to fp32.
        float kf[D];
        {
            KRow<KT, D> k;
            k.load(kc + row * D);
            if constexpr (kE4M3) {
#pragma unroll
                for (int c = 0; c < D / 4; ++c) {
                    const float2 lo = e4m3x2_to_f32<false>(k.u[c]);
                    const float2 hi = e4m3x2_to_f32<true>(k.u[c]);
                    kf[4 * c] = lo.x; kf[4 * c + 1] = lo.y; kf[4 * c + 2] = hi.x; kf[4 * c + 3] = hi.y;
                }
            } else {
#pragma unroll
                for (int d = 0; d < D; ++d) kf[d] = k.get(d);
            }
        }
        const QT *__restrict__ q = q_idx + i * (int64_t)(H * D);
#pragma unroll 1
        for (int h = 0; h < H; ++h) {
            float dot = 0.0f;
#pragma unroll
            for (int d0 = 0; d0 < D; d0 += 32) {
                float qv[32];
                load_q<32>(q, h * D + d0, qv);
#pragma unroll
                for (int e = 0; e < 32; ++e) dot = mac<false>(dot, qv[e], kf[d0 + e]);
            }
            if constexpr (kE4M3) dot = dot * sc;
            const float r = dot > 0.0f ? dot : 0.0f;
            const float t = wi[h] * r;
            s = s + t;
        }
    }
    if (active) scores[i * ld + b] = s;
}

template <typename QT, typename KT, int D>
hipError_t dispatch_h(const qsa_indexer &ix, int log2r, const qsa_batch &b, float *scores,
                      int64_t ld, dim3 grid, hipStream_t st) {
    const QT *q = static_cast<const QT *>(ix.q_idx);
    const KT *kc = static_cast<const KT *>(ix.kc);
    dim3 block(kScoreThreads);
#define QSA_SCORE_LAUNCH(HH)                                                                   \
    hipLaunchKernelGGL((score_canonical_kernel<QT, KT, D, HH>), grid, block, 0, st, q, ix.w, kc, \
                       ix.kc_scale, b.kv_offsets, b.blk_offsets, b.q_offsets, b.num_seqs, log2r,  \
                       scores, ld)
    switch (ix.h_idx) {
    case 1: QSA_SCORE_LAUNCH(1); break;
    case 2: QSA_SCORE_LAUNCH(2); break;
    case 4: QSA_SCORE_LAUNCH(4); break;
    case 8: QSA_SCORE_LAUNCH(8); break;
    default: QSA_SCORE_LAUNCH(16); break;
    }
#undef QSA_SCORE_LAUNCH
    return hipGetLastError();
}

template <typename QT, typename KT>
hipError_t dispatch_d(const qsa_indexer &ix, int log2r, const qsa_batch &b, float *scores,
                      int64_t ld, dim3 grid, hipStream_t st) {
    return ix.d_idx == 64 ? dispatch_h<QT, KT, 64>(ix, log2r, b, scores, ld, grid, st)
                          : dispatch_h<QT, KT, 128>(ix, log2r, b, scores, ld, grid, st);
}

}  // namespace

hipError_t launch_score_canonical(const qsa_indexer &ix, int ratio, const qsa_batch &b,
                                  float *scores, int64_t ld, hipStream_t st) {
    const int log2r = __builtin_ctz((unsigned)ratio);
    const int64_t max_nb = b.max_kv_len >> log2r;
    if (b.total_q == 0 || max_nb == 0) return hipSuccess;
    dim3 grid((unsigned)b.total_q, (unsigned)((max_nb + kScoreThreads - 1) / kScoreThreads));
    trace("score_canonical grid=(%u,%u) h_idx=%d d_idx=%d q=%d kc=%d", grid.x, grid.y, ix.h_idx,
          ix.d_idx, ix.q_dtype, ix.kc_dtype);
    const bool qb = ix.q_dtype == QSA_BF16;
    switch (ix.kc_dtype) {
    case QSA_F32:
        return qb ? dispatch_d<uint16_t, float>(ix, log2r, b, scores, ld, grid, st)
                  : dispatch_d<float, float>(ix, log2r, b, scores, ld, grid, st);
    case QSA_BF16:
        return qb ? dispatch_d<uint16_t, uint16_t>(ix, log2r, b, scores, ld, grid, st)
                  : dispatch_d<float, uint16_t>(ix, log2r, b, scores, ld, grid, st);
    default:
        return qb ? dispatch_d<uint16_t, uint8_t>(ix, log2r, b, scores, ld, grid, st)
                  : dispatch_d<float, uint8_t>(ix, log2r, b, scores, ld, grid, st);
    }
}

}  // namespace qsa
