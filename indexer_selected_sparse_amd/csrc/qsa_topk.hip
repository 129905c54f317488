// Block top-k per query, on device (no host round trip, so a decode step stays
// graph-capturable — the "Agentic shootout" page, "PR 16 review" sections
// (b)/(c), names host-side top-k that vetoes graphs as the v1 cliff).
//
// Semantics (vLLM report section (a)6: block top-k of budget/ratio groups,
// -1 padded; "PR 16 review" (a): top-512 + tail, inert below the bound):
//   nb <= K:  idx = 0, 1, ..., nb-1, -1, ...              (dense regime)
//   nb >  K:  the K blocks with the largest score, ties to the lower index,
//             written in ascending block order.
//
// Algorithm: one 1024-thread workgroup per query row.  Scores become
// order-preserving uint32 keys, cached in LDS (rows up to 32K blocks; longer
// rows are re-read from memory on each pass).
//  1. min/max of the row.
//  2. A histogram of 2048 bins LINEAR in the score between min and max.  The
//     bin map x -> floor((x - min) * 2048/(max - min)) is monotone, so every
//     block of a higher bin scores strictly higher than every block of a lower
//     bin, and the K-th largest score T lies in the bin tb where the count
//     from the top first reaches K.  (Linear bins spread the bulk of the row
//     over many bins, so the LDS atomics rarely collide.)
//  3. The blocks of bin tb (typically a few dozen) are copied out and an exact
//     MSB-first radix select on their keys yields T, how many keys equal T
//     exist and how many of them the selection still needs.  A degenerate
//     row (too many blocks in one bin, e.g. all scores equal) runs the same
//     exact radix select over the whole row instead.
//  4. An ordered pass emits every key > T and the first `need` keys == T by
//     index: elements are visited round-major (index order), and per
//     (round, wave) counts, scanned once, give each output position.
#include "qsa_device.hpp"
#include "qsa_lists.hpp"
#include "qsa_internal.hpp"

namespace qsa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kBins = 2048;                  // linear bins of step 2
constexpr int kDigitBits = 11;               // radix digits of step 3
constexpr int kMaxRounds = 128;              // => nb <= 131072 per row
constexpr int kMaskWords = kMaxRounds / 32;
constexpr int kCandMax = 2048;               // blocks of the threshold bin kept in LDS
constexpr int kLdsKeys = 32 * 1024;          // rows cached in LDS (128 KB)

static_assert(kMaxRounds * kTopkWaves <= kBins, "emit counts reuse the histogram");

__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

struct TopkShared {
    uint32_t hist[kBins];        // bin / digit counts; later per-(round, wave) counts
    uint32_t cand[kCandMax];     // keys of the threshold bin
    uint32_t wsum[kTopkWaves];   // per-wave partials of workgroup scans/reductions
    uint32_t wmin[kTopkWaves], wmax[kTopkWaves];
    uint32_t s0, s1, s2, s3;     // broadcast slots
};

// Workgroup exclusive prefix sum (thread order); returns (excl, total).
__device__ __forceinline__ uint32_t wg_scan(uint32_t v, TopkShared &S, uint32_t &total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_scan(v);
    if (lane == kWave - 1) S.wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
        const uint32_t x = S.wsum[w];
        before += (w < wave) ? x : 0u;
        tot += x;
    }
    __syncthreads();
    total = tot;
    return before + incl - v;
}

// Workgroup min and max of uint keys.
__device__ __forceinline__ void wg_minmax(uint32_t &mn, uint32_t &mx, TopkShared &S) {
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) { S.wmin[wave] = mn; S.wmax[wave] = mx; }
    __syncthreads();
    mn = S.wmin[0];
    mx = S.wmax[0];
#pragma unroll
    for (int w = 1; w < kTopkWaves; ++w) { mn = min(mn, S.wmin[w]); mx = max(mx, S.wmax[w]); }
    __syncthreads();
}

// Find the bin where the count from the top first reaches `need` among
// nbins (<= 2048) bins of S.hist: each thread owns two adjacent bins
// (descending); a workgroup scan gives the count above them.  Returns the
// bin; `above` = count in higher bins.
__device__ __forceinline__ int find_bin(int nbins, uint32_t need, TopkShared &S, uint32_t &above) {
    const int hi = nbins - 1 - 2 * (int)threadIdx.x;
    const uint32_t h0 = hi >= 0 ? S.hist[hi] : 0u;
    const uint32_t h1 = hi >= 1 ? S.hist[hi - 1] : 0u;
    uint32_t tot;
    const uint32_t ex = wg_scan(h0 + h1, S, tot);
    if (ex < need && need <= ex + h0 + h1) {
        if (ex + h0 >= need) { S.s0 = (uint32_t)hi; S.s1 = ex; }
        else { S.s0 = (uint32_t)(hi - 1); S.s1 = ex + h0; }
    }
    __syncthreads();
    above = S.s1;
    const int bin = (int)S.s0;
    __syncthreads();
    return bin;
}

// Exact `need`-th largest key among keys(b), b < n (MSB-first radix, digits
// of 11 bits starting below the bits shared by kmin and kmax).  Returns T;
// need_eq = keys equal to T still to take; total_eq = keys equal to T.
template <typename KeyF>
__device__ uint32_t radix_select(const KeyF &key, int64_t n, uint32_t need, uint32_t kmin,
                                 uint32_t kmax, TopkShared &S, uint32_t &need_eq,
                                 uint32_t &total_eq) {
    const uint32_t diff = kmin ^ kmax;
    if (diff == 0) {
        need_eq = need;
        total_eq = (uint32_t)n;
        return kmin;
    }
    const int hi_bit = 31 - __builtin_clz(diff);
    uint32_t prefix = hi_bit == 31 ? 0u : (kmax & ~((2u << hi_bit) - 1u));
    int lo_bit = hi_bit + 1;                     // bits >= lo_bit are fixed
    total_eq = 0;
    while (lo_bit > 0) {
        const int width = lo_bit >= kDigitBits ? kDigitBits : lo_bit;
        const int shift = lo_bit - width;
        const uint32_t mask_hi = lo_bit >= 32 ? 0u : ~((1u << lo_bit) - 1u);
        for (int t = threadIdx.x; t < kBins; t += kTopkThreads) S.hist[t] = 0;
        __syncthreads();
#pragma unroll 4
        for (int64_t b = threadIdx.x; b < n; b += kTopkThreads) {
            const uint32_t k = key(b);
            if ((k & mask_hi) == prefix) atomicAdd(&S.hist[(k >> shift) & ((1u << width) - 1u)], 1u);
        }
        __syncthreads();
        uint32_t above;
        const int d = find_bin(1 << width, need, S, above);
        total_eq = S.hist[d];
        prefix |= (uint32_t)d << shift;
        need -= above;
        lo_bit = shift;
        __syncthreads();
    }
    need_eq = need;
    return prefix;
}

// Replace per-(round, wave) counts cnt[0..n) by their exclusive prefix sums.
__device__ __forceinline__ void scan_counts(uint32_t *cnt, int n, TopkShared &S) {
    uint32_t tot;
    const int t0 = 2 * (int)threadIdx.x;
    const uint32_t c0 = t0 < n ? cnt[t0] : 0u, c1 = t0 + 1 < n ? cnt[t0 + 1] : 0u;
    const uint32_t ex = wg_scan(c0 + c1, S, tot);
    if (t0 < n) cnt[t0] = ex;
    if (t0 + 1 < n) cnt[t0 + 1] = ex + c0;
    __syncthreads();
}

// Ordered output: every key > T, then the first need_eq keys == T by index.
template <typename KeyF>
__device__ void emit_selection(const KeyF &key, int64_t nb, uint32_t T, uint32_t need_eq,
                               uint32_t total_eq, int32_t *__restrict__ out, int K, TopkShared &S) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int rounds = (int)((nb + kTopkThreads - 1) / kTopkThreads);
    const int ncnt = rounds * kTopkWaves;
    const bool all_eq = need_eq >= total_eq;
    uint32_t *cnt = S.hist;
    // selected-element masks, one bit per round
    uint32_t selm[kMaskWords];
#pragma unroll
    for (int g = 0; g < kMaskWords; ++g) {
        selm[g] = 0;
        if (g * 32 >= rounds) continue;
#pragma unroll
        for (int u = 0; u < 32; ++u) {
            const int j = g * 32 + u;
            const int64_t b = (int64_t)j * kTopkThreads + threadIdx.x;
            if (j < rounds && b < nb && key(b) >= T) selm[g] |= 1u << u;
        }
    }
    if (!all_eq) {
        // Ties at T: rank them in index order and keep the first need_eq.
#pragma unroll
        for (int g = 0; g < kMaskWords; ++g) {
            if (g * 32 >= rounds) continue;
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                const int j = g * 32 + u;
                const int64_t b = (int64_t)j * kTopkThreads + threadIdx.x;
                const bool eq = j < rounds && b < nb && key(b) == T;
                const uint64_t m = __ballot(eq);
                if (lane == 0 && j < rounds) cnt[j * kTopkWaves + wave] = (uint32_t)__builtin_popcountll(m);
            }
        }
        __syncthreads();
        scan_counts(cnt, ncnt, S);
#pragma unroll
        for (int g = 0; g < kMaskWords; ++g) {
            if (g * 32 >= rounds) continue;
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                const int j = g * 32 + u;
                const int64_t b = (int64_t)j * kTopkThreads + threadIdx.x;
                const bool eq = j < rounds && b < nb && key(b) == T;
                const uint64_t m = __ballot(eq);
                if (eq) {
                    const uint32_t rank = cnt[j * kTopkWaves + wave] + lanes_below(m);
                    if (rank >= need_eq) selm[g] &= ~(1u << u);
                }
            }
        }
        __syncthreads();
    }
    // per-(round, wave) counts of selected elements -> output offsets
#pragma unroll
    for (int g = 0; g < kMaskWords; ++g) {
        if (g * 32 >= rounds) continue;
#pragma unroll
        for (int u = 0; u < 32; ++u) {
            const int j = g * 32 + u;
            const uint64_t m = __ballot((selm[g] >> u) & 1u);
            if (lane == 0 && j < rounds) cnt[j * kTopkWaves + wave] = (uint32_t)__builtin_popcountll(m);
        }
    }
    __syncthreads();
    scan_counts(cnt, ncnt, S);
#pragma unroll
    for (int g = 0; g < kMaskWords; ++g) {
        if (g * 32 >= rounds) continue;
#pragma unroll
        for (int u = 0; u < 32; ++u) {
            const int j = g * 32 + u;
            const bool sel = (selm[g] >> u) & 1u;
            const uint64_t m = __ballot(sel);
            if (sel) {
                const uint32_t pos = cnt[j * kTopkWaves + wave] + lanes_below(m);
                if (pos < (uint32_t)K) out[pos] = (int32_t)((int64_t)j * kTopkThreads + threadIdx.x);
            }
        }
    }
}

struct GlobalKey {
    const float *__restrict__ row;
    __device__ __forceinline__ uint32_t operator()(int64_t b) const { return order_key(row[b]); }
};

struct LdsKey {
    const uint32_t *keys;
    __device__ __forceinline__ uint32_t operator()(int64_t b) const { return keys[b]; }
};

// The K-th largest key T of the row, how many keys equal T the selection
// still needs (need_eq) and how many there are (total_eq).
template <typename KeyF>
__device__ uint32_t find_threshold(const KeyF &key, int64_t nb, int K, uint32_t kmin, uint32_t kmax,
                                   TopkShared &S, uint32_t &need_eq, uint32_t &total_eq) {
    const float vmin = key_value(kmin), vmax = key_value(kmax);
    const float scale = (float)kBins / (vmax - vmin);
    if (kmin == kmax || !(scale < 3.0e38f)) {
        // flat (or numerically flat) row: exact radix over the row
        return radix_select(key, nb, (uint32_t)K, kmin, kmax, S, need_eq, total_eq);
    }
    for (int t = threadIdx.x; t < kBins; t += kTopkThreads) S.hist[t] = 0;
    if (threadIdx.x == 0) S.s2 = 0;
    __syncthreads();
#pragma unroll 4
    for (int64_t b = threadIdx.x; b < nb; b += kTopkThreads) {
        const float x = key_value(key(b));
        const int bin = min(kBins - 1, (int)((x - vmin) * scale));
        atomicAdd(&S.hist[bin], 1u);
    }
    __syncthreads();
    uint32_t above;
    const int tb = find_bin(kBins, (uint32_t)K, S, above);
    const uint32_t m = S.hist[tb];
    const uint32_t need = (uint32_t)K - above;
    __syncthreads();
    if (m > (uint32_t)kCandMax) return radix_select(key, nb, (uint32_t)K, kmin, kmax, S, need_eq, total_eq);
    // copy the threshold bin's keys, tracking their range
    uint32_t cmin = 0xffffffffu, cmax = 0u;
#pragma unroll 4
    for (int64_t b = threadIdx.x; b < nb; b += kTopkThreads) {
        const uint32_t k = key(b);
        const int bin = min(kBins - 1, (int)((key_value(k) - vmin) * scale));
        if (bin == tb) {
            S.cand[atomicAdd(&S.s2, 1u)] = k;
            cmin = min(cmin, k);
            cmax = max(cmax, k);
        }
    }
    wg_minmax(cmin, cmax, S);      // its barriers publish S.cand
    return radix_select(LdsKey{S.cand}, (int64_t)m, need, cmin, cmax, S, need_eq, total_eq);
}

template <typename KeyF>
__device__ void select_row(const KeyF &key, int64_t nb, int K, uint32_t kmin, uint32_t kmax,
                           int32_t *__restrict__ out, TopkShared &S) {
    uint32_t need_eq, total_eq;
    const uint32_t T = find_threshold(key, nb, K, kmin, kmax, S, need_eq, total_eq);
    emit_selection(key, nb, T, need_eq, total_eq, out, K, S);
}

// Row -> order keys in LDS (rows of at most kLdsKeys blocks) and their range.
// One streaming pass: every load of the thread (at most 32) is issued before
// the first is consumed, so the row costs one memory latency.
__device__ __forceinline__ void cache_row(const float *__restrict__ row, int64_t nb,
                                          uint32_t *lds_keys, uint32_t &kmin, uint32_t &kmax,
                                          TopkShared &S) {
    constexpr int kR = kLdsKeys / kTopkThreads;
    uint32_t kk[kR];
#pragma unroll
    for (int u = 0; u < kR; ++u) {
        const int64_t b = (int64_t)u * kTopkThreads + threadIdx.x;
        kk[u] = b < nb ? order_key(row[b]) : 0u;
    }
    kmin = 0xffffffffu;
    kmax = 0u;
#pragma unroll
    for (int u = 0; u < kR; ++u) {
        const int64_t b = (int64_t)u * kTopkThreads + threadIdx.x;
        if (b < nb) {
            lds_keys[b] = kk[u];
            kmin = min(kmin, kk[u]);
            kmax = max(kmax, kk[u]);
        }
    }
    wg_minmax(kmin, kmax, S);     // its barrier also publishes lds_keys
}

template <bool CACHED>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float *__restrict__ scores, int64_t ld, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ q_off, int num_seqs, int log2r, int K, int32_t *__restrict__ idx, int ldi) {
    __shared__ TopkShared S;
    extern __shared__ uint32_t lds_keys[];
    const int64_t i = blockIdx.x;
    const QueryPos qp = query_pos(kv_off, nullptr, q_off, num_seqs, i);
    const int64_t nb = qp.L >> log2r;
    int32_t *out = idx + i * (int64_t)ldi;
    if (nb <= K) {
        for (int t = threadIdx.x; t < K; t += kTopkThreads) out[t] = (t < nb) ? t : -1;
        return;
    }
    const float *__restrict__ row = scores + i * ld;
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    if constexpr (CACHED) {
        cache_row(row, nb, lds_keys, kmin, kmax, S);
        select_row(LdsKey{lds_keys}, nb, K, kmin, kmax, out, S);
    } else {
        const GlobalKey key{row};
#pragma unroll 4
        for (int64_t b = threadIdx.x; b < nb; b += kTopkThreads) {
            const uint32_t k = key(b);
            kmin = min(kmin, k);
            kmax = max(kmax, k);
        }
        wg_minmax(kmin, kmax, S);
        select_row(key, nb, K, kmin, kmax, out, S);
    }
}

// ------------------------------------------------------------------------
// Certified selection from approximate (matrix-core) scores.
//
// The scores a_b come from a summation order other than the canonical one.
// Both a_b and the canonical c_b are fp32 evaluations of
//   S_b = sum_h w_h ReLU(q_h . k_b)
// whose D-term dots have bf16*bf16 (or exactly widened) products.  With unit
// roundoff u = 2^-23 (valid for round-to-nearest and for truncation) and
// gamma_n = n u / (1 - n u), the classic summation bound (Higham, Accuracy and
// Stability of Numerical Algorithms, section 4.2) gives, for any order,
// |dot - q.k| <= gamma_(D+1) sum_d |q_d k_d| <= gamma_(D+1) |q| |k| (Cauchy-
// Schwarz; the +1 covers an e4m3 scale multiply).  ReLU is 1-Lipschitz, and
// the head sum of H rounded products adds gamma_(H+1) sum_h |w_h| r_h.  Hence
//   |a_b - S_b|, |c_b - S_b| <= (gamma_(D+1) + gamma_(H+1)(1 + gamma_(D+1))) P_b
//   with P_b = sum_h |w_h| |q_h| |k_b|,
// and |a_b - c_b| <= 2 (D + H + 2) u P_b (1 + O(nu)).  The kernel uses
//   E = 4 (D + H + 2) u * F * n_max * (1 + 2^-10) + (1 + sum_h |w_h|) 2^-100,
//   F = sum_h |w_h| |q_h|,  n_max = max_b |k_b| over the sequence,
// i.e. twice the bound, so that the fp32 evaluation of F, n_max and t +- 2E
// below stays on the safe side (their relative errors are O((D+H)u), far
// below the slack), and the absolute term covers products or head terms
// that underflow (flushed or subnormal).
//
// With t the K-th largest a, a block with a_b > t + 2E is certainly among
// the canonical top K (at most K-1 blocks have a > t, and every block that
// could beat it has c > t + E), and a block with a_b < t - 2E is certainly
// out (at least K blocks have c >= t - E > c_b).  The remaining band blocks
// (typically tens) are recomputed in the canonical order; the free slots go
// to the band's best by (c desc, index asc).  The result is the canonical
// selection, bit for bit.  A band larger than the candidate buffer (flat or
// adversarial rows) recomputes the whole row canonically instead.

constexpr int kNormThreads = 256;
constexpr int kMaxHD = 16 * 128;

// Max over chunks of kNormThreads blocks of |kc_b| (fp32; e4m3 codes times
// the block scale): part[s * n_chunks + chunk].  Every slot is written.
__global__ __launch_bounds__(kNormThreads) void block_norm_kernel(
    const void *__restrict__ kc, int kc_dtype, const float *__restrict__ kc_scale, int D,
    const int64_t *__restrict__ blk_off, int n_chunks, float *__restrict__ part) {
    __shared__ float wmax[kNormThreads / kWave];
    const int s = blockIdx.y;
    const int64_t kb0 = blk_off[s];
    const int64_t nblk = blk_off[s + 1] - kb0;
    const int64_t b = (int64_t)blockIdx.x * kNormThreads + threadIdx.x;
    float n = 0.0f;
    if (b < nblk) {
        float ss = 0.0f;
        const int64_t row = kb0 + b;
        if (kc_dtype == QSA_F32) {
            const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(kc) + row * D);
            for (int c = 0; c < D / 4; ++c) {
                const float4 x = p[c];
                ss = ss + x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
            }
        } else if (kc_dtype == QSA_BF16) {
            const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(kc) + row * D);
            for (int c = 0; c < D / 8; ++c) {
                const uint4 x = p[c];
                const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float lo = bf16lo(u[j]), hi = bf16hi(u[j]);
                    ss = ss + lo * lo + hi * hi;
                }
            }
        } else {
            const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(kc) + row * D);
            for (int c = 0; c < D / 16; ++c) {
                const uint4 x = p[c];
                const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float2 lo = e4m3x2_to_f32<false>(u[j]), hi = e4m3x2_to_f32<true>(u[j]);
                    ss = ss + lo.x * lo.x + lo.y * lo.y + hi.x * hi.x + hi.y * hi.y;
                }
            }
        }
        n = __builtin_sqrtf(ss);
        if (kc_dtype == QSA_FP8_E4M3) n = n * kc_scale[row];
    }
    n = wave_max(n);
    if ((threadIdx.x & (kWave - 1)) == 0) wmax[threadIdx.x / kWave] = n;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = wmax[0];
        for (int w = 1; w < kNormThreads / kWave; ++w) m = fmaxf(m, wmax[w]);
        part[(int64_t)s * n_chunks + blockIdx.x] = m;
    }
}

struct CertIndexer {
    const void *q_idx;
    const float *w;
    const void *kc;
    const float *kc_scale;
    int q_dtype, kc_dtype, H, D;
};

// Canonical dot of query head row qh (fp32, LDS) with key row `row`:
// +0, then d ascending, rounded product then rounded sum; e4m3 keys are
// code values times the block scale afterwards.
__device__ float canonical_dot(const CertIndexer &ix, const float *qh, int64_t row) {
    const int D = ix.D;
    float dot = 0.0f;
    if (ix.kc_dtype == QSA_F32) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(ix.kc) + row * D);
        for (int c = 0; c < D / 4; ++c) {
            const float4 x = p[c];
            dot = dot + qh[4 * c + 0] * x.x;
            dot = dot + qh[4 * c + 1] * x.y;
            dot = dot + qh[4 * c + 2] * x.z;
            dot = dot + qh[4 * c + 3] * x.w;
        }
    } else if (ix.kc_dtype == QSA_BF16) {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(ix.kc) + row * D);
        for (int c = 0; c < D / 8; ++c) {
            const uint4 x = p[c];
            const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dot = dot + qh[8 * c + 2 * j] * bf16lo(u[j]);
                dot = dot + qh[8 * c + 2 * j + 1] * bf16hi(u[j]);
            }
        }
    } else {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(ix.kc) + row * D);
        for (int c = 0; c < D / 16; ++c) {
            const uint4 x = p[c];
            const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float2 lo = e4m3x2_to_f32<false>(u[j]), hi = e4m3x2_to_f32<true>(u[j]);
                dot = dot + qh[16 * c + 4 * j + 0] * lo.x;
                dot = dot + qh[16 * c + 4 * j + 1] * lo.y;
                dot = dot + qh[16 * c + 4 * j + 2] * hi.x;
                dot = dot + qh[16 * c + 4 * j + 3] * hi.y;
            }
        }
        dot = dot * ix.kc_scale[row];
    }
    return dot;
}

struct CertShared {
    float q[kMaxHD + 16];        // query rows, head stride D+1
    float w[16];
    float part[kMaxHD / kWave];
    float F, wabs, nmax;
};

struct BandKey {
    const uint32_t *cand;
    const uint32_t *keys;
    __device__ __forceinline__ uint32_t operator()(int64_t j) const { return keys[cand[j]]; }
};

// At most 64 VGPRs (8 waves per SIMD), so that two rows' workgroups share a
// CU as with the plain selection; at 90 VGPRs one row held a CU alone and
// a prefill batch took twice as long.
__global__ __launch_bounds__(kTopkThreads, 8) void topk_cert_kernel(
    const float *__restrict__ scores, int64_t ld, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ blk_off, const int64_t *__restrict__ q_off, int num_seqs,
    int log2r, int K, int32_t *__restrict__ idx, int ldi, CertIndexer ix,
    const float *__restrict__ norm_part, int n_norm_chunks) {
    __shared__ TopkShared S;
    __shared__ CertShared C;
    extern __shared__ uint32_t lds_keys[];
    const int64_t i = blockIdx.x;
    const QueryPos qp = query_pos(kv_off, blk_off, q_off, num_seqs, i);
    const int64_t nb = qp.L >> log2r;
    int32_t *out = idx + i * (int64_t)ldi;
    if (nb <= K) {
        for (int t = threadIdx.x; t < K; t += kTopkThreads) out[t] = (t < nb) ? t : -1;
        return;
    }
    const int H = ix.H, D = ix.D, HD = H * D;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    // query rows to LDS (fp32, exact widening) and |q|^2 partials per group
    // of 64 consecutive elements (a group never straddles heads: D is a
    // multiple of 64)
    for (int e0 = 0; e0 < HD; e0 += kTopkThreads) {
        const int e = e0 + (int)threadIdx.x;
        float x = 0.0f;
        if (e < HD) {
            x = ix.q_dtype == QSA_F32 ? static_cast<const float *>(ix.q_idx)[i * HD + e]
                                      : bf16_to_f32(static_cast<const uint16_t *>(ix.q_idx)[i * HD + e]);
            const int h = e / D, d = e - h * D;
            C.q[h * (D + 1) + d] = x;
        }
        const float sq = wave_sum(x * x);
        if (lane == 0) C.part[e / kWave] = sq;
    }
    if ((int)threadIdx.x < H) C.w[threadIdx.x] = ix.w[i * H + threadIdx.x];
    // n_max over the sequence's chunks (every block of the sequence bounds
    // the visible ones)
    float nm = 0.0f;
    for (int c = threadIdx.x; c < n_norm_chunks; c += kTopkThreads)
        nm = fmaxf(nm, norm_part[(int64_t)qp.seq * n_norm_chunks + c]);
    nm = wave_max(nm);
    const float *__restrict__ row = scores + i * ld;
    uint32_t kmin, kmax;
    cache_row(row, nb, lds_keys, kmin, kmax, S);     // barriers publish C.part too
    if (lane == 0) S.wmax[wave] = __float_as_uint(nm);
    __syncthreads();
    if (threadIdx.x == 0) {
        float F = 0.0f, wabs = 0.0f;
        const int wpd = D / kWave;
        for (int h = 0; h < H; ++h) {
            float ss = 0.0f;
            for (int j = 0; j < wpd; ++j) ss = ss + C.part[h * wpd + j];
            F = F + fabsf(C.w[h]) * __builtin_sqrtf(ss);
            wabs = wabs + fabsf(C.w[h]);
        }
        float n = 0.0f;
        for (int w = 0; w < kTopkWaves; ++w) n = fmaxf(n, __uint_as_float(S.wmax[w]));
        C.F = F;
        C.wabs = wabs;
        C.nmax = n;
        S.s2 = 0;
        S.s3 = 0;
    }
    __syncthreads();
    const float c_rel = 4.0f * (float)(D + H + 2) * 0x1p-23f * (1.0f + 0x1p-10f);
    const float E = c_rel * C.F * C.nmax + (1.0f + C.wabs) * 0x1p-100f;

    uint32_t need_eq, total_eq;
    bool overflow = !(E <= 1.0e30f);
    if (!overflow) {
        // t = K-th largest approximate score; classify against t -+ 2E
        const uint32_t T = find_threshold(LdsKey{lds_keys}, nb, K, kmin, kmax, S, need_eq, total_eq);
        const float t = key_value(T);
        const uint32_t k_in = order_key(t + 2.0f * E), k_out = order_key(t - 2.0f * E);
        if (threadIdx.x == 0) { S.s2 = 0; S.s3 = 0; }
        __syncthreads();
        uint32_t n_in = 0;
        for (int64_t b = threadIdx.x; b < nb; b += kTopkThreads) {
            const uint32_t k = lds_keys[b];
            if (k > k_in) {
                lds_keys[b] = 0xffffffffu;          // certainly selected
                ++n_in;
            } else if (k < k_out) {
                lds_keys[b] = 0u;                   // certainly not
            } else {
                const uint32_t pos = atomicAdd(&S.s2, 1u);
                if (pos < (uint32_t)kCandMax) S.cand[pos] = (uint32_t)b;
            }
        }
        atomicAdd(&S.s3, n_in);
        __syncthreads();
        overflow = S.s2 > (uint32_t)kCandMax;
    }
    const uint32_t n_band = S.s2, n_in = S.s3;
    const int64_t items = overflow ? nb : (int64_t)n_band;
    // canonical recompute: item j, head h on thread (j % per) * H + h
    const int per = kTopkThreads / H;
    float *dots = reinterpret_cast<float *>(S.hist);
    for (int64_t j0 = 0; j0 < items; j0 += per) {
        __syncthreads();
        const int64_t j = j0 + threadIdx.x / H;
        const int h = threadIdx.x % H;
        if ((int)threadIdx.x < per * H && j < items) {
            const int64_t b = overflow ? j : (int64_t)S.cand[j];
            dots[threadIdx.x] = canonical_dot(ix, C.q + h * (D + 1), qp.blk_row0 + b);
        }
        __syncthreads();
        if ((int)threadIdx.x < per && j0 + threadIdx.x < items) {
            const int64_t jj = j0 + threadIdx.x;
            const int64_t b = overflow ? jj : (int64_t)S.cand[jj];
            float sc = 0.0f;
            for (int hh = 0; hh < H; ++hh) {
                const float dt = dots[threadIdx.x * H + hh];
                const float r = dt > 0.0f ? dt : 0.0f;
                sc = sc + C.w[hh] * r;
            }
            lds_keys[b] = order_key(sc);
        }
    }
    __syncthreads();
    if (overflow) {
        // every key is canonical now: the plain selection
        kmin = 0xffffffffu;
        kmax = 0u;
        for (int64_t b = threadIdx.x; b < nb; b += kTopkThreads) {
            kmin = min(kmin, lds_keys[b]);
            kmax = max(kmax, lds_keys[b]);
        }
        wg_minmax(kmin, kmax, S);
        select_row(LdsKey{lds_keys}, nb, K, kmin, kmax, out, S);
        return;
    }
    // free slots K - n_in go to the band's best by (canonical key, index)
    const BandKey bk{S.cand, lds_keys};
    uint32_t bmin = 0xffffffffu, bmax = 0u;
    for (int64_t j = threadIdx.x; j < (int64_t)n_band; j += kTopkThreads) {
        bmin = min(bmin, bk(j));
        bmax = max(bmax, bk(j));
    }
    wg_minmax(bmin, bmax, S);
    const uint32_t T = radix_select(bk, (int64_t)n_band, (uint32_t)K - n_in, bmin, bmax, S, need_eq,
                                    total_eq);
    // certainly-in keys are all-ones (> any finite key), certainly-out keys
    // are 0 (< any finite key): only band keys can equal T
    emit_selection(LdsKey{lds_keys}, nb, T, need_eq, total_eq, out, K, S);
}

// ------------------------------------------------------------------------
// Few-row batches (decode): each row is spread over many CUs.
//
// A single workgroup per row is bounded by what one CU can pull from the
// memory hierarchy (a 32K-block row of scores alone is 128 KB).  For batches
// of at most kMultiMaxRows rows the selection runs in two kernels, each
// spread over the GPU, with the same exact result:
//  1. classify (row x 2048-block chunks).  Every workgroup of a row takes the
//     same deterministic sample of the row (64 segments of 32 consecutive
//     blocks spread evenly; the whole row when it has at most 2048 blocks),
//     histograms it over 2048 bins linear in the score between the sample's
//     min and max, and picks two bins: jH, above which about (k - margin)
//     sample scores lie, and jL, above which about (k + margin) lie, k being
//     the rank the K-th largest score would have in the sample.  The bin map
//     is monotone in the score, so "bin > jH" (in), "jL <= bin <= jH"
//     (candidate) and "bin < jL" (out) split the scores in order.  Each
//     workgroup writes the in and candidate blocks of its chunk to its own
//     region of the workspace (no atomics, nothing to clear between calls).
//     Dense rows (nb <= K) get their identity selection from chunk 0.
//  2. finish (one workgroup per row).  If #in <= K <= #in + #candidates and
//     nothing overflowed, the K - #in best candidates by (score desc, index
//     asc) are found with the exact radix select; the selected blocks are
//     marked in an LDS bitmap and written in ascending order by a scan.
//     Otherwise (adversarial or heavily tied rows) the row is selected by the
//     exact single-workgroup method.  Either way the output is exact.
constexpr int kMultiMaxRows = 256;
constexpr int kSample = 2048;
constexpr int kSegLen = 32;
constexpr int kClassifyChunk = 2048;
constexpr int kClassifyThreads = 256;
constexpr int kChunkCandCap = 1024;        // candidates one chunk may record
constexpr int kMultiCandMax = 3072;        // candidates a row may have in total
constexpr int kBitmapWordsMax = 131072 / 32;
constexpr int kMaxChunks = 131072 / kClassifyChunk;

__host__ __device__ constexpr size_t chunk_region_bytes(int K) {
    return 16 + (size_t)K * 4 + (size_t)kChunkCandCap * 8;
}

// Region of chunk c of row i: counts {n_in, n_cand}, in[K], cand_key[cap],
// cand_idx[cap].
struct ChunkWs {
    uint32_t *cnt;
    uint32_t *in_idx;
    uint32_t *cand_key;
    uint32_t *cand_idx;
};

__device__ __forceinline__ ChunkWs chunk_ws(const void *ws, int64_t i, int c, int nchunks, int K) {
    uint8_t *base = const_cast<uint8_t *>(static_cast<const uint8_t *>(ws)) +
                    ((size_t)i * nchunks + c) * chunk_region_bytes(K);
    ChunkWs r;
    r.cnt = reinterpret_cast<uint32_t *>(base);
    r.in_idx = reinterpret_cast<uint32_t *>(base + 16);
    r.cand_key = r.in_idx + K;
    r.cand_idx = r.cand_key + kChunkCandCap;
    return r;
}

__global__ __launch_bounds__(kClassifyThreads) void topk_classify_kernel(
    const float *__restrict__ scores, int64_t ld, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ q_off, int num_seqs, int log2r, int K, int nchunks,
    int32_t *__restrict__ idx, int ldi, void *__restrict__ ws) {
    __shared__ uint32_t hist[kSample];
    __shared__ uint32_t red[kClassifyThreads / kWave];
    __shared__ float fred[2][kClassifyThreads / kWave];
    __shared__ int sel[2];
    const int64_t i = blockIdx.y;
    const int c = blockIdx.x;
    const QueryPos qp = query_pos(kv_off, nullptr, q_off, num_seqs, i);
    const int64_t nb = qp.L >> log2r;
    if (nb <= K) {
        if (c == 0) {
            int32_t *out = idx + i * (int64_t)ldi;
            for (int t = threadIdx.x; t < K; t += kClassifyThreads) out[t] = (t < nb) ? t : -1;
        }
        return;
    }
    const int64_t b0 = (int64_t)c * kClassifyChunk;
    if (b0 >= nb) return;                          // uniform over the workgroup
    const float *__restrict__ row = scores + i * ld;
    constexpr int kPer = kClassifyChunk / kClassifyThreads;   // 8
    // this chunk's scores and this thread's part of the sample, loaded together
    float x[kPer], smp[kPer];
    const bool whole = nb <= kSample;
    const int ns = whole ? (int)nb : kSample;
    constexpr int kSegs = kSample / kSegLen;
    const int64_t seg_step = whole ? 0 : (nb - kSegLen) / (kSegs - 1);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int64_t b = b0 + u * kClassifyThreads + threadIdx.x;
        x[u] = b < nb ? row[b] : 0.0f;
        const int t = u * kClassifyThreads + threadIdx.x;
        const int64_t sb = whole ? t : (t / kSegLen) * seg_step + (t % kSegLen);
        smp[u] = t < ns ? row[sb] : 0.0f;
    }
    for (int t = threadIdx.x; t < kSample; t += kClassifyThreads) hist[t] = 0;
    // sample range
    float vmin = INFINITY, vmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        if (u * kClassifyThreads + (int)threadIdx.x < ns) {
            vmin = fminf(vmin, smp[u]);
            vmax = fmaxf(vmax, smp[u]);
        }
    }
    vmin = wave_min_f32(vmin);
    vmax = wave_max_f32(vmax);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    if (lane == 0) { fred[0][wave] = vmin; fred[1][wave] = vmax; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kClassifyThreads / kWave; ++w) {
        vmin = fminf(vmin, fred[0][w]);
        vmax = fmaxf(vmax, fred[1][w]);
    }
    // monotone bin map: -1 below the sample range, 2047 at and above its top
    const float span = vmax - vmin;
    const float scale = span > 0.0f ? (float)kSample / span : 0.0f;
    auto bin_of = [&](float v) -> int {
        if (!(span > 0.0f)) return v < vmin ? -1 : (v > vmin ? kSample - 1 : 0);
        const float t = (v - vmin) * scale;
        return t < 0.0f ? -1 : (t >= (float)(kSample - 1) ? kSample - 1 : (int)t);
    };
#pragma unroll
    for (int u = 0; u < kPer; ++u)
        if (u * kClassifyThreads + (int)threadIdx.x < ns) atomicAdd(&hist[bin_of(smp[u])], 1u);
    __syncthreads();
    // sample ranks of the bracket
    uint32_t rank_hi, rank_lo;
    if (whole) {
        rank_hi = rank_lo = (uint32_t)K;
    } else {
        const float frac = (float)K / (float)nb;
        const float ks = frac * (float)ns;
        const float sd = __builtin_sqrtf(ks * (1.0f - frac));
        const int margin = (int)(4.0f * sd) + 8;
        const int kr = (int)__builtin_ceilf(ks);
        rank_hi = (uint32_t)(kr - margin < 1 ? 1 : kr - margin);
        rank_lo = (uint32_t)(kr + margin > ns ? ns : kr + margin);
    }
    // descending cumulative counts: thread t owns bins 8t..8t+7 from the top
    constexpr int kBpt = kSample / kClassifyThreads;
    uint32_t own = 0;
    const int top = kSample - 1 - (int)threadIdx.x * kBpt;
#pragma unroll
    for (int e = 0; e < kBpt; ++e) own += hist[top - e];
    // exclusive scan of `own` over threads (in order)
    const uint32_t incl = wave_incl_scan(own);
    if (lane == kWave - 1) red[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kClassifyThreads / kWave; ++w) before += w < wave ? red[w] : 0u;
    uint32_t cum = before + incl - own;            // sample scores in bins above `top`
#pragma unroll
    for (int e = 0; e < kBpt; ++e) {
        const uint32_t h = hist[top - e];
        // jH: the bin where the count from the top first reaches rank_hi, etc.
        if (cum < rank_hi && cum + h >= rank_hi) sel[0] = top - e;
        if (cum < rank_lo && cum + h >= rank_lo) sel[1] = top - e;
        cum += h;
    }
    __syncthreads();
    const int jH = sel[0], jL = sel[1];
    // classify this chunk: in = bin > jH, candidate = jL <= bin <= jH
    const ChunkWs r = chunk_ws(ws, i, c, nchunks, K);
    uint32_t n_in = 0, n_cd = 0;
    uint64_t m_in[kPer], m_cd[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int64_t b = b0 + u * kClassifyThreads + threadIdx.x;
        const bool ok = b < nb;
        const int bn = bin_of(x[u]);
        m_in[u] = __ballot(ok && bn > jH);
        m_cd[u] = __ballot(ok && bn >= jL && bn <= jH);
        n_in += (uint32_t)__builtin_popcountll(m_in[u]);
        n_cd += (uint32_t)__builtin_popcountll(m_cd[u]);
    }
    // per-wave totals -> offsets of this wave inside the chunk's lists
    __shared__ uint32_t wcnt[2][kClassifyThreads / kWave];
    if (lane == 0) { wcnt[0][wave] = n_in; wcnt[1][wave] = n_cd; }
    __syncthreads();
    uint32_t off_in = 0, off_cd = 0, tot_in = 0, tot_cd = 0;
#pragma unroll
    for (int w = 0; w < kClassifyThreads / kWave; ++w) {
        off_in += w < wave ? wcnt[0][w] : 0u;
        off_cd += w < wave ? wcnt[1][w] : 0u;
        tot_in += wcnt[0][w];
        tot_cd += wcnt[1][w];
    }
    if (threadIdx.x == 0) { r.cnt[0] = tot_in; r.cnt[1] = tot_cd; }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const uint32_t b = (uint32_t)(b0 + u * kClassifyThreads + threadIdx.x);
        if ((m_in[u] >> lane) & 1u) {
            const uint32_t pos = off_in + lanes_below(m_in[u]);
            if (pos < (uint32_t)K) r.in_idx[pos] = b;
        }
        if ((m_cd[u] >> lane) & 1u) {
            const uint32_t pos = off_cd + lanes_below(m_cd[u]);
            if (pos < (uint32_t)kChunkCandCap) {
                r.cand_key[pos] = order_key(x[u]);
                r.cand_idx[pos] = b;
            }
        }
        off_in += (uint32_t)__builtin_popcountll(m_in[u]);
        off_cd += (uint32_t)__builtin_popcountll(m_cd[u]);
    }
}

__global__ __launch_bounds__(kTopkThreads) void topk_finish_kernel(
    const float *__restrict__ scores, int64_t ld, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ q_off, int num_seqs, int log2r, int K, int nchunks,
    int32_t *__restrict__ idx, int ldi, const void *__restrict__ ws) {
    __shared__ TopkShared S;
    __shared__ uint32_t ck[kMultiCandMax], ci[kMultiCandMax];
    __shared__ uint32_t bitmap[kBitmapWordsMax];
    __shared__ uint32_t c_in[kMaxChunks + 1], c_cd[kMaxChunks + 1];
    __shared__ uint32_t bad;
    const int64_t i = blockIdx.x;
    const QueryPos qp = query_pos(kv_off, nullptr, q_off, num_seqs, i);
    const int64_t nb = qp.L >> log2r;
    if (nb <= K) return;                           // written by the classify kernel
    int32_t *out = idx + i * (int64_t)ldi;
    const int nch = (int)((nb + kClassifyChunk - 1) / kClassifyChunk);
    // per-chunk counts -> prefix offsets: lane c of wave 0 reads chunk c
    // (at most 64 chunks), then a wave scan
    if (threadIdx.x < kWave) {
        const int ln0 = threadIdx.x;
        uint32_t ni = 0, nd = 0;
        if (ln0 < nch) {
            const ChunkWs r = chunk_ws(ws, i, ln0, nchunks, K);
            ni = r.cnt[0];
            nd = r.cnt[1];
        }
        const bool over = __ballot(ln0 < nch && (ni > (uint32_t)K || nd > (uint32_t)kChunkCandCap)) != 0;
        const uint32_t si = wave_incl_scan(ni), sd = wave_incl_scan(nd);
        if (ln0 < nch) { c_in[ln0] = si - ni; c_cd[ln0] = sd - nd; }
        if (ln0 == nch - 1) {
            c_in[nch] = si;
            c_cd[nch] = sd;
            bad = over || si > (uint32_t)K || sd > (uint32_t)kMultiCandMax || si + sd < (uint32_t)K;
        }
    }
    __syncthreads();
    if (bad) {
        // the bracket missed: exact select over the whole row
        const GlobalKey key{scores + i * ld};
        uint32_t kmin = 0xffffffffu, kmax = 0u;
        for (int64_t b = threadIdx.x; b < nb; b += kTopkThreads) {
            const uint32_t k = key(b);
            kmin = min(kmin, k);
            kmax = max(kmax, k);
        }
        wg_minmax(kmin, kmax, S);
        select_row(key, nb, K, kmin, kmax, out, S);
        return;
    }
    const uint32_t n_in = c_in[nch], n_cand = c_cd[nch];
    const uint32_t need = (uint32_t)K - n_in;
    const int nwords = (int)((nb + 31) / 32);
    for (int w = threadIdx.x; w < nwords; w += kTopkThreads) bitmap[w] = 0u;
    // gather the candidates of every chunk (wave w takes chunks w, w+16, ...)
    const int wv = threadIdx.x / kWave, ln = threadIdx.x & (kWave - 1);
    uint32_t cmin = 0xffffffffu, cmax = 0u;
    for (int c = wv; c < nch; c += kTopkWaves) {
        const ChunkWs r = chunk_ws(ws, i, c, nchunks, K);
        const uint32_t nd = c_cd[c + 1] - c_cd[c];
        for (uint32_t j = ln; j < nd; j += kWave) {
            const uint32_t k = r.cand_key[j];
            ck[c_cd[c] + j] = k;
            ci[c_cd[c] + j] = r.cand_idx[j];
            cmin = min(cmin, k);
            cmax = max(cmax, k);
        }
    }
    wg_minmax(cmin, cmax, S);                      // barriers publish ck, ci, bitmap
    for (int c = wv; c < nch; c += kTopkWaves) {
        const ChunkWs r = chunk_ws(ws, i, c, nchunks, K);
        const uint32_t ni = c_in[c + 1] - c_in[c];
        for (uint32_t j = ln; j < ni; j += kWave) {
            const uint32_t b = r.in_idx[j];
            atomicOr(&bitmap[b >> 5], 1u << (b & 31));
        }
    }
    if (need > 0) {
        uint32_t need_eq, total_eq;
        const uint32_t T = radix_select(LdsKey{ck}, (int64_t)n_cand, need, cmin, cmax, S, need_eq,
                                        total_eq);
        const bool all_eq = need_eq >= total_eq;
        for (uint32_t j = threadIdx.x; j < n_cand; j += kTopkThreads) {
            const uint32_t k = ck[j];
            bool take = k > T;
            if (k == T) {
                if (all_eq) {
                    take = true;
                } else {
                    // ties at T go to the lower block index
                    const uint32_t me = ci[j];
                    uint32_t rank = 0;
                    for (uint32_t q = 0; q < n_cand; ++q) rank += (ck[q] == T && ci[q] < me) ? 1u : 0u;
                    take = rank < need_eq;
                }
            }
            if (take) atomicOr(&bitmap[ci[j] >> 5], 1u << (ci[j] & 31));
        }
    }
    __syncthreads();
    // ascending output: per-thread runs of words, popcounts scanned
    const int per = (nwords + kTopkThreads - 1) / kTopkThreads;
    const int w0 = threadIdx.x * per;
    uint32_t cnt = 0;
    for (int w = w0; w < w0 + per && w < nwords; ++w) cnt += (uint32_t)__builtin_popcount(bitmap[w]);
    uint32_t tot;
    uint32_t pos = wg_scan(cnt, S, tot);
    for (int w = w0; w < w0 + per && w < nwords; ++w) {
        uint32_t m = bitmap[w];
        while (m) {
            const int bit = __builtin_ctz(m);
            m &= m - 1;
            if (pos < (uint32_t)K) out[pos] = w * 32 + bit;
            ++pos;
        }
    }
}

// Few-row batches whose rows have at most kFusedMaxBlocks blocks: one
// 1024-thread workgroup per row runs the same selection as classify + finish
// in a single kernel.  The row's scores stay in registers (KPT per thread,
// block u*1024 + thread), the sample bracket is taken as in classify, the
// in / candidate split is counted with ballots, candidates are compacted
// straight into LDS and the in blocks set in the LDS bitmap; then the exact
// radix select over the candidates and the ordered bitmap output of finish.
// No workspace and no second launch; the exact whole-row select remains the
// fallback when the bracket misses.  Measured on one MI355X (K = 512): 32 rows
// of 8K blocks 12.4 us against about 17 us for classify + finish; from 16K
// blocks per row one workgroup pulling the whole row is the slower of the two.
constexpr int kFusedMaxBlocks = 8192;       // measured: from 16K blocks the two-kernel path is faster

template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void topk_fused_kernel(
    const float *__restrict__ scores, int64_t ld, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ q_off, int num_seqs, int log2r, int K, int32_t *__restrict__ idx, int ldi) {
    static_assert(KPT <= 16 && KPT * kTopkThreads / 32 <= kTopkThreads && kSample == 2 * kTopkThreads,
                  "row fits the registers; one bitmap word per thread; two sample values per thread");
    __shared__ TopkShared S;
    __shared__ uint32_t bitmap[KPT * kTopkThreads / 32];   // selected blocks
    __shared__ uint32_t tbits[KPT * kTopkThreads / 32];    // blocks whose key equals the threshold
    __shared__ uint32_t wcnt[2][kTopkWaves];
    __shared__ float fred[2][kTopkWaves];
    __shared__ int sel[2];
    const int64_t i = blockIdx.x;
    const QueryPos qp = query_pos(kv_off, nullptr, q_off, num_seqs, i);
    const int64_t nb = qp.L >> log2r;
    int32_t *out = idx + i * (int64_t)ldi;
    if (nb <= K) {
        for (int t = threadIdx.x; t < K; t += kTopkThreads) out[t] = (t < nb) ? t : -1;
        return;
    }
    const float *__restrict__ row = scores + i * ld;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    // the row and this thread's part of the sample, loaded together
    constexpr int kSmp = kSample / kTopkThreads;                 // 2
    float x[KPT], smp[kSmp];
    const bool whole = nb <= kSample;
    const int ns = whole ? (int)nb : kSample;
    constexpr int kSegs = kSample / kSegLen;
    const int64_t seg_step = whole ? 0 : (nb - kSegLen) / (kSegs - 1);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const int64_t b = (int64_t)u * kTopkThreads + threadIdx.x;
        x[u] = b < nb ? row[b] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kSmp; ++u) {
        const int t = u * kTopkThreads + threadIdx.x;
        const int64_t sb = whole ? t : (t / kSegLen) * seg_step + (t % kSegLen);
        smp[u] = t < ns ? row[sb] : 0.0f;
    }
    const int nwords = (int)((nb + 31) / 32);
    for (int t = threadIdx.x; t < kSample; t += kTopkThreads) S.hist[t] = 0;
    for (int w = threadIdx.x; w < nwords; w += kTopkThreads) { bitmap[w] = 0u; tbits[w] = 0u; }

    // sample range
    float vmin = INFINITY, vmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kSmp; ++u) {
        if (u * kTopkThreads + (int)threadIdx.x < ns) {
            vmin = fminf(vmin, smp[u]);
            vmax = fmaxf(vmax, smp[u]);
        }
    }
    vmin = wave_min_f32(vmin);
    vmax = wave_max_f32(vmax);
    if (lane == 0) { fred[0][wave] = vmin; fred[1][wave] = vmax; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
        vmin = fminf(vmin, fred[0][w]);
        vmax = fmaxf(vmax, fred[1][w]);
    }
    // monotone bin map: -1 below the sample range, 2047 at and above its top
    const float span = vmax - vmin;
    const float scale = span > 0.0f ? (float)kSample / span : 0.0f;
    auto bin_of = [&](float v) -> int {
        if (!(span > 0.0f)) return v < vmin ? -1 : (v > vmin ? kSample - 1 : 0);
        const float t = (v - vmin) * scale;
        return t < 0.0f ? -1 : (t >= (float)(kSample - 1) ? kSample - 1 : (int)t);
    };
#pragma unroll
    for (int u = 0; u < kSmp; ++u)
        if (u * kTopkThreads + (int)threadIdx.x < ns) atomicAdd(&S.hist[bin_of(smp[u])], 1u);
    __syncthreads();
    // sample ranks of the bracket (as in classify)
    uint32_t rank_hi, rank_lo;
    if (whole) {
        rank_hi = rank_lo = (uint32_t)K;
    } else {
        const float frac = (float)K / (float)nb;
        const float ks = frac * (float)ns;
        const float sd = __builtin_sqrtf(ks * (1.0f - frac));
        const int margin = (int)(4.0f * sd) + 8;
        const int kr = (int)__builtin_ceilf(ks);
        rank_hi = (uint32_t)(kr - margin < 1 ? 1 : kr - margin);
        rank_lo = (uint32_t)(kr + margin > ns ? ns : kr + margin);
    }
    // descending cumulative counts: thread t owns bins 2t, 2t+1 from the top
    constexpr int kBpt = kSample / kTopkThreads;
    const int top = kSample - 1 - (int)threadIdx.x * kBpt;
    uint32_t own = 0;
#pragma unroll
    for (int e = 0; e < kBpt; ++e) own += S.hist[top - e];
    uint32_t tot_s;
    uint32_t cum = wg_scan(own, S, tot_s);          // sample scores in bins above `top`
#pragma unroll
    for (int e = 0; e < kBpt; ++e) {
        const uint32_t h = S.hist[top - e];
        if (cum < rank_hi && cum + h >= rank_hi) sel[0] = top - e;
        if (cum < rank_lo && cum + h >= rank_lo) sel[1] = top - e;
        cum += h;
    }
    __syncthreads();
    const int jH = sel[0], jL = sel[1];
    // Classify every element once (in: above the bracket; candidate: inside
    // it); the counts and the candidates' key range come from one reduction.
    uint32_t kx[KPT];
    uint32_t cls = 0;                              // bit u: candidate; bit 16 + u: in
    uint32_t n_in = 0, n_cd = 0, cmin = 0xffffffffu, cmax = 0u;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const int64_t b = (int64_t)u * kTopkThreads + threadIdx.x;
        const bool ok = b < nb;
        const int bn = bin_of(x[u]);
        kx[u] = order_key(x[u]);
        if (ok && bn > jH) {
            cls |= 1u << (16 + u);
            ++n_in;
        } else if (ok && bn >= jL) {
            cls |= 1u << u;
            ++n_cd;
            cmin = min(cmin, kx[u]);
            cmax = max(cmax, kx[u]);
        }
    }
    {
        const uint32_t w_in = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(n_in), kWave - 1);
        const uint32_t w_cd = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(n_cd), kWave - 1);
        const uint32_t w_mn = wave_min_u32(cmin), w_mx = wave_max_u32(cmax);
        if (lane == 0) { wcnt[0][wave] = w_in; wcnt[1][wave] = w_cd; S.wmin[wave] = w_mn; S.wmax[wave] = w_mx; }
    }
    __syncthreads();
    uint32_t tot_in = 0, tot_cd = 0;
    cmin = 0xffffffffu;
    cmax = 0u;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
        tot_in += wcnt[0][w];
        tot_cd += wcnt[1][w];
        cmin = min(cmin, S.wmin[w]);
        cmax = max(cmax, S.wmax[w]);
    }
    if (tot_in > (uint32_t)K || tot_in + tot_cd < (uint32_t)K) {
        // the bracket missed: exact select over the whole row
        __syncthreads();                           // every wave has read S.wmin / S.wmax
        uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int64_t b = (int64_t)u * kTopkThreads + threadIdx.x;
            if (b < nb) {
                kmin = min(kmin, kx[u]);
                kmax = max(kmax, kx[u]);
            }
        }
        wg_minmax(kmin, kmax, S);
        select_row(GlobalKey{row}, nb, K, kmin, kmax, out, S);
        return;
    }
    // The threshold: the need-th largest candidate key, by MSB-first radix
    // digits over the candidates held in registers (as radix_select does
    // over a list).
    const uint32_t need0 = (uint32_t)K - tot_in;
    uint32_t T = 0xffffffffu, need_eq = 0, total_eq = 0;
    if (need0 > 0) {
        const uint32_t diff = cmin ^ cmax;
        if (diff == 0) {
            T = cmin;
            need_eq = need0;
            total_eq = tot_cd;
        } else {
            const int hi_bit = 31 - __builtin_clz(diff);
            uint32_t prefix = hi_bit == 31 ? 0u : (cmax & ~((2u << hi_bit) - 1u));
            uint32_t need = need0;
            int lo_bit = hi_bit + 1;
            while (lo_bit > 0) {
                const int width = lo_bit >= kDigitBits ? kDigitBits : lo_bit;
                const int shift = lo_bit - width;
                const uint32_t mask_hi = lo_bit >= 32 ? 0u : ~((1u << lo_bit) - 1u);
                for (int t = threadIdx.x; t < kBins; t += kTopkThreads) S.hist[t] = 0;
                __syncthreads();
#pragma unroll
                for (int u = 0; u < KPT; ++u)
                    if (((cls >> u) & 1u) && (kx[u] & mask_hi) == prefix)
                        atomicAdd(&S.hist[(kx[u] >> shift) & ((1u << width) - 1u)], 1u);
                __syncthreads();
                uint32_t above;
                const int d = find_bin(1 << width, need, S, above);
                total_eq = S.hist[d];
                prefix |= (uint32_t)d << shift;
                need -= above;
                lo_bit = shift;
                __syncthreads();
            }
            T = prefix;
            need_eq = need;
        }
    }
    // Mark: in blocks and candidates above T are selected; candidates equal
    // to T are all selected when all of them are needed, else they go to
    // the tie bitmap, where the lowest block indices win.
    const bool split_ties = need0 > 0 && need_eq < total_eq;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const uint32_t b = (uint32_t)(u * kTopkThreads + threadIdx.x);
        const uint32_t bit = 1u << (b & 31);
        if ((cls >> (16 + u)) & 1u) {
            atomicOr(&bitmap[b >> 5], bit);
        } else if (need0 > 0 && ((cls >> u) & 1u)) {
            if (kx[u] > T) atomicOr(&bitmap[b >> 5], bit);
            else if (kx[u] == T) atomicOr(split_ties ? &tbits[b >> 5] : &bitmap[b >> 5], bit);
        }
    }
    __syncthreads();
    // Ascending output: thread t owns bitmap word t.
    const int w = threadIdx.x;
    uint32_t word = w < nwords ? bitmap[w] : 0u;
    if (split_ties) {
        uint32_t tm = w < nwords ? tbits[w] : 0u;
        uint32_t tall;
        uint32_t r = wg_scan((uint32_t)__builtin_popcount(tm), S, tall);   // ties in lower words
        while (tm && r < need_eq) {
            word |= 1u << __builtin_ctz(tm);
            tm &= tm - 1;
            ++r;
        }
    }
    uint32_t tot;
    uint32_t pos = wg_scan((uint32_t)__builtin_popcount(word), S, tot);
    while (word) {
        const int bit = __builtin_ctz(word);
        word &= word - 1;
        if (pos < (uint32_t)K) out[pos] = w * 32 + bit;
        ++pos;
    }
}

// ------------------------------------------------------------------------
// Selection from the scorer's per-chunk candidate lists (qsa_lists.hpp):
// one 1024-thread workgroup per row, few barriers.
//  1. The row's listed keys (requested together with the row's offsets, for
//     the first kSpecEntries entries) go to LDS with their block ids, in list
//     order (ascending block order); one exchange gives the listed keys' min
//     and max, how many are real (not padding) and the largest chunk cutoff.
//  2. A histogram of 1024 bins linear in the score between min and max (one
//     bin per thread): the bin map is monotone, so the K-th largest key T
//     lies in the bin where the count from the top first reaches K.
//  3. That bin's keys (typically a handful) go to a short LDS list, and one
//     wave finds T among them exactly by bisection (MSB first, two bits per
//     step); more than 64 keys in the bin (heavy ties, adversarial spreads)
//     take the exact radix select over the whole list instead.
//  4. Certificate: T > 0 and every chunk cutoff < T (then every block with
//     key >= T is listed).  Output in ascending order: thread t owns list
//     entries [t*E, t*E + E); one scan of (keys > T, keys == T) per thread
//     gives its first output position, above + min(ties before, ties needed),
//     because ties are taken in list (= block) order.
// A row that fails the certificate, or whose lists exceed the LDS (`cap`
// entries), is selected from its whole score row.
constexpr int kListBins = kTopkThreads;             // one bin per thread
constexpr int kSpecEntries = 4 * kTopkThreads;      // list entries requested before the length is known
constexpr int kBinCandMax = kWave;                  // threshold-bin keys one wave resolves

__global__ __launch_bounds__(kTopkThreads) void topk_lists_kernel(
    const float *__restrict__ scores, int64_t ld, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ q_off, int num_seqs, int log2r, int K, int32_t *__restrict__ idx, int ldi,
    ListArgs la, int cap) {
    __shared__ TopkShared S;
    __shared__ uint32_t bcand[kBinCandMax];
    extern __shared__ uint32_t lds_lists[];          // keys [cap], then lanes [cap] (bytes)
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t i = blockIdx.x;
    const uint32_t *__restrict__ gk = la.keys + i * la.stride;
    const uint8_t *__restrict__ gl = la.loc + i * la.stride;
    const uint32_t *__restrict__ gc = la.cut + i * la.cstride;
    // Speculative requests (inside the row's regions whatever its length):
    // the first list entries and chunk cutoffs, alongside the offsets.
    const int spec_n = (int)(la.stride < kSpecEntries ? la.stride : kSpecEntries);
    const int spec_c = (int)(la.cstride < kTopkThreads ? la.cstride : kTopkThreads);
    uint32_t k[4], l[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = (int)threadIdx.x + u * kTopkThreads;
        k[u] = j < spec_n ? gk[j] : 0u;
        l[u] = j < spec_n ? gl[j] : 0u;
    }
    const uint32_t c0 = (int)threadIdx.x < spec_c ? gc[threadIdx.x] : 0u;
    const uint32_t mode = *la.mode;
    const QueryPos qp = query_pos(kv_off, nullptr, q_off, num_seqs, i);
    const int64_t nb = qp.L >> log2r;
    int32_t *out = idx + i * (int64_t)ldi;
    if (nb <= K) {
        for (int t = threadIdx.x; t < K; t += kTopkThreads) out[t] = (t < nb) ? t : -1;
        return;
    }
    const int kk = list_len(nb, K);
    const int nch = (int)((nb + kListChunk - 1) / kListChunk);
    const int M = nch * kk;
    // the last entry of a row whose newest token completed a block is that
    // block, scored by the append (its chunk left the slot)
    const bool nslot = list_new_block_slot(mode, qp.L, log2r);
    const uint32_t nkey = nslot ? list_order_key(scores[i * ld + nb - 1]) : 0u;
    const uint32_t nloc = (uint32_t)((nb - 1) & (kListChunk - 1));
    if (M <= cap) {
        uint32_t *keys = lds_lists;
        uint8_t *locs = reinterpret_cast<uint8_t *>(lds_lists + cap);
        // entries j = t + u*1024 (u < 4) stay in registers too (kr); the
        // rest (rows with more than 4096 entries) are read back from LDS
        uint32_t kmin = 0xffffffffu, kmax = 0u, nreal = 0u;
        uint32_t mcut = (int)threadIdx.x < nch ? c0 : 0u;
        for (int c = (int)threadIdx.x + kTopkThreads; c < nch; c += kTopkThreads) mcut = max(mcut, gc[c]);
        auto note = [&](uint32_t key) {
            if (key != 0u) {                         // padding (key 0) is not a block
                kmin = min(kmin, key);
                kmax = max(kmax, key);
                ++nreal;
            }
        };
        uint32_t kr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = (int)threadIdx.x + u * kTopkThreads;
            kr[u] = 0u;
            if (j < M) {
                const bool nj = nslot && j == M - 1;
                kr[u] = nj ? nkey : (j < spec_n ? k[u] : gk[j]);
                keys[j] = kr[u];
                locs[j] = (uint8_t)(nj ? nloc : (j < spec_n ? l[u] : gl[j]));
                note(kr[u]);
            }
        }
        for (int j = (int)threadIdx.x + 4 * kTopkThreads; j < M; j += kTopkThreads) {
            const bool nj = nslot && j == M - 1;
            const uint32_t key = nj ? nkey : gk[j];
            keys[j] = key;
            locs[j] = nj ? (uint8_t)nloc : gl[j];
            note(key);
        }
        S.hist[threadIdx.x] = 0u;                    // the linear histogram's bin
        // one exchange for the four reductions (its barrier also publishes keys / locs)
        {
            const uint32_t w_mn = wave_min_u32(kmin), w_mx = wave_max_u32(kmax), w_mc = wave_max_u32(mcut);
            const uint32_t w_n = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(nreal), kWave - 1);
            if (lane == 0) {
                S.wmin[wave] = w_mn;
                S.wmax[wave] = w_mx;
                S.wsum[wave] = w_n;
                S.cand[wave] = w_mc;
            }
            __syncthreads();
            kmin = S.wmin[0];
            kmax = S.wmax[0];
            nreal = S.wsum[0];
            mcut = S.cand[0];
#pragma unroll
            for (int w = 1; w < kTopkWaves; ++w) {
                kmin = min(kmin, S.wmin[w]);
                kmax = max(kmax, S.wmax[w]);
                nreal += S.wsum[w];
                mcut = max(mcut, S.cand[w]);
            }
        }
        uint32_t T = 0u, need_eq = 0u, total_eq = 0u;
        bool found = false, hopeless = false;
        if (nreal < (uint32_t)K || mcut >= kmax) {
            // fewer listed blocks than K, or a cutoff at or above every
            // listed key: the certificate cannot hold
        } else if (kmin == kmax) {
            T = kmin;
            need_eq = (uint32_t)K;
            total_eq = nreal;
            found = true;
        } else {
            // A certified threshold exceeds every cutoff, so only keys from
            // lo = max(kmin, mcut + 1) up can be it (a short chunk listed
            // whole can hold keys far below the rest, which would crowd
            // coarse bins).  kListBins bins linear in the key.
            const uint32_t lo = max(kmin, mcut + 1u);
            const uint32_t span = kmax - lo;
            const int sh = span < (uint32_t)kListBins ? 0 : (32 - __builtin_clz(span)) - 10;
            static_assert(kListBins == 1024, "bin shift assumes 1024 bins");
            auto bin_of = [&](uint32_t key) { return (int)((key - lo) >> sh); };
            int kb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                kb[u] = kr[u] >= lo ? bin_of(kr[u]) : -1;
                if (kb[u] >= 0) atomicAdd(&S.hist[kb[u]], 1u);
            }
            for (int j = (int)threadIdx.x + 4 * kTopkThreads; j < M; j += kTopkThreads) {
                const uint32_t key = keys[j];
                if (key >= lo) atomicAdd(&S.hist[bin_of(key)], 1u);
            }
            if (threadIdx.x == 0) {
                S.s2 = 0u;
                S.s0 = 0xffffffffu;                  // no bin holds the K-th key yet
            }
            __syncthreads();
            // thread t owns bin kListBins-1-t: the count above it by one scan
            const int bin = kListBins - 1 - (int)threadIdx.x;
            const uint32_t h = S.hist[bin];
            uint32_t tot;
            const uint32_t above = wg_scan(h, S, tot);
            if (above < (uint32_t)K && (uint32_t)K <= above + h) {
                S.s0 = (uint32_t)bin;
                S.s1 = above;
                S.s3 = h;
            }
            __syncthreads();
            // fewer than K keys above the cutoffs: the certificate cannot hold
            hopeless = S.s0 == 0xffffffffu;
            const int tb = (int)S.s0;
            const uint32_t need = (uint32_t)K - S.s1;
            const uint32_t nbin = hopeless ? 0xffffffffu : S.s3;
            if (nbin <= (uint32_t)kBinCandMax) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (kb[u] == tb) bcand[atomicAdd(&S.s2, 1u)] = kr[u];
                for (int j = (int)threadIdx.x + 4 * kTopkThreads; j < M; j += kTopkThreads) {
                    const uint32_t key = keys[j];
                    if (key >= lo && bin_of(key) == tb) bcand[atomicAdd(&S.s2, 1u)] = key;
                }
                __syncthreads();
                if (wave == 0) {
                    // the need-th largest of the bin's nbin keys, exactly: lane
                    // l < nbin counts the bin's keys above and equal to its own
                    // (broadcast reads), and the key whose rank range holds
                    // `need` is T
                    const bool own = lane < (int)nbin;
                    const uint32_t key = own ? bcand[lane] : 0u;
                    uint32_t gt = 0, eq = 0;
                    for (int j = 0; j < (int)nbin; ++j) {
                        const uint32_t o = bcand[j];
                        gt += o > key ? 1u : 0u;
                        eq += o == key ? 1u : 0u;
                    }
                    const bool hit = own && gt < need && need <= gt + eq;
                    const uint64_t m = __ballot(hit);
                    if (hit && lane == (int)__builtin_ctzll(m)) {
                        S.s0 = key;
                        S.s1 = need - gt;
                        S.s3 = eq;
                    }
                }
                __syncthreads();
                T = S.s0;
                need_eq = S.s1;
                total_eq = S.s3;
                found = true;
            }
        }
        if (!found && !hopeless && nreal >= (uint32_t)K && mcut < kmax) {
            __syncthreads();
            T = radix_select(LdsKey{keys}, (int64_t)M, (uint32_t)K, kmin, kmax, S, need_eq, total_eq);
        }
        if (T != 0u && mcut < T) {
            // ordered output: thread t owns list entries [t*E, t*E + E); entry j
            // is lane locs[j] of chunk j / kk
            const int E = (M + kTopkThreads - 1) / kTopkThreads;
            const int j0 = (int)threadIdx.x * E;
            const int j1 = j0 + E < M ? j0 + E : M;
            uint32_t ngt = 0, neq = 0;
            for (int j = j0; j < j1; ++j) {
                const uint32_t key = keys[j];
                ngt += key > T ? 1u : 0u;
                neq += key == T ? 1u : 0u;
            }
            uint32_t tot;
            const uint32_t before = wg_scan((ngt << 16) | neq, S, tot);   // both counts < 2^16
            uint32_t tie = before & 0xffffu;
            uint32_t pos = (before >> 16) + min(tie, need_eq);
            int chunk = j0 < M ? j0 / kk : 0;
            int slot = j0 - chunk * kk;
            for (int j = j0; j < j1; ++j) {
                const uint32_t key = keys[j];
                bool take = key > T;
                if (key == T) {
                    take = tie < need_eq;
                    ++tie;
                }
                if (take) {
                    if (pos < (uint32_t)K) out[pos] = chunk * kListChunk + locs[j];
                    ++pos;
                }
                if (++slot == kk) {
                    slot = 0;
                    ++chunk;
                }
            }
            return;
        }
        __syncthreads();
    }
    // the whole score row
    const float *__restrict__ row = scores + i * ld;
    const GlobalKey key{row};
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll 4
    for (int64_t b = threadIdx.x; b < nb; b += kTopkThreads) {
        const uint32_t kx = key(b);
        kmin = min(kmin, kx);
        kmax = max(kmax, kx);
    }
    wg_minmax(kmin, kmax, S);
    select_row(key, nb, K, kmin, kmax, out, S);
}

}  // namespace

// Candidate lists of a score + select call: row stride of ceil(max_nb/64)
// chunks of 64 entries (keys u32, then chunk cutoffs u32, then lanes u8).
static int64_t list_chunks(const qsa_batch &b, int ratio) {
    const int64_t max_nb = b.max_kv_len / ratio;
    return max_nb > 0 ? (max_nb + kListChunk - 1) / kListChunk : 1;
}

bool score_topk_uses_lists(const qsa_batch &b) { return b.total_q >= 1 && b.total_q <= kMultiMaxRows; }

size_t score_topk_workspace_bytes(const qsa_batch &b, int budget, int ratio) {
    if (!score_topk_uses_lists(b)) return topk_workspace_bytes(b, budget, ratio, nullptr);
    const size_t rows = (size_t)b.total_q, nch = (size_t)list_chunks(b, ratio);
    const size_t keys = rows * nch * kListChunk * 4, cuts = rows * nch * 4, locs = rows * nch * kListChunk;
    // keys, cutoffs, lanes, then the lists' mode word
    return ((keys + 255) & ~(size_t)255) + ((cuts + 255) & ~(size_t)255) + ((locs + 255) & ~(size_t)255) + 256;
}

ListArgs list_args(const qsa_batch &b, int budget, int ratio, void *ws) {
    const int64_t nch = list_chunks(b, ratio);
    const size_t rows = (size_t)b.total_q;
    uint8_t *base = static_cast<uint8_t *>(ws);
    const size_t keys_bytes = (rows * nch * kListChunk * 4 + 255) & ~(size_t)255;
    const size_t cuts_bytes = (rows * nch * 4 + 255) & ~(size_t)255;
    const size_t locs_bytes = (rows * nch * kListChunk + 255) & ~(size_t)255;
    ListArgs la;
    la.keys = reinterpret_cast<uint32_t *>(base);
    la.cut = reinterpret_cast<uint32_t *>(base + keys_bytes);
    la.loc = base + keys_bytes + cuts_bytes;
    la.mode = reinterpret_cast<uint32_t *>(base + keys_bytes + cuts_bytes + locs_bytes);
    la.stride = nch * kListChunk;
    la.cstride = nch;
    la.K = budget / ratio;
    return la;
}

hipError_t launch_topk_from_lists(const float *scores, int64_t ld, int budget, int ratio, const qsa_batch &b,
                                  int32_t *idx, const ListArgs &la, hipStream_t st) {
    if (b.total_q == 0) return hipSuccess;
    const int K = budget / ratio;
    const int64_t nch = list_chunks(b, ratio);
    const int64_t bound = nch * kListChunk;
    const int cap = (int)(bound < kListMaxEntries ? bound : kListMaxEntries);
    const size_t lds = (size_t)cap * 5;
    hipError_t e = enable_dyn_lds((const void *)topk_lists_kernel, (int)lds);
    if (e != hipSuccess) return e;
    const int log2r = __builtin_ctz((unsigned)ratio);
    trace("topk lists rows=%lld K=%d chunks=%lld cap=%d", (long long)b.total_q, K, (long long)nch, cap);
    hipLaunchKernelGGL(topk_lists_kernel, dim3((unsigned)b.total_q), dim3(kTopkThreads), lds, st, scores, ld,
                       b.kv_offsets, b.q_offsets, b.num_seqs, log2r, K, idx, K, la, cap);
    return hipGetLastError();
}

hipError_t launch_score_topk(const qsa_indexer &ix, int budget, int ratio, const qsa_batch &b, float *scores,
                             int64_t ld, int32_t *idx, void *ws, const qsa_paged_kv *pg, hipStream_t st) {
    if (b.total_q == 0) return hipSuccess;
    const int K = budget / ratio;
    if (!score_topk_uses_lists(b)) {
        hipError_t e = launch_score_canonical(ix, ratio, b, scores, ld, pg, st, ListArgs{});
        if (e != hipSuccess) return e;
        return launch_topk(scores, ld, nullptr, budget, ratio, b, idx, K, ws, st);
    }
    const ListArgs la = list_args(b, budget, ratio, ws);
    hipError_t e = launch_score_canonical(ix, ratio, b, scores, ld, pg, st, la);
    if (e != hipSuccess) return e;
    return launch_topk_from_lists(scores, ld, budget, ratio, b, idx, la, st);
}

static int64_t norm_chunks(const qsa_batch &b, int ratio) {
    const int64_t max_nb = b.max_kv_len / ratio;
    return max_nb > 0 ? (max_nb + kNormThreads - 1) / kNormThreads : 1;
}

size_t topk_workspace_bytes(const qsa_batch &b, int budget, int ratio, const qsa_indexer *recheck) {
    if (recheck == nullptr) {
        // few-row batches use the multi-workgroup select and its row lists
        if (b.total_q < 1 || b.total_q > kMultiMaxRows) return 0;
        const int64_t max_nb = b.max_kv_len / ratio;
        const int64_t nch = max_nb > 0 ? (max_nb + kClassifyChunk - 1) / kClassifyChunk : 1;
        return (size_t)b.total_q * (size_t)nch * chunk_region_bytes(budget / ratio) + 256;
    }
    return (size_t)b.num_seqs * (size_t)norm_chunks(b, ratio) * sizeof(float) + 256;
}

hipError_t launch_topk(const float *scores, int64_t ld, const qsa_indexer *recheck, int budget,
                       int ratio, const qsa_batch &b, int32_t *idx, int ldi, void *ws, hipStream_t st) {
    if (b.total_q == 0) return hipSuccess;
    const int log2r = __builtin_ctz((unsigned)ratio);
    const int K = budget / ratio;
    const int64_t max_nb = b.max_kv_len >> log2r;
    const size_t lds = (size_t)(max_nb > 0 ? max_nb : 1) * sizeof(uint32_t);
    dim3 grid((unsigned)b.total_q);
    // Dynamic LDS above the 64 KB default must be enabled per kernel (and device).
    hipError_t attr_err = enable_dyn_lds((const void *)topk_kernel<true>, (int)(kLdsKeys * sizeof(uint32_t)));
    if (attr_err == hipSuccess)
        attr_err = enable_dyn_lds((const void *)topk_cert_kernel, (int)(kLdsKeys * sizeof(uint32_t)));
    if (attr_err != hipSuccess) return attr_err;
    if (recheck != nullptr) {
        if (max_nb > kTopkRecheckMaxBlocks) return hipErrorNotSupported;
        const int nch = (int)norm_chunks(b, ratio);
        float *part = static_cast<float *>(ws);
        trace("topk_cert norms grid=%dx%d", nch, b.num_seqs);
        hipLaunchKernelGGL(block_norm_kernel, dim3((unsigned)nch, (unsigned)b.num_seqs),
                           dim3(kNormThreads), 0, st, recheck->kc, recheck->kc_dtype,
                           static_cast<const float *>(recheck->kc_scale), recheck->d_idx, b.blk_offsets, nch, part);
        const CertIndexer cix{recheck->q_idx, recheck->w, recheck->kc, static_cast<const float *>(recheck->kc_scale),
                              recheck->q_dtype, recheck->kc_dtype, recheck->h_idx, recheck->d_idx};
        trace("topk_cert grid=%u K=%d ratio=%d lds_keys=%lld", grid.x, K, ratio, (long long)max_nb);
        hipLaunchKernelGGL(topk_cert_kernel, grid, dim3(kTopkThreads), lds, st, scores, ld,
                           b.kv_offsets, b.blk_offsets, b.q_offsets, b.num_seqs, log2r, K, idx, ldi, cix,
                           part, nch);
        return hipGetLastError();
    }
    if (b.total_q <= kMultiMaxRows && max_nb <= kFusedMaxBlocks) {
        trace("topk fused rows=%lld K=%d ratio=%d max_nb=%lld", (long long)b.total_q, K, ratio,
              (long long)max_nb);
#define QSA_TOPK_FUSED(KPT)                                                                        \
    hipLaunchKernelGGL(topk_fused_kernel<KPT>, grid, dim3(kTopkThreads), 0, st, scores, ld,         \
                       b.kv_offsets, b.q_offsets, b.num_seqs, log2r, K, idx, ldi)
        static_assert(kFusedMaxBlocks == 8 * kTopkThreads, "fused instantiations cover the limit");
        if (max_nb <= 2 * kTopkThreads) QSA_TOPK_FUSED(2);
        else if (max_nb <= 4 * kTopkThreads) QSA_TOPK_FUSED(4);
        else QSA_TOPK_FUSED(8);
#undef QSA_TOPK_FUSED
        return hipGetLastError();
    }
    if (b.total_q <= kMultiMaxRows && max_nb <= (int64_t)kBitmapWordsMax * 32) {
        const int chunks = (int)(max_nb > 0 ? (max_nb + kClassifyChunk - 1) / kClassifyChunk : 1);
        trace("topk multi rows=%lld K=%d ratio=%d chunks=%d", (long long)b.total_q, K, ratio, chunks);
        hipLaunchKernelGGL(topk_classify_kernel, dim3((unsigned)chunks, (unsigned)b.total_q),
                           dim3(kClassifyThreads), 0, st, scores, ld, b.kv_offsets, b.q_offsets,
                           b.num_seqs, log2r, K, chunks, idx, ldi, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(topk_finish_kernel, grid, dim3(kTopkThreads), 0, st, scores, ld,
                           b.kv_offsets, b.q_offsets, b.num_seqs, log2r, K, chunks, idx, ldi, ws);
        return hipGetLastError();
    }
    if (max_nb <= kLdsKeys) {
        trace("topk grid=%u K=%d ratio=%d lds_keys=%lld", grid.x, K, ratio, (long long)max_nb);
        hipLaunchKernelGGL(topk_kernel<true>, grid, dim3(kTopkThreads), lds, st, scores, ld,
                           b.kv_offsets, b.q_offsets, b.num_seqs, log2r, K, idx, ldi);
    } else {
        trace("topk grid=%u K=%d ratio=%d streaming", grid.x, K, ratio);
        hipLaunchKernelGGL(topk_kernel<false>, grid, dim3(kTopkThreads), 0, st, scores, ld,
                           b.kv_offsets, b.q_offsets, b.num_seqs, log2r, K, idx, ldi);
    }
    return hipGetLastError();
}

// Recent window kept: row i of idx (stride ldi) holds the ascending top-K
// selection, -1 padded; rewrite it in place as the ascending union of that
// selection and the last min(w, nb) complete blocks, -1 padded to K + w
// entries.  The selection's entries below the window stay where they are,
// so one wave per row counts them and writes only what follows.
__global__ __launch_bounds__(kWave) void topk_local_kernel(
    const int64_t *__restrict__ kv_off, const int64_t *__restrict__ q_off, int num_seqs, int log2r,
    int K, int w, int32_t *__restrict__ idx, int ldi) {
    const int64_t i = blockIdx.x;
    const int lane = threadIdx.x;
    const QueryPos qp = query_pos(kv_off, nullptr, q_off, num_seqs, i);
    const int64_t nb = qp.L >> log2r;
    const int64_t wv = nb < w ? nb : w;
    const int64_t bound = nb - wv;                 // first block of the window
    int32_t *row = idx + i * (int64_t)ldi;
    uint32_t keep = 0;                             // entries in [0, bound): a prefix of the row
    for (int j = lane; j < K; j += kWave) {
        const int32_t e = row[j];
        keep += (e >= 0 && (int64_t)e < bound) ? 1u : 0u;
    }
    keep = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(keep), 63);
    for (int j = (int)keep + lane; j < K + w; j += kWave) {
        const int64_t t = j - (int64_t)keep;
        row[j] = t < wv ? (int32_t)(bound + t) : -1;
    }
}

hipError_t launch_topk_local(int budget, int ratio, int local_blocks, const qsa_batch &b, int32_t *idx,
                             int ldi, hipStream_t st) {
    if (b.total_q == 0) return hipSuccess;
    const int log2r = __builtin_ctz((unsigned)ratio);
    trace("topk_local rows=%lld K=%d w=%d", (long long)b.total_q, budget / ratio, local_blocks);
    hipLaunchKernelGGL(topk_local_kernel, dim3((unsigned)b.total_q), dim3(kWave), 0, st, b.kv_offsets,
                       b.q_offsets, b.num_seqs, log2r, budget / ratio, local_blocks, idx, ldi);
    return hipGetLastError();
}

}  // namespace qsa
