// Device helpers shared by the libqsa kernels (gfx950 / CDNA4).
//
// The whole library is compiled with -ffp-contract=off: no multiply-add is
// fused unless a kernel asks for it with an explicit fma, which it does only
// where the product is exact (bf16*bf16, bf16*e4m3) and the fused result is
// therefore the same as a rounded multiply followed by a rounded add.
#pragma once

#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

// ---- wave-wide (64-lane) scans and reductions on the DPP network.  Shuffles
// (__shfl_*) go through ds_bpermute, an LDS round trip per step; these use
// DPP row shifts and the row broadcasts of the gfx9 family instead, a few
// cycles per step.  Lanes whose DPP source is outside the row (or rows not
// selected by the row mask) receive `old`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes (lane order).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += dpp_u32<kDppRowShr1>(0u, x);
    x += dpp_u32<kDppRowShr2>(0u, x);
    x += dpp_u32<kDppRowShr4>(0u, x);
    x += dpp_u32<kDppRowShr8>(0u, x);          // prefix within each row of 16
    x += dpp_u32<kDppRowBcast15, 0xa>(0u, x);  // rows 1, 3 += last lane of rows 0, 2
    x += dpp_u32<kDppRowBcast31, 0xc>(0u, x);  // rows 2, 3 += lane 31 (rows 0-1 total)
    return x;
}
// Wave-uniform reductions (the result of lane 63, read into a scalar).
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x, Op op) {
    x = op(x, dpp_u32<kDppRowShr1>(x, x));
    x = op(x, dpp_u32<kDppRowShr2>(x, x));
    x = op(x, dpp_u32<kDppRowShr4>(x, x));
    x = op(x, dpp_u32<kDppRowShr8>(x, x));
    x = op(x, dpp_u32<kDppRowBcast15, 0xa>(x, x));
    x = op(x, dpp_u32<kDppRowBcast31, 0xc>(x, x));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
    return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ float wave_max_f32(float x) {
    return __uint_as_float(wave_reduce_u32(__float_as_uint(x), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    }));
}
__device__ __forceinline__ float wave_sum_f32(float x) {
    return __uint_as_float(wave_reduce_u32(__float_as_uint(x), [](uint32_t a, uint32_t b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}
__device__ __forceinline__ float wave_min_f32(float x) {
    return __uint_as_float(wave_reduce_u32(__float_as_uint(x), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
    }));
}

// Paged caches: logical row t of sequence s lives in pool row
// table[s * stride + (t >> log2_rows)] << log2_rows | (t & (2^log2_rows - 1)),
// where 2^log2_rows rows make a page (token rows: page_size; compressed rows:
// page_size / ratio).  table == nullptr: the contiguous layout (no paging).
struct PageMap {
    const int32_t *table;
    int64_t stride;
    int log2_page;           // token rows per page
};
inline PageMap page_map(const qsa_paged_kv *pg) {
    PageMap m{nullptr, 0, 0};
    if (pg) {
        m.table = pg->block_table;
        m.stride = pg->max_pages;
        m.log2_page = __builtin_ctz((unsigned)pg->page_size);
    }
    return m;
}
__device__ __forceinline__ int64_t paged_row(const PageMap &pm, int64_t seq, int64_t t, int log2_rows) {
    const int64_t page = pm.table[seq * pm.stride + (t >> log2_rows)];
    return (page << log2_rows) | (t & ((int64_t(1) << log2_rows) - 1));
}

// Compile-time loop: f(integral_constant<int, B>) ... f(integral_constant<int, E-1>).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs): add
// 0x7fff plus the parity of the kept LSB, then truncate.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Pack two floats as bf16 (RNE) into one dword: lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------- e4m3
// OCP E4M3FN (bias 7, max finite 448).  Decode uses the gfx950 conversion
// instruction (OCP format on this target); two codes per call.
template <bool HIGH_WORD>
__device__ __forceinline__ float2 e4m3x2_to_f32(uint32_t packed) {
    auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)packed, HIGH_WORD);
    return make_float2(v[0], v[1]);
}

// fp32 -> E4M3FN code, round to nearest even, for |y| <= 448 (callers clamp).
// Normal range (|y| >= 2^-6): integer round at fp32 mantissa bit 20 and
// re-bias the exponent (127 -> 7).  Below 2^-6 the code is the integer
// rint(|y| * 2^9) (subnormal step 2^-9; 8 becomes the smallest normal).
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
    uint32_t u = __float_as_uint(y);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    uint32_t mag;
    if (a >= 0x3c800000u) {                       // 2^-6
        uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
        mag = (r >> 20) - (120u << 3);
    } else {
        mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    }
    return sign | mag;
}

__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

// ------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = v + __shfl_xor(v, o, kWave);
    return v;
}

// Query -> sequence for varlen batches: the s with q_off[s] <= i < q_off[s+1]
// (binary search over B+1 device offsets; uniform across the wave).
__device__ __forceinline__ int find_seq(const int64_t *__restrict__ q_off, int num_seqs, int64_t i) {
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (q_off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Visible length of query i: sequence s, its own position + 1.
struct QueryPos {
    int seq;
    int64_t L;        // visible tokens
    int64_t kv_row0;  // first row of the sequence in K/V/k_idx
    int64_t blk_row0; // first row of the sequence in kc
};

__device__ __forceinline__ QueryPos query_pos(const int64_t *__restrict__ kv_off,
                                              const int64_t *__restrict__ blk_off,
                                              const int64_t *__restrict__ q_off, int num_seqs,
                                              int64_t i) {
    QueryPos p;
    if (q_off == nullptr) {
        p.seq = (int)i;
        p.kv_row0 = kv_off[i];
        p.L = kv_off[i + 1] - p.kv_row0;
    } else {
        p.seq = find_seq(q_off, num_seqs, i);
        p.kv_row0 = kv_off[p.seq];
        int64_t n = kv_off[p.seq + 1] - p.kv_row0;
        int64_t nq = q_off[p.seq + 1] - q_off[p.seq];
        p.L = n - nq + (i - q_off[p.seq]) + 1;
    }
    p.blk_row0 = blk_off ? blk_off[p.seq] : 0;
    return p;
}

}  // namespace qsa
