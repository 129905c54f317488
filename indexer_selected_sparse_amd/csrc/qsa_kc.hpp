// Compressed-key arithmetic shared by the batch compression pass and the
// per-step ingest: the fp32 widening of one raw indexer-key row, and the
// mean -> fp32 / bf16 / e4m3(+scale) store of one compressed row ("Agentic
// shootout" page, "Flash-Next support: vLLM vs Atlas", section (a)6: one
// mean-pooled key per complete group; the long-context decode workload's
// e4m3 index plane with one fp32 scale max|x|/448 per block).
//
// A wave owns one row: lane l holds dims l*DPL .. l*DPL+DPL-1 of a
// DPL*64-wide row.  Both callers sum the block's rows in token order in fp32
// starting from +0 and multiply by 1/ratio, so a block compressed either
// way is bit-identical.
#pragma once

#include "qsa_device.hpp"

namespace qsa {

template <typename TIn, int DPL>
__device__ __forceinline__ void load_row(const TIn *__restrict__ p, float (&x)[DPL]);

template <>
__device__ __forceinline__ void load_row<uint16_t, 1>(const uint16_t *__restrict__ p, float (&x)[1]) {
    x[0] = bf16_to_f32(p[0]);
}
template <>
__device__ __forceinline__ void load_row<uint16_t, 2>(const uint16_t *__restrict__ p, float (&x)[2]) {
    uint32_t u = *reinterpret_cast<const uint32_t *>(p);
    x[0] = bf16lo(u);
    x[1] = bf16hi(u);
}
template <>
__device__ __forceinline__ void load_row<float, 1>(const float *__restrict__ p, float (&x)[1]) {
    x[0] = p[0];
}
template <>
__device__ __forceinline__ void load_row<float, 2>(const float *__restrict__ p, float (&x)[2]) {
    float2 v = *reinterpret_cast<const float2 *>(p);
    x[0] = v.x;
    x[1] = v.y;
}

// E2M1 code of y: the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 in magnitude,
// ties to the even mantissa (code bit 0), magnitudes past 6 give 6; the sign
// bit of y is kept (bit 3).
__device__ __forceinline__ uint32_t f32_to_e2m1(float y) {
    const float a = fabsf(y);
    const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                     : a <= 2.5f  ? 4u : a < 3.5f  ? 5u : a <= 5.0f  ? 6u : 7u;
    return c | ((__float_as_uint(y) >> 28) & 8u);
}

// KC: 0 = fp32, 1 = bf16 (round to nearest even), 2 = e4m3 + fp32 scale
// (kc_scale: float per row), 3 = fp4: E2M1 codes two per byte, one E8M0
// scale byte per 32 dims (kc_scale: bytes [rows, D/32]) with exponent
// X = floor(log2(amax of the group)) - 2 in [-127, 127] (-127 for amax 0).
// m = this lane's DPL means; the whole wave must call it (e4m3 and fp4
// reduce amax over lanes).  dec receives the stored key's values as the
// scorer widens them (exact): bf16 and fp32 values, e4m3 code values (sc =
// the row's scale, applied after the dot), fp4 code values times 2^X.
template <int KC, int DPL>
__device__ __forceinline__ void store_kc(const float (&m)[DPL], void *__restrict__ kc,
                                         void *__restrict__ kc_scale, int64_t out_row, int lane,
                                         float (&dec)[DPL], float &sc) {
    constexpr int D = DPL * kWave;
    sc = 1.0f;
    const int64_t o = out_row * D + lane * DPL;
    if constexpr (KC == 3) {
        constexpr int LPG = 32 / DPL;                 // lanes per 32-dim group
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) amax = fmaxf(amax, fabsf(m[e]));
#pragma unroll
        for (int off = LPG / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
        int X = -127;
        if (amax != 0.0f) {
            X = __builtin_amdgcn_frexp_expf(amax) - 1 - 2;   // amax = f * 2^k, f in [0.5, 1)
            X = X < -127 ? -127 : (X > 127 ? 127 : X);
        }
        uint32_t c[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) c[e] = f32_to_e2m1(__builtin_amdgcn_ldexpf(m[e], -X));
        {
            const uint32_t E = (uint32_t)(X + 127);
            const float scl = __uint_as_float(E ? (E << 23) : 0x00400000u);   // 2^X (E = 0: 2^-127)
            uint32_t word = c[0];
            if constexpr (DPL == 2) word |= c[1] << 4;
            const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scl, 0);
            dec[0] = v[0];
            if constexpr (DPL == 2) dec[1] = v[1];
        }
        uint8_t *codes = static_cast<uint8_t *>(kc) + out_row * (D / 2);
        if constexpr (DPL == 2) {
            codes[lane] = (uint8_t)(c[0] | (c[1] << 4));
        } else {
            const uint32_t hi = (uint32_t)__shfl_xor((int)c[0], 1, kWave);
            if ((lane & 1) == 0) codes[lane >> 1] = (uint8_t)(c[0] | (hi << 4));
        }
        if (lane % LPG == 0)
            static_cast<uint8_t *>(kc_scale)[out_row * (D / 32) + lane / LPG] = (uint8_t)(X + 127);
    } else if constexpr (KC == 0) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            static_cast<float *>(kc)[o + e] = m[e];
            dec[e] = m[e];
        }
    } else if constexpr (KC == 1) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            const uint32_t bits = f32_to_bf16_bits(m[e]);
            static_cast<uint16_t *>(kc)[o + e] = (uint16_t)bits;
            dec[e] = bf16_to_f32((uint16_t)bits);
        }
    } else {
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) amax = fmaxf(amax, fabsf(m[e]));
        amax = wave_max_f32(amax);             // DPP steps, no LDS round trips (max is exact in any order)
        const float scale = amax / 448.0f;    // correctly rounded division
        if (lane == 0) static_cast<float *>(kc_scale)[out_row] = scale;
        sc = scale;
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            uint32_t c = 0;
            if (scale != 0.0f) {
                float y = m[e] / scale;
                y = fminf(fmaxf(y, -448.0f), 448.0f);
                c = f32_to_e4m3(y);
            }
            static_cast<uint8_t *>(kc)[o + e] = (uint8_t)c;
            dec[e] = e4m3x2_to_f32<false>(c).x;
        }
    }
}

template <int KC, int DPL>
__device__ __forceinline__ void store_kc(const float (&m)[DPL], void *__restrict__ kc,
                                         void *__restrict__ kc_scale, int64_t out_row, int lane) {
    float dec[DPL], sc;
    store_kc<KC, DPL>(m, kc, kc_scale, out_row, lane, dec, sc);
}

// The values of a stored compressed-key row as the scorer widens them (this
// lane's DPL dims; sc = the e4m3 row scale, else 1).
template <int KC, int DPL>
__device__ __forceinline__ void load_kc_values(const void *__restrict__ kc, const void *__restrict__ kc_scale,
                                               int64_t row, int lane, float (&dec)[DPL], float &sc) {
    constexpr int D = DPL * kWave;
    sc = 1.0f;
    if constexpr (KC == 3) {
        const uint8_t *codes = static_cast<const uint8_t *>(kc) + row * (D / 2);
        const uint32_t E = static_cast<const uint8_t *>(kc_scale)[row * (D / 32) + lane * DPL / 32];
        const float scl = __uint_as_float(E ? (E << 23) : 0x00400000u);
        const uint32_t byte = codes[lane * DPL / 2];
        const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, scl, 0);
        if constexpr (DPL == 2) {
            dec[0] = v[0];
            dec[1] = v[1];
        } else {
            dec[0] = (lane & 1) ? v[1] : v[0];
        }
    } else if constexpr (KC == 2) {
        sc = static_cast<const float *>(kc_scale)[row];
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            dec[e] = e4m3x2_to_f32<false>(static_cast<const uint8_t *>(kc)[row * D + lane * DPL + e]).x;
    } else if constexpr (KC == 1) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) dec[e] = bf16_to_f32(static_cast<const uint16_t *>(kc)[row * D + lane * DPL + e]);
    } else {
#pragma unroll
        for (int e = 0; e < DPL; ++e) dec[e] = static_cast<const float *>(kc)[row * D + lane * DPL + e];
    }
}

}  // namespace qsa
