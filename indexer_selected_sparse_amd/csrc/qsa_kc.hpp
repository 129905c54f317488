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

// KC: 0 = fp32, 1 = bf16 (round to nearest even), 2 = e4m3 + fp32 scale.
// m = this lane's DPL means; the whole wave must call it (e4m3 reduces amax
// over the wave).
template <int KC, int DPL>
__device__ __forceinline__ void store_kc(const float (&m)[DPL], void *__restrict__ kc,
                                         float *__restrict__ kc_scale, int64_t out_row, int lane) {
    constexpr int D = DPL * kWave;
    const int64_t o = out_row * D + lane * DPL;
    if constexpr (KC == 0) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) static_cast<float *>(kc)[o + e] = m[e];
    } else if constexpr (KC == 1) {
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            static_cast<uint16_t *>(kc)[o + e] = (uint16_t)f32_to_bf16_bits(m[e]);
    } else {
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) amax = fmaxf(amax, fabsf(m[e]));
        amax = wave_max(amax);
        const float scale = amax / 448.0f;    // correctly rounded division
        if (lane == 0) kc_scale[out_row] = scale;
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            uint32_t c = 0;
            if (scale != 0.0f) {
                float y = m[e] / scale;
                y = fminf(fmaxf(y, -448.0f), 448.0f);
                c = f32_to_e4m3(y);
            }
            static_cast<uint8_t *>(kc)[o + e] = (uint8_t)c;
        }
    }
}

}  // namespace qsa
