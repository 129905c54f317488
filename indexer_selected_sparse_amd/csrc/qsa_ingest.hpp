// One-token append of the per-step ingest, shared by the ingest kernel and
// the fused append + score kernel: ring and K/V argument blocks, and the body
// that appends one sequence's new token (raw key into the ring, K/V rows,
// the block it completes compressed with the batch pass's arithmetic, the
// slot's window and status).  See qsa_ingest.hip for the rules.
#pragma once

#include "qsa_device.hpp"
#include "qsa_kc.hpp"

namespace qsa {

struct RingArgs {
    void *keys;
    int64_t *window;
    const int32_t *slots;
    int64_t num_slots;
    int64_t cap;
};

struct KvArgs {
    const uint8_t *k_new, *v_new;
    uint8_t *k, *v;
    int row_bytes;   // 0: no K/V append
};

// One row of `bytes` (a multiple of 16) copied by one wave, 16 bytes per lane.
__device__ __forceinline__ void copy_row(uint8_t *__restrict__ dst, const uint8_t *__restrict__ src,
                                         int bytes, int lane) {
    for (int c = lane * 16; c < bytes; c += kWave * 16)
        *reinterpret_cast<uint4 *>(dst + c) = *reinterpret_cast<const uint4 *>(src + c);
}

// p mod cap for a position p >= 0 (32-bit division when it fits)
__device__ __forceinline__ int64_t pos_mod(int64_t p, int64_t cap) {
    return p <= 0x7fffffffLL ? (int64_t)((uint32_t)p % (uint32_t)cap) : p % cap;
}

constexpr int kKvChunks = 4;       // 16-byte K/V row pieces a lane holds (rows up to 4 KB)
constexpr int kMaxOldRows = 7;     // old raw keys read together (ratio up to 8)

// One new token per sequence (a decode step), one wave: straight line.  Everything that does not depend on the length is requested first
// (offsets, slot and window, the new raw key, the new K/V rows); then the one
// block-table entry the token and its block share, and the ring rows of the
// block's older tokens; then every store.
// What a one-token append did to the block its token completes.
template <int DPL>
struct AppendOut {
    bool complete = false;   // the token completes block g = N/ratio - 1
    bool stored = false;     // and this append wrote that block's compressed key
    int64_t kc_row = 0;      // kc row of block g (valid when complete)
    float dec[DPL];          // stored: the key's values as the scorer widens them
    float sc = 1.0f;         // stored e4m3: the row scale
};

template <typename TIn, int DPL, int KC>
__device__ __forceinline__ AppendOut<DPL> append_one(
    const TIn *__restrict__ k_new, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ blk_off, int s, int log2r, float inv_ratio, const RingArgs &ring,
    void *__restrict__ kc, void *__restrict__ kc_scale, const KvArgs &kv, int32_t *__restrict__ status,
    const PageMap &pm, int lane) {
    constexpr int D = DPL * kWave;
    constexpr int kKeyChunks = D * (int)sizeof(TIn) / 16;
    AppendOut<DPL> out;

    const int64_t row0 = kv_off[s];
    const int64_t N = kv_off[s + 1] - row0;
    const int64_t blk0 = pm.table ? 0 : blk_off[s];
    const int slot = ring.slots ? ring.slots[s] : s;
    const TIn *key = k_new + (int64_t)s * D;
    uint4 kraw = {0, 0, 0, 0};
    if (lane < kKeyChunks) kraw = reinterpret_cast<const uint4 *>(key)[lane];
    float xn[DPL];
    load_row<TIn, DPL>(key + lane * DPL, xn);
    const bool kv_regs = kv.row_bytes > 0 && kv.row_bytes <= kKvChunks * kWave * 16;
    uint4 kk[kKvChunks], vv[kKvChunks];
    if (kv_regs) {
#pragma unroll
        for (int i = 0; i < kKvChunks; ++i) {
            const int c = (i * kWave + lane) * 16;
            if (c < kv.row_bytes) {
                kk[i] = *reinterpret_cast<const uint4 *>(kv.k_new + (int64_t)s * kv.row_bytes + c);
                vv[i] = *reinterpret_cast<const uint4 *>(kv.v_new + (int64_t)s * kv.row_bytes + c);
            }
        }
    }
    const bool slot_ok = slot >= 0 && slot < ring.num_slots;
    int64_t lo = 0, hi = 0;
    if (slot_ok) {
        lo = ring.window[2 * (int64_t)slot];
        hi = ring.window[2 * (int64_t)slot + 1];
    }
    int code = QSA_INGEST_OK;
    if (!slot_ok) code = QSA_INGEST_BAD_SLOT;
    else if (N < 1 || (pm.table && N > (pm.stride << pm.log2_page))) code = QSA_INGEST_TOO_LONG;
    const int ratio = 1 << log2r;
    const int64_t p = N - 1;                         // the new token's position
    const int64_t g = p >> log2r;
    // the block the token completes, even when nothing is appended (its key
    // is then the one already stored)
    const bool in_table = N >= 1 && (!pm.table || N <= (pm.stride << pm.log2_page));
    out.complete = in_table && (N & (ratio - 1)) == 0;
    int64_t dst = row0 + p, kc_row = blk0 + g;
    if (pm.table && in_table) {   // a page holds whole blocks: one entry maps the token and its block
        const int64_t page = pm.table[s * pm.stride + (p >> pm.log2_page)];
        dst = (page << pm.log2_page) | (p & ((int64_t(1) << pm.log2_page) - 1));
        const int lb = pm.log2_page - log2r;
        kc_row = (page << lb) | (g & ((int64_t(1) << lb) - 1));
    }
    out.kc_row = kc_row;
    if (code != QSA_INGEST_OK) {
        if (lane == 0 && status) status[s] = code;
        return out;
    }

    const int64_t cap = ring.cap;
    TIn *const rkeys = static_cast<TIn *>(ring.keys) + (int64_t)slot * cap * D;
    const bool complete = out.complete;
    const int64_t lo_eff = p <= hi ? (lo < p ? lo : p) : p;
    const int64_t b0 = N - ratio;                    // first position of the completed block
    const bool lost = complete && lo_eff > b0;
    float m[DPL];
    if (complete && !lost) {
        float acc[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
        if (ratio - 1 <= kMaxOldRows) {
            float xs[kMaxOldRows][DPL];
#pragma unroll
            for (int j = 0; j < kMaxOldRows; ++j)
                if (j < ratio - 1) load_row<TIn, DPL>(rkeys + pos_mod(b0 + j, cap) * D + lane * DPL, xs[j]);
#pragma unroll
            for (int j = 0; j < kMaxOldRows; ++j)
                if (j < ratio - 1) {
#pragma unroll
                    for (int e = 0; e < DPL; ++e) acc[e] = acc[e] + xs[j][e];
                }
        } else {
            for (int j = 0; j < ratio - 1; ++j) {
                float x[DPL];
                load_row<TIn, DPL>(rkeys + pos_mod(b0 + j, cap) * D + lane * DPL, x);
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[e] = acc[e] + x[e];
            }
        }
#pragma unroll
        for (int e = 0; e < DPL; ++e) m[e] = (acc[e] + xn[e]) * inv_ratio;
    }

    // stores (the ring row of p is not one the block reads: cap >= ratio)
    if (lane < kKeyChunks)
        reinterpret_cast<uint4 *>(rkeys + pos_mod(p, cap) * D)[lane] = kraw;
    if (kv_regs) {
#pragma unroll
        for (int i = 0; i < kKvChunks; ++i) {
            const int c = (i * kWave + lane) * 16;
            if (c < kv.row_bytes) {
                *reinterpret_cast<uint4 *>(kv.k + dst * kv.row_bytes + c) = kk[i];
                *reinterpret_cast<uint4 *>(kv.v + dst * kv.row_bytes + c) = vv[i];
            }
        }
    } else if (kv.row_bytes) {
        copy_row(kv.k + dst * kv.row_bytes, kv.k_new + (int64_t)s * kv.row_bytes, kv.row_bytes, lane);
        copy_row(kv.v + dst * kv.row_bytes, kv.v_new + (int64_t)s * kv.row_bytes, kv.row_bytes, lane);
    }
    if (complete && !lost) {
        store_kc<KC, DPL>(m, kc, kc_scale, kc_row, lane, out.dec, out.sc);
        out.stored = true;
    }
    if (lane == 0) {
        int64_t *const win = ring.window + 2 * (int64_t)slot;
        win[0] = lo_eff > N - cap ? lo_eff : N - cap;
        win[1] = N;
        if (status) status[s] = lost ? QSA_INGEST_LOST_KEYS : QSA_INGEST_OK;
    }
    return out;
}


}  // namespace qsa
