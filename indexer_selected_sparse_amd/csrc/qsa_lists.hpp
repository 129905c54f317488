// Per-chunk candidate lists that the canonical scorer writes for the block
// top-k of few-row (decode) batches.
//
// Every wave of the scorer holds the scores of one chunk of 64 consecutive
// blocks of a query row.  Besides the scores it writes the chunk's best
// list_len(nb, K) blocks by (score desc, index asc) — their order keys and
// lanes, in ascending block order, padded with key 0 (below every real key)
// — and, when the chunk held more blocks than that, the key of its last
// listed block (the cutoff; 0 when the list holds the whole chunk).  The
// lists of a row, chunk after chunk, are therefore in ascending block order.
//
// The finish kernel selects from the lists alone when that is provably the
// same as selecting from the whole row: with T the K-th largest listed key,
// if T > 0 and every cutoff is strictly below T, then every block with key
// >= T is listed (an unlisted block has key <= its chunk's cutoff < T), so T
// and the lowest-index blocks among the keys equal to T are exactly those
// of the whole row.  Otherwise it selects from the whole row.
//
// With the append inside the scoring launch, the block a row's newest token
// completes is scored by the append, not by its chunk's wave.  That chunk
// then lists one block fewer (its cutoff is the (kk-1)-th largest key of its
// other blocks) and leaves its last slot, which is the row's last list entry,
// to the selection, which fills it from the score row: every unlisted block
// is still bounded by its chunk's cutoff, and the new block is listed.  The
// scorer records which form it wrote in one device word (`mode`).
//
// list_len: m = ceil(64 K / nb) is the expected number of selected blocks in
// a chunk (scores without locality); the list keeps m + 4 ceil(sqrt(m)) + 3,
// at most 64, so for independent scores a chunk overflows its list with a
// probability of order 1e-6 (Poisson tail), and the row falls back.
#pragma once

#include <stdint.h>

#include "qsa_device.hpp"

namespace qsa {

constexpr int kListChunk = 64;                 // blocks per chunk (one scorer wave)
static_assert(kListChunk == 64, "a chunk is one wave");
constexpr int64_t kListMaxEntries = 16384;     // listed entries a row may have (finish holds them in LDS)

// (32-bit arithmetic: nb <= 131072 and K <= 2048.)
__host__ __device__ inline int list_len(int64_t nb, int K) {
    const uint32_t n = (uint32_t)nb;
    const uint32_t m = (kListChunk * (uint32_t)K + n - 1u) / n;
    uint32_t s = 0;
    while (s * s < m) ++s;
    const uint32_t k = m + 4u * s + 3u;
    return k > (uint32_t)kListChunk ? kListChunk : (int)k;
}

// The most entries one row's lists can hold over rows of at most nb_max
// blocks (rows of at most K blocks list nothing).  ceil(nb / 64) *
// list_len(nb, K) is not monotone in nb, but list_len depends on nb only
// through m = ceil(64 K / nb), which for nb > K takes the values 1 .. 64;
// within one value of m the count is largest at the largest nb.
inline int64_t list_max_entries(int64_t nb_max, int K) {
    if (K <= 0) return 0;
    const int64_t t = (int64_t)kListChunk * K;
    int64_t best = 0;
    for (int64_t m = 1; m <= kListChunk; ++m) {
        // nb with ceil(t / nb) == m: t / m <= nb < t / (m - 1)
        const int64_t lo = (t + m - 1) / m;
        int64_t hi = m == 1 ? nb_max : (t + m - 2) / (m - 1) - 1;
        if (hi > nb_max) hi = nb_max;
        const int64_t first = lo > K ? lo : (int64_t)K + 1;
        if (first > hi) continue;
        const int64_t n = ((hi + kListChunk - 1) / kListChunk) * list_len(hi, K);
        if (n > best) best = n;
    }
    return best;
}

// Lists of one call: row i's entries start at i * stride, its cutoffs at
// i * cstride (one per chunk).  keys == nullptr: no lists.  *mode: 0, or
// kListNewBlockSlot when rows whose newest token completes a block leave
// their last entry to the selection.
constexpr uint32_t kListNewBlockSlot = 1u;
struct ListArgs {
    uint32_t *keys;
    uint8_t *loc;
    uint32_t *cut;
    int64_t stride;
    int64_t cstride;
    int K;
    uint32_t *mode;
};

// Whether the selection of row i (visible length L) must fill its last list
// entry with the block its newest token completed (the lists' mode read from
// the device word).
__host__ __device__ inline bool list_new_block_slot(uint32_t mode, int64_t L, int log2r) {
    return mode == kListNewBlockSlot && (L & ((int64_t(1) << log2r) - 1)) == 0;
}

// Order-preserving map of a finite float to uint32 (larger float, larger
// key); never 0 for a finite input, which leaves 0 free for padding.
__device__ __forceinline__ uint32_t list_order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t list_lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The wave's list for the chunk whose first block is `chunk0` (a multiple
// of 64) of query row `row` with nb visible blocks: lane l holds block
// chunk0 + l, its score s and whether it is listed (`active`).  `reserve`:
// the chunk holds the block the append scores; list one block fewer and pad
// the last slot.
__device__ __forceinline__ void emit_chunk_list(const ListArgs &la, int64_t row, int64_t nb, int64_t chunk0,
                                                bool active, float s, int lane, bool reserve = false) {
    if (chunk0 >= nb) return;                                  // uniform over the wave
    const int kk = list_len(nb, la.K);                         // slots per chunk
    const int kc = kk - (reserve ? 1 : 0);                     // entries chosen here
    const uint32_t key = active ? list_order_key(s) : 0u;
    const uint64_t act = __ballot(active);
    uint64_t sel = act;
    uint32_t cut = 0;
    if (__builtin_popcountll(act) > kc) {
        // t = the kc-th largest key: the largest t with #(key >= t) >= kc,
        // two bits per step (three independent counts), MSB first
        uint32_t t = 0;
        for (int bit = 30; bit >= 0; bit -= 2) {
            const uint32_t c3 = t | (3u << bit), c2 = t | (2u << bit), c1 = t | (1u << bit);
            const int n3 = __builtin_popcountll(__ballot(key >= c3));
            const int n2 = __builtin_popcountll(__ballot(key >= c2));
            const int n1 = __builtin_popcountll(__ballot(key >= c1));
            t = n3 >= kc ? c3 : (n2 >= kc ? c2 : (n1 >= kc ? c1 : t));
        }
        const uint64_t gt = __ballot(key > t);
        const uint64_t eq = __ballot(key == t);
        const uint32_t need = (uint32_t)kc - (uint32_t)__builtin_popcountll(gt);
        sel = gt | __ballot(key == t && list_lanes_below(eq) < need);
        cut = t;
    }
    const int64_t base = row * la.stride + (chunk0 >> 6) * kk;
    const int nsel = __builtin_popcountll(sel);
    if ((sel >> lane) & 1u) {                                 // slots 0 .. nsel-1
        const uint32_t pos = list_lanes_below(sel);
        la.keys[base + pos] = key;
        la.loc[base + pos] = (uint8_t)lane;
    }
    if (lane >= nsel && lane < kk) {                          // padding: slots nsel .. kk-1
        la.keys[base + lane] = 0u;
        la.loc[base + lane] = 0;
    }
    if (lane == 0) la.cut[row * la.cstride + (chunk0 >> 6)] = cut;
}

}  // namespace qsa
