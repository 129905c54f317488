// Sparse gather attention over the selected blocks plus the tail, decode and
// prefill/verify ("Agentic shootout" page: vLLM report section (a)6 — GQA
// attention over the expanded selection, -1 padded; "llama.cpp vs Atlas"
// section (a)3 — the incomplete tail block is always visible; "llama.cpp vs
// Atlas" #2, risks — top-k gather attention performance is the unknown).
//
// For query i with visible length L, nb = floor(L/ratio) complete blocks and
// nsel = min(K, nb) selected blocks (idx row, ascending, -1 padding after
// nsel), the token set is T = {idx[s]*ratio + j : s < nsel, j < ratio} plus
// the tail ratio*nb .. L-1.  In the dense regime (nb <= K) idx lists every
// complete block, so T = 0..L-1 and the result is dense causal attention.
//
// Work decomposition: a query's selected slots are cut into n_part parts (the
// last part also owns the tail); one wave per (query, part, KV head), and the
// waves of a workgroup are consecutive KV heads of the same (query, part), so
// a workgroup reads whole token rows (all heads) contiguously.  With more than
// one part (decode) each wave writes an unnormalised (m, l, o) partial and a
// small combine kernel finishes.  The part count depends only on budget/ratio
// (decode) or is 1 (prefill), so a query's arithmetic never depends on the
// rest of the batch.
//
// The G = hq/hkv query heads of the KV head share every K/V load.  Tokens are
// processed 16 per step, the next step's K/V loads in flight meanwhile:
//  * QK: lane (tk = lane/8, ds = lane%8) loads dims ds*16..+16 of tokens tk
//    and tk+8 straight from HBM and forms partial dots for all G heads with
//    v_dot2_f32_bf16 (query slices come from LDS).  The heads are laid out in
//    a per-lane order chosen so that a 3-step transpose-reduce over the 8 ds
//    lanes is three DPP adds per kept value (each lane keeps its first half
//    and adds the partner's second half); every lane ends with the full dots
//    of G/8 heads.
//  * online softmax in fp32 (exp2 domain), one running max per head; the max
//    over the 8 token lanes uses DPP and the gfx950 permlane swaps.
//  * PV: lane p owns dims 2p, 2p+1 of every head; V rows are read as one
//    coalesced row per token from a scalar base address; fp32 probabilities
//    come through LDS and meet fp32-widened V in plain FMAs.  (bf16
//    probabilities would cost up to 2^-8 relative per weight, visible when a
//    few tokens carry the softmax.)
#include <atomic>
#include <mutex>

#include "qsa_device.hpp"
#include "qsa_internal.hpp"
#include "qsa_lists.hpp"

namespace qsa {
namespace {

constexpr int kD = 128;
constexpr int kWgWaves = 4;             // waves (parts) per workgroup
constexpr int kStep = 16;               // tokens per step
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
    const void *q, *k, *v;
    const int32_t *idx;
    const int64_t *kv_off, *q_off;
    int num_seqs, hq, hkv, log2r, K;
    int n_part;              // parts per query
    float c;                 // softmax_scale * log2(e)
    int64_t total_q;
    void *out;
    float *ws_o;             // [total_q, hq, n_part, D]
    float *ws_ml;            // [total_q, hq, n_part, 2]
    PageMap pm;              // paged K/V pools (pm.table == nullptr: contiguous)
    // selection inside the decode kernel (qsa_decode_step): the scorer's
    // candidate lists, the score rows (exact fallback) and the idx rows the
    // workgroups of KV head 0, part 0 write
    ListArgs la;
    const float *scores;
    int64_t ld;
    int32_t *idx_out;
    int32_t sel_pref;        // list entries a row can hold at most (requested up front)
};

// Several layers that share one selection in one launch (blockIdx.y = layer):
// each layer's q, k, v, out and its own slice of the partials workspace.
constexpr int kMaxLayers = QSA_MAX_LAYERS;
struct LayerPtrs {
    const void *q[kMaxLayers], *k[kMaxLayers], *v[kMaxLayers];
    void *out[kMaxLayers];
    float c[kMaxLayers];     // softmax_scale * log2(e) of each layer
    int64_t ws_stride;       // floats between the layers' workspace slices
};

template <int G>
constexpr int ilog2() { return G <= 1 ? 0 : 1 + ilog2<G / 2>(); }

// ---------------------------------------------------------- cross-lane ops
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xf, 0xf, false);
}
constexpr int kDppHalfMirror = 0x141;   // lane ^ 7 within 8
constexpr int kDppXor2 = 0x4e;          // quad_perm [2,3,0,1]
constexpr int kDppXor1 = 0xb1;          // quad_perm [1,0,3,2]
constexpr int kDppRor8 = 0x128;         // lane ^ 8 within 16

// max / sum over the 8 lanes {l ^ 8k}: same ds, all token slots
__device__ __forceinline__ float tok_max(float x) {
    x = fmaxf(x, dpp<kDppRor8>(x));
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float tok_sum(float x) {
    x = x + dpp<kDppRor8>(x);
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Head held in partial-sum slot j of lane ds (G >= 8, unit U = G/8): the
// order makes each transpose step "keep my first half, add my partner's
// second half" — partners are ds^7, ds^2, ds^1 in turn, and the unit map
// {0,1,2,3,7,6,5,4} satisfies gp(u+4) = gp(u)^7, gp(u+2) = gp(u)^2 (u < 2),
// gp(1) = gp(0)^1.  Lane ds ends with heads U*ds .. U*ds+U-1.
__device__ __forceinline__ int slot_head(int j, int ds, int U) {
    constexpr int gp[8] = {0, 1, 2, 3, 7, 6, 5, 4};
    return U * (ds ^ gp[j / U]) + (j % U);
}

template <int G>
__device__ __forceinline__ void transpose_reduce(const float (&p)[G], float (&r)[(G >= 8 ? G / 8 : 1)],
                                                 int ds) {
    if constexpr (G >= 8) {
        float a4[G / 2], a2[G / 4];
#pragma unroll
        for (int j = 0; j < G / 2; ++j) a4[j] = p[j] + dpp<kDppHalfMirror>(p[G / 2 + j]);
#pragma unroll
        for (int j = 0; j < G / 4; ++j) a2[j] = a4[j] + dpp<kDppXor2>(a4[G / 4 + j]);
#pragma unroll
        for (int j = 0; j < G / 8; ++j) r[j] = a2[j] + dpp<kDppXor1>(a2[G / 8 + j]);
    } else {
        // G < 8: natural head order; keep the half selected by the lane's bit
        float a[G];
#pragma unroll
        for (int h = 0; h < G; ++h) a[h] = p[h];
        int n = G;
        const int masks[3] = {4, 2, 1};
#pragma unroll
        for (int st = 0; st < 3; ++st) {
            const int m = masks[st];
            const bool upper = ds & m;
            if (n > 1) {
#pragma unroll
                for (int j = 0; j < G / 2; ++j) {
                    if (j < n / 2) {
                        const float mine = upper ? a[n / 2 + j] : a[j];
                        const float send = upper ? a[j] : a[n / 2 + j];
                        a[j] = mine + __shfl_xor(send, m, kWave);
                    }
                }
                n /= 2;
            } else {
                a[0] = a[0] + __shfl_xor(a[0], m, kWave);
            }
        }
        r[0] = a[0];
    }
}

template <int G>
__device__ __forceinline__ int head_base(int ds) {
    if constexpr (G >= 8) return ds * (G / 8);
    else return ds >> (3 - ilog2<G>());
}

// Head of partial-sum slot j for lane ds.
template <int G>
__device__ __forceinline__ int qk_head(int j, int ds) {
    if constexpr (G >= 8) return slot_head(j, ds, G / 8);
    else return j;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool BF16>
struct KVTypes;
template <>
struct KVTypes<true> {
    using elem = uint16_t;
    static constexpr int kDwordsPerLaneK = 8;   // 16 bf16 dims
    static constexpr int kDwordsPerLaneV = 1;   // 2 bf16 dims
};
template <>
struct KVTypes<false> {
    using elem = float;
    static constexpr int kDwordsPerLaneK = 16;  // 16 fp32 dims
    static constexpr int kDwordsPerLaneV = 2;   // 2 fp32 dims
};

// Registers of one 16-token step: the K slices of this lane's two QK tokens,
// the V dims of every token, and which tokens exist.
template <bool BF16>
struct StepBuf {
    static constexpr int KW = KVTypes<BF16>::kDwordsPerLaneK;
    static constexpr int VW = KVTypes<BF16>::kDwordsPerLaneV;
    uint32_t kA[KW], kB[KW];
    uint32_t v[kStep][VW];
    uint32_t valid;          // wave-uniform bit mask over the 16 tokens
};

// Wave-uniform description of the tokens one wave processes.
struct WaveWork {
    const int32_t *__restrict__ sel;  // idx row + first slot of this part
    int nslot;                        // selected slots of the part
    int nblk_tok;                     // tokens from selected blocks
    int ntok;                         // + tail tokens
    int64_t tail0;                    // first tail position (ratio * nb)
    int64_t nb;                       // complete blocks visible to the query
    int log2r;
};

// A selected block id as the table holds it for the kernels: with paged K/V
// the physical block of the pool (a page holds whole blocks), -1 for an id
// outside [0, nb) (which the kernels then treat as "no token").
__device__ __forceinline__ int slot_phys(int b, const PageMap &pm, int64_t seq, int64_t nb, int log2r) {
    if (pm.table == nullptr) return b;
    if (b < 0 || (int64_t)b >= nb) return -1;
    return (int)paged_row(pm, seq, b, pm.log2_page - log2r);
}
// Paged pools: the tail's first pool row, and no logical bound on block ids
// (they were checked when translated).
__device__ __forceinline__ void page_wave(WaveWork &W, const PageMap &pm, int64_t seq, int64_t L) {
    if (pm.table == nullptr) return;
    W.tail0 = L > W.tail0 ? paged_row(pm, seq, W.tail0, pm.log2_page) : 0;
    W.nb = int64_t(1) << 62;
}

// Issue the loads of step `st`.  Lane t < 16 resolves token 16*st+t to a row
// of the sequence (a selected block id from the slot table, one slot per
// lane, or a tail position; malformed ids and positions past the end give "no
// token" and read row 0).  K rows reach the QK lanes by a cross-lane permute
// (with every lane active); V rows become wave-uniform addresses, so each V
// row is one coalesced load from a scalar base.
template <bool BF16>
__device__ __forceinline__ void issue_step(const WaveWork &W, int st, int lane, int tk, int ds,
                                           uint32_t slot_tab, int tab_base,
                                           const typename KVTypes<BF16>::elem *__restrict__ kbase,
                                           const typename KVTypes<BF16>::elem *__restrict__ vbase,
                                           int64_t row_stride, StepBuf<BF16> &B) {
    using T = typename KVTypes<BF16>::elem;
    constexpr int KW = StepBuf<BF16>::KW;
    const int t = st * kStep + (lane & (kStep - 1));
    int rel = (t >> W.log2r) - tab_base;             // slot within the table
    rel = rel < 0 ? 0 : (rel > kWave - 1 ? kWave - 1 : rel);
    const int b = __builtin_amdgcn_ds_bpermute(rel << 2, (int)slot_tab);
    int row = 0;
    bool ok = false;
    if (t < W.nblk_tok) {
        ok = b >= 0 && (int64_t)b < W.nb;
        row = ok ? (b << W.log2r) + (t & ((1 << W.log2r) - 1)) : 0;
    } else if (t < W.ntok) {
        row = (int)(W.tail0 + (t - W.nblk_tok));
        ok = true;
    }
    const uint64_t okm = __ballot(ok && lane < kStep);
    B.valid = (uint32_t)okm & 0xffffu;
    const int rA = __builtin_amdgcn_ds_bpermute(tk << 2, row);
    const int rB = __builtin_amdgcn_ds_bpermute((tk + 8) << 2, row);
    {
        const uint4 *sa = reinterpret_cast<const uint4 *>(kbase + (int64_t)rA * row_stride + ds * 16);
        const uint4 *sb = reinterpret_cast<const uint4 *>(kbase + (int64_t)rB * row_stride + ds * 16);
#pragma unroll
        for (int c4 = 0; c4 < KW / 4; ++c4) {
            const uint4 x = sa[c4], y = sb[c4];
            B.kA[4 * c4 + 0] = x.x; B.kA[4 * c4 + 1] = x.y; B.kA[4 * c4 + 2] = x.z; B.kA[4 * c4 + 3] = x.w;
            B.kB[4 * c4 + 0] = y.x; B.kB[4 * c4 + 1] = y.y; B.kB[4 * c4 + 2] = y.z; B.kB[4 * c4 + 3] = y.w;
        }
    }
#pragma unroll
    for (int tt = 0; tt < kStep; ++tt) {
        const int r = __builtin_amdgcn_readlane(row, tt);
        const T *src = vbase + (int64_t)r * row_stride;
        if constexpr (BF16) {
            B.v[tt][0] = reinterpret_cast<const uint32_t *>(src)[lane];
        } else {
            const uint2 x = reinterpret_cast<const uint2 *>(src)[lane];
            B.v[tt][0] = x.x;
            B.v[tt][1] = x.y;
        }
    }
}

template <int G>
struct AttnState {
    static constexpr int NH = G >= 8 ? G / 8 : 1;
    float m_run[NH], l_run[NH];
    float o[G][2];
};

// This lane's query slices for the QK mapping: slot j holds dims ds*16..+16
// of head qk_head(j, ds), as dwords (bf16 pairs or fp32).
template <bool BF16, int G>
struct QSlices {
    uint32_t v[G][KVTypes<BF16>::kDwordsPerLaneK];
};

// Consume one step: QK, online softmax, PV.
template <bool BF16, int G>
__device__ __forceinline__ void compute_step(const StepBuf<BF16> &B, const QSlices<BF16, G> &Q,
                                             float c, int tk, int ds, int hb,
                                             float (*sh_p)[G], float *sh_alpha, AttnState<G> &S) {
    constexpr int NH = AttnState<G>::NH;
    constexpr int KW = KVTypes<BF16>::kDwordsPerLaneK;
    // ---- QK partial dots over this lane's 16 dims, heads in slot order
    float dA[G], dB[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const uint32_t (&qv)[KW] = Q.v[j];
        float a = 0.0f, b = 0.0f;
        if constexpr (BF16) {
            typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int e = 0; e < KW; ++e) {
                const bf2 qq = __builtin_bit_cast(bf2, qv[e]);
                a = __builtin_amdgcn_fdot2_f32_bf16(qq, __builtin_bit_cast(bf2, B.kA[e]), a, false);
                b = __builtin_amdgcn_fdot2_f32_bf16(qq, __builtin_bit_cast(bf2, B.kB[e]), b, false);
            }
        } else {
#pragma unroll
            for (int e = 0; e < KW; ++e) {
                const float qq = __uint_as_float(qv[e]);
                a = __builtin_fmaf(qq, __uint_as_float(B.kA[e]), a);
                b = __builtin_fmaf(qq, __uint_as_float(B.kB[e]), b);
            }
        }
        dA[j] = a;
        dB[j] = b;
    }
    float sA[NH], sB[NH];
    transpose_reduce<G>(dA, sA, ds);
    transpose_reduce<G>(dB, sB, ds);

    // ---- online softmax (exp2 domain), one running max per head
    const bool okA = (B.valid >> tk) & 1u, okB = (B.valid >> (tk + 8)) & 1u;
    bool rescale = false;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const float xa = okA ? sA[h] * c : -INFINITY;
        const float xb = okB ? sB[h] * c : -INFINITY;
        const float mx = tok_max(fmaxf(xa, xb));
        const float m_new = fmaxf(S.m_run[h], mx);
        const float m_safe = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = exp2f(S.m_run[h] - m_safe);
        rescale |= m_new != S.m_run[h];
        const float ea = exp2f(xa - m_safe), eb = exp2f(xb - m_safe);
        S.m_run[h] = m_new;
        sh_p[tk][hb + h] = ea;
        sh_p[tk + 8][hb + h] = eb;
        S.l_run[h] = S.l_run[h] * alpha + (ea + eb);
        if (tk == 0) sh_alpha[hb + h] = alpha;
    }
    const bool any_rescale = __ballot(rescale) != 0;
    wave_lds_sync();

    // ---- PV: lane owns dims 2*lane, 2*lane+1 of every head
    if (any_rescale) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float al = sh_alpha[h];
            S.o[h][0] *= al;
            S.o[h][1] *= al;
        }
    }
#pragma unroll
    for (int tt = 0; tt < kStep; ++tt) {
        float v0, v1;
        if constexpr (BF16) {
            v0 = bf16lo(B.v[tt][0]);
            v1 = bf16hi(B.v[tt][0]);
        } else {
            v0 = __uint_as_float(B.v[tt][0]);
            v1 = __uint_as_float(B.v[tt][1]);
        }
        float pv[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pv[h] = sh_p[tt][h];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            S.o[h][0] = __builtin_fmaf(pv[h], v0, S.o[h][0]);
            S.o[h][1] = __builtin_fmaf(pv[h], v1, S.o[h][1]);
        }
    }
    // Likewise keep each token's probability reads next to its FMAs (reading
    // all 16 x G probabilities up front would hold 16*G registers).
#pragma unroll
    for (int tt = 0; tt < kStep; ++tt) {
        __builtin_amdgcn_sched_group_barrier(0x100, G >= 4 ? G / 4 : 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2 * G + (BF16 ? 2 : 0), 0);
    }
    wave_lds_sync();
}

template <int G>
struct AttnLds {
    // 16-byte aligned rows so a token's probabilities load as ds_read_b128
    alignas(16) float p[kWgWaves][kStep][G];   // probabilities [token][head], per wave
    alignas(16) float alpha[kWgWaves][G];
    alignas(16) float l[kWgWaves][G];
    alignas(16) float m[kWgWaves][G];
};

template <bool BF16, int G>
__device__ __forceinline__ void attn_body(const AttnArgs &A) {
    using T = typename KVTypes<BF16>::elem;
    constexpr int NH = AttnState<G>::NH;
    __shared__ __align__(16) AttnLds<G> L;

    const int lane = threadIdx.x & (kWave - 1);
    // The wave index is uniform across the wave; saying so keeps everything
    // derived from it (part, positions) in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t wid = (int64_t)blockIdx.x * kWgWaves + wave;
    const int g = (int)(wid % A.hkv);
    const int64_t t2 = wid / A.hkv;
    const int c = (int)(t2 % A.n_part);              // part of this wave
    const int64_t i = t2 / A.n_part;
    if (i >= A.total_q) return;                      // uniform over the wave

    const QueryPos qp = query_pos(A.kv_off, nullptr, A.q_off, A.num_seqs, i);
    const int64_t nb = qp.L >> A.log2r;
    const int64_t nsel = nb < A.K ? nb : (int64_t)A.K;
    const int64_t per = (nsel + A.n_part - 1) / A.n_part;
    const int64_t s_beg = imin64((int64_t)c * per, nsel);
    const int64_t s_end = imin64(s_beg + per, nsel);
    WaveWork W;
    W.sel = A.idx + i * (int64_t)A.K + s_beg;
    W.nslot = (int)(s_end - s_beg);
    W.log2r = A.log2r;
    W.nblk_tok = W.nslot << A.log2r;
    W.tail0 = nb << A.log2r;
    W.nb = nb;
    W.ntok = W.nblk_tok + ((c == A.n_part - 1) ? (int)(qp.L - W.tail0) : 0);
    page_wave(W, A.pm, qp.seq, qp.L);
    const int64_t row0 = A.pm.table ? 0 : qp.kv_row0;     // rows are pool rows when paged

    const int tk = lane >> 3, ds = lane & 7;
    const int hb = head_base<G>(ds);
    const int qh0 = g * G;                          // first query head of this KV head
    const int64_t row_stride = (int64_t)A.hkv * kD; // elements between consecutive tokens
    const T *__restrict__ kbase = static_cast<const T *>(A.k) + (row0 * A.hkv + g) * kD;
    const T *__restrict__ vbase = static_cast<const T *>(A.v) + (row0 * A.hkv + g) * kD;

    // query slices for the QK mapping (kept in registers for the whole part)
    QSlices<BF16, G> Q;
    {
        constexpr int KW = KVTypes<BF16>::kDwordsPerLaneK;
        const T *qrow = static_cast<const T *>(A.q) + (i * A.hq + qh0) * kD + ds * 16;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const uint4 *src = reinterpret_cast<const uint4 *>(qrow + qk_head<G>(j, ds) * kD);
#pragma unroll
            for (int c4 = 0; c4 < KW / 4; ++c4) {
                const uint4 x = src[c4];
                Q.v[j][4 * c4] = x.x; Q.v[j][4 * c4 + 1] = x.y;
                Q.v[j][4 * c4 + 2] = x.z; Q.v[j][4 * c4 + 3] = x.w;
            }
        }
    }

    AttnState<G> S;
#pragma unroll
    for (int h = 0; h < NH; ++h) { S.m_run[h] = -INFINITY; S.l_run[h] = 0.0f; }
#pragma unroll
    for (int h = 0; h < G; ++h) { S.o[h][0] = 0.0f; S.o[h][1] = 0.0f; }

    // Slot table: lane j holds selected block id of slot tab_base + j.
    int tab_base = 0;
    uint32_t slot_tab = (uint32_t)slot_phys(lane < W.nslot ? W.sel[lane] : -1, A.pm, qp.seq, nb, A.log2r);
    const int nsteps = (W.ntok + kStep - 1) / kStep;
    auto ensure_table = [&](int st) {
        const int first = (st * kStep) >> W.log2r;
        const int last = (st * kStep + kStep - 1) >> W.log2r;
        if (st * kStep < W.nblk_tok && (first < tab_base || last >= tab_base + kWave)) {
            tab_base = first;
            slot_tab = (uint32_t)slot_phys(tab_base + lane < W.nslot ? W.sel[tab_base + lane] : -1, A.pm,
                                           qp.seq, nb, A.log2r);
        }
    };

    StepBuf<BF16> b0, b1;
    if (nsteps > 0) {
        ensure_table(0);
        issue_step<BF16>(W, 0, lane, tk, ds, slot_tab, tab_base, kbase, vbase, row_stride, b0);
    }
    for (int st = 0; st < nsteps; st += 2) {
        if (st + 1 < nsteps) {
            ensure_table(st + 1);
            issue_step<BF16>(W, st + 1, lane, tk, ds, slot_tab, tab_base, kbase, vbase, row_stride, b1);
        }
        compute_step<BF16, G>(b0, Q, A.c, tk, ds, hb, L.p[wave], L.alpha[wave], S);
        if (st + 1 >= nsteps) break;
        if (st + 2 < nsteps) {
            ensure_table(st + 2);
            issue_step<BF16>(W, st + 2, lane, tk, ds, slot_tab, tab_base, kbase, vbase, row_stride, b0);
        }
        compute_step<BF16, G>(b1, Q, A.c, tk, ds, hb, L.p[wave], L.alpha[wave], S);
    }

    // ---- denominators over the 8 token lanes; running max per head
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const float l = tok_sum(S.l_run[h]);
        if (tk == 0) {
            L.l[wave][hb + h] = l;
            L.m[wave][hb + h] = S.m_run[h];
        }
    }
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if (A.n_part == 1) {
            const float l = L.l[wave][h];
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            const int64_t off = (i * A.hq + qh0 + h) * kD + 2 * lane;
            if constexpr (BF16) {
                reinterpret_cast<uint32_t *>(A.out)[off >> 1] = pack_bf16x2(S.o[h][0] * inv, S.o[h][1] * inv);
            } else {
                reinterpret_cast<float2 *>(A.out)[off >> 1] = make_float2(S.o[h][0] * inv, S.o[h][1] * inv);
            }
        } else {
            const int64_t slot = (i * A.hq + qh0 + h) * A.n_part + c;
            reinterpret_cast<float2 *>(A.ws_o + slot * kD)[lane] = make_float2(S.o[h][0], S.o[h][1]);
            if (lane == 0) {
                A.ws_ml[slot * 2 + 0] = L.m[wave][h];
                A.ws_ml[slot * 2 + 1] = L.l[wave][h];
            }
        }
    }
}

// bf16 with G <= 4 fits three waves per SIMD (<= 168 VGPRs) without spills;
// the wider variants keep the compiler's default budget.
template <bool BF16, int G>
__global__ __launch_bounds__(kWgWaves * kWave)
__attribute__((amdgpu_waves_per_eu(3))) void attn_kernel_w3(AttnArgs A) {
    attn_body<BF16, G>(A);
}
template <bool BF16, int G>
__global__ __launch_bounds__(kWgWaves * kWave) void attn_kernel(AttnArgs A) {
    attn_body<BF16, G>(A);
}

// ---------------------------------------------------------------------------
// Decode, bf16: K/V staged through a per-wave LDS ring by direct-to-LDS loads.
//
// A gather of scattered 256-byte rows only reaches HBM speed with a great
// deal of data in flight per CU; register double-buffering caps that at two
// steps per wave.  Here every step's K and V tiles (16 tokens x 256 B each)
// are fetched with global_load_lds_dwordx4 straight into a ring of D slots of
// LDS, issued D-1 steps ahead of the step being computed, so a wave keeps
// (D-1) x 8 KB in flight without holding registers for it.  Completion is
// tracked with vmcnt (the loads complete in order), and a slot is refilled
// only after the step that used it has been read back into registers.  The
// arithmetic of a step is the shared compute_step, so decode and prefill
// compute the same operations on the same values.
constexpr int kSlotBytes = 2 * kStep * kD * 2;      // K tile + V tile, bf16: 8 KB

// s_waitcnt immediate meaning "vmcnt <= n", leaving expcnt and lgkmcnt free.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// LDS byte address of a pointer into this workgroup's shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const lds_void_t *)p;
}

// One global_load_lds_dwordx4: lane l's 16 bytes from `src` land at LDS byte
// lds_dst + 16*l.  Issued through inline assembly so that the compiler does
// not treat every later LDS read as dependent on every load still in flight
// (it cannot tell the ring slots apart and would drain the whole ring before
// each read); the kernel orders the ring itself with explicit vmcnt waits.
// M0 carries the LDS destination; nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_dst) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_dst))
                 : "memory", "m0");
}
// The same with a wave-uniform 64-bit base (SGPRs) and a 32-bit byte offset
// per lane, so a row address costs one 32-bit multiply-add.
__device__ __forceinline__ void dma16_off(const void *base, uint32_t off, uint32_t lds_dst) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_dst))
                 : "memory", "m0");
}
#pragma clang diagnostic pop

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Issue the 8 direct-to-LDS loads of step `st` (16 tokens) into the slot at
// LDS address `slot` and return the step's wave-uniform token-valid mask.
// A token's row is resolved from the slot table (up to 128 part slots held in
// two registers: lane j of tab0 / tab1 = block id of part slot j / 64 + j), a
// selected block id giving rows b*ratio.., a tail position giving itself;
// malformed ids and positions past the end give "no token" and read row 0.
// Lanes 0..15 end up holding the rows of tokens 0..15.  Row byte offsets are
// 32-bit (the launcher checks that a sequence's K rows, or the pool's with paged K/V, span less
// than 4 GiB).  Load j covers tokens
// 4j..4j+3: lane l fills LDS bytes l*16.. of the j-th kilobyte (the hardware
// places lane l's 16 bytes at l*16), i.e. position p = l%16 of token
// t = 4j + l/16.  Position p of token t holds the row's 16-byte chunk p ^ t
// (a per-token rotation of the 16 chunks), in the K tile and in the V tile,
// so the matrix-operand reads below hit 16 different LDS bank groups.
__device__ __forceinline__ uint32_t issue_step_lds(const WaveWork &W, int st, int lane,
                                                   uint32_t tab0, uint32_t tab1,
                                                   const uint16_t *__restrict__ kbase,
                                                   const uint16_t *__restrict__ vbase,
                                                   uint32_t row_bytes, uint32_t slot) {
    const int t = st * kStep + (lane & (kStep - 1));
    int rel = t >> W.log2r;                          // slot of the part, < 2 * 64
    rel = rel > 2 * kWave - 1 ? 2 * kWave - 1 : rel;
    const int b0 = __builtin_amdgcn_ds_bpermute((rel & (kWave - 1)) << 2, (int)tab0);
    const int b1 = __builtin_amdgcn_ds_bpermute((rel & (kWave - 1)) << 2, (int)tab1);
    const int b = rel < kWave ? b0 : b1;
    int row = 0;
    bool ok = false;
    if (t < W.nblk_tok) {
        ok = b >= 0 && (int64_t)b < W.nb;
        row = ok ? (b << W.log2r) + (t & ((1 << W.log2r) - 1)) : 0;
    } else if (t < W.ntok) {
        row = (int)(W.tail0 + (t - W.nblk_tok));
        ok = true;
    }
    const uint32_t valid = (uint32_t)__ballot(ok && lane < kStep) & 0xffffu;
    const int p = lane & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tq = 4 * j + (lane >> 4);
        const int r = __builtin_amdgcn_ds_bpermute(tq << 2, row);
        const uint32_t off = (uint32_t)r * row_bytes + (uint32_t)((p ^ tq) << 4);
        dma16_off(kbase, off, slot + j * 1024);
        dma16_off(vbase, off, slot + 4096 + j * 1024);
    }
    return valid;
}

// Slots a wave holds in LDS when its share of a part exceeds the 128 that
// tab0 / tab1 hold (prefill with more than 512 selected blocks, or a decode
// launch with few parts): at most ceil(2048 / 4) (K <= 2048, one part).
constexpr int kBigTabSlots = 2048 / kWgWaves;
constexpr int kBigTabBytes = kBigTabSlots * 4;
typedef __attribute__((address_space(3))) int32_t lds_i32_t;

// issue_step_lds with the wave's slot table in LDS at byte address `tab`
// (up to kBigTabSlots entries; entries past the wave's nslot slots are read
// but not used): each of lanes 0..15 reads the block id of its own token's
// slot.
__device__ __forceinline__ uint32_t issue_step_lds_tab(const WaveWork &W, int st, int lane, uint32_t tab,
                                                       const uint16_t *__restrict__ kbase,
                                                       const uint16_t *__restrict__ vbase,
                                                       uint32_t row_bytes, uint32_t slot) {
    const int t = st * kStep + (lane & (kStep - 1));
    int rel = t >> W.log2r;
    rel = rel > kBigTabSlots - 1 ? kBigTabSlots - 1 : rel;
    const int b = *(const lds_i32_t *)(uintptr_t)(tab + 4u * (uint32_t)rel);
    int row = 0;
    bool ok = false;
    if (t < W.nblk_tok) {
        ok = b >= 0 && (int64_t)b < W.nb;
        row = ok ? (b << W.log2r) + (t & ((1 << W.log2r) - 1)) : 0;
    } else if (t < W.ntok) {
        row = (int)(W.tail0 + (t - W.nblk_tok));
        ok = true;
    }
    const uint32_t valid = (uint32_t)__ballot(ok && lane < kStep) & 0xffffu;
    const int p = lane & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tq = 4 * j + (lane >> 4);
        const int r = __builtin_amdgcn_ds_bpermute(tq << 2, row);
        const uint32_t off = (uint32_t)r * row_bytes + (uint32_t)((p ^ tq) << 4);
        dma16_off(kbase, off, slot + j * 1024);
        dma16_off(vbase, off, slot + 4096 + j * 1024);
    }
    return valid;
}

// Wait until step `st` has landed when only `left` later steps are in flight
// (the ring's drain at the end of a part).
template <int D>
__device__ __forceinline__ void wait_drain(int left) {
    if constexpr (D > 3) { if (left == 3) { wait_vmcnt<24>(); return; } }
    if constexpr (D > 2) { if (left == 2) { wait_vmcnt<16>(); return; } }
    if (left == 1) { wait_vmcnt<8>(); return; }
    wait_vmcnt<0>();
}

__device__ __forceinline__ float quad_group_max(float x) {
    // max over lanes l, l^16, l^32, l^48 (same lane%16)
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float quad_group_sum(float x) {
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// Selection inside the decode kernel (qsa_decode_step).  Every workgroup
// (query i, KV head g, part c) derives the block ids of its own part of the
// query's ascending selection — positions [p_beg, p_end) — from the scorer's
// per-chunk candidate lists (qsa_lists.hpp), with the same certificate as
// the list finish of qsa_index_score_topk; a row the certificate does not
// cover (or whose lists do not fit) is selected exactly from its whole
// score row.  The workgroup of KV head 0, part 0 also writes the idx row.
// No workgroup waits for another.  Scratch lives in the LDS of the ring
// (the part of it the query rows, requested at the start, do not land in),
// which is free until the first step is issued; the selection goes to a
// table in the LDS region after the rings whose slot p is position p of the
// query's selection (K entries; the region holds kWgWaves * kBigTabSlots of
// them, plus kBigTabSlots so that a wave's reads stay inside).
constexpr int kSelThreads = kWgWaves * kWave;          // 256
constexpr int kSelBins = 1024;
constexpr int kSelBinCand = kWave;
struct SelScratch {
    uint32_t hist[kSelBins];
    uint32_t red[4][kWgWaves];
    uint32_t s[8];
    uint32_t bcw[kWgWaves][kSelBinCand];   // the threshold bin's keys, per wave
    uint32_t bcn[kWgWaves];
    uint32_t tot[8][kWgWaves];             // per register group (at most 8)
};
constexpr int kSelScratchBytes = (int)((sizeof(SelScratch) + 255) & ~(size_t)255);

// Exclusive prefix sum over the 256 threads (thread order); total in `tot`.
// `slot` picks one of the four exchange rows (consecutive calls use
// different rows, so no trailing barrier is needed).
__device__ __forceinline__ uint32_t sel_scan(uint32_t v, SelScratch &X, int slot, uint32_t &tot) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_scan(v);
    if (lane == kWave - 1) X.red[slot][wave] = incl;
    __syncthreads();
    uint32_t before = 0, t = 0;
#pragma unroll
    for (int w = 0; w < kWgWaves; ++w) {
        const uint32_t x = X.red[slot][w];
        before += w < wave ? x : 0u;
        t += x;
    }
    tot = t;
    return before + incl - v;
}

// Exact need-th largest key among key(j), j < n (MSB-first radix, 8-bit
// digits below the bits kmin and kmax share); 256 threads.
template <typename KeyF>
__device__ __forceinline__ uint32_t sel_radix(const KeyF &key, int64_t n, uint32_t need, uint32_t kmin, uint32_t kmax,
                              SelScratch &X, uint32_t &need_eq, uint32_t &total_eq) {
    const uint32_t diff = kmin ^ kmax;
    if (diff == 0) {
        need_eq = need;
        total_eq = (uint32_t)n;
        return kmin;
    }
    const int hi_bit = 31 - __builtin_clz(diff);
    uint32_t prefix = hi_bit == 31 ? 0u : (kmax & ~((2u << hi_bit) - 1u));
    int lo_bit = hi_bit + 1;
    total_eq = 0;
    while (lo_bit > 0) {
        const int width = lo_bit >= 8 ? 8 : lo_bit;
        const int shift = lo_bit - width;
        const uint32_t mask_hi = lo_bit >= 32 ? 0u : ~((1u << lo_bit) - 1u);
        __syncthreads();
        X.hist[threadIdx.x] = 0u;
        __syncthreads();
        for (int64_t j = threadIdx.x; j < n; j += kSelThreads) {
            const uint32_t k = key(j);
            if ((k & mask_hi) == prefix) atomicAdd(&X.hist[(k >> shift) & ((1u << width) - 1u)], 1u);
        }
        __syncthreads();
        // thread t owns digit (2^width - 1 - t), counting from the top
        const int d = (1 << width) - 1 - (int)threadIdx.x;
        const uint32_t h = d >= 0 ? X.hist[d] : 0u;
        uint32_t tot;
        const uint32_t above = sel_scan(h, X, 0, tot);
        if (d >= 0 && above < need && need <= above + h) {
            X.s[4] = (uint32_t)d;
            X.s[5] = above;
            X.s[6] = h;
        }
        __syncthreads();
        prefix |= X.s[4] << shift;
        need -= X.s[5];
        total_eq = X.s[6];
        lo_bit = shift;
    }
    need_eq = need;
    return prefix;
}

// Ordered output of a selection over n entries in ascending block order:
// thread t owns entries [t*E, t*E + E); an entry is selected when its key is
// > T, or == T among the first need_eq such entries.  Selected position p
// gets the entry's logical block id in LDS table slot p.
template <typename KeyF, typename BlkF>
__device__ __forceinline__ void sel_emit(const KeyF &key, const BlkF &blk_of, int64_t n, uint32_t T, uint32_t need_eq,
                                         uint32_t tab, SelScratch &X) {
    const int64_t E = (n + kSelThreads - 1) / kSelThreads;
    const int64_t j0 = (int64_t)threadIdx.x * E;
    const int64_t j1 = j0 + E < n ? j0 + E : n;
    uint32_t ngt = 0, neq = 0;
    for (int64_t j = j0; j < j1; ++j) {
        const uint32_t k = key(j);
        ngt += k > T ? 1u : 0u;
        neq += k == T ? 1u : 0u;
    }
    uint32_t tgt, teq;
    const uint32_t gbefore = sel_scan(ngt, X, 1, tgt);
    const uint32_t ebefore = sel_scan(neq, X, 2, teq);
    uint32_t tie = ebefore;
    uint32_t pos = gbefore + min(tie, need_eq);
    for (int64_t j = j0; j < j1; ++j) {
        const uint32_t k = key(j);
        bool take = k > T;
        if (k == T) {
            take = tie < need_eq;
            ++tie;
        }
        if (take) {
            *(lds_i32_t *)(uintptr_t)(tab + 4u * pos) = blk_of(j);
            ++pos;
        }
    }
}

// Lists of at most sel_reg_entries(NG) entries are selected from registers:
// NG = 4 groups (4096 entries: every row of at most 32768 blocks at
// K <= 512) or NG = 8 (8192 entries: rows of 32768 blocks at K = 2048).
// Thread t holds the entries 4g .. 4g+3 for g = t + 256u, u < NG, so for
// each u the four waves hold 1024 consecutive entries, wave after wave and
// lane after lane: ascending order is (u, wave, lane, e).  The first
// sel_reg_entries(NG) entries and NG/2 * 256 cutoffs of the row's lists are
// requested at the kernel's start, before the query's length is known (they
// lie inside the row's region of the workspace whatever the length; entries
// past the row's own lists are masked once it is known).
__host__ __device__ constexpr int sel_reg_entries(int NG) { return 4 * NG * kSelThreads; }
static_assert(sel_reg_entries(8) / 8 <= 4 * kSelThreads,
              "a list of sel_reg_entries(NG) entries has at most NG/2 * 256 chunks (>= 8 entries each)");
template <int NG>
struct SelPre {
    static_assert(NG == 4 || NG == 8, "register groups");
    uint4 k[NG];
    uint32_t l[NG];
    uint32_t c[NG / 2];
    uint32_t mode;                                   // the lists' form (qsa_lists.hpp)
};

template <int NG>
__device__ __forceinline__ void sel_prefetch(const AttnArgs &A, int64_t i, SelPre<NG> &pf) {
    constexpr int kSelRegEntries = sel_reg_entries(NG), kSelRegGroups = NG, kSelRegCuts = NG / 2;
    const uint4 *__restrict__ gk = reinterpret_cast<const uint4 *>(A.la.keys + i * A.la.stride);
    const uint32_t *__restrict__ gl = reinterpret_cast<const uint32_t *>(A.la.loc + i * A.la.stride);
    const uint32_t *__restrict__ gc = A.la.cut + i * A.la.cstride;
    const int pref = A.sel_pref < kSelRegEntries ? A.sel_pref : kSelRegEntries;
    const int s4 = (int)(A.la.stride / 4 < (pref + 3) / 4 ? A.la.stride / 4 : (pref + 3) / 4);
    const int nc = (int)(A.la.cstride < kSelRegCuts * kSelThreads ? A.la.cstride : kSelRegCuts * kSelThreads);
#pragma unroll
    for (int u = 0; u < kSelRegGroups; ++u) {
        const int g = (int)threadIdx.x + u * kSelThreads;
        pf.k[u] = g < s4 ? gk[g] : make_uint4(0u, 0u, 0u, 0u);
        pf.l[u] = g < s4 ? gl[g] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kSelRegCuts; ++u) {
        const int cc = (int)threadIdx.x + u * kSelThreads;
        pf.c[u] = cc < nc ? gc[cc] : 0u;
    }
    pf.mode = *A.la.mode;
}

__device__ __forceinline__ uint32_t &u4_at(uint4 &v, int e) {
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// The selection from the registers (M = nch * kk <= kSelRegEntries listed
// entries), written to LDS table slots 0 .. K-1 as logical block ids.
// Returns false, after a barrier, when it cannot decide the row (the
// certificate fails, or more than 64 keys share the threshold's bin): the
// caller then selects from the whole row.  Five barriers: the list
// statistics, the histogram, the threshold bin's keys, the emit counts, the
// finished table.
// `nslot`: entry M-1 is the block the row's newest token completed (key
// nkey, lane nloc), which its chunk left to the selection.
template <int NG>
__device__ __forceinline__ bool select_part_regs(const AttnArgs &A, int kk, int nch, int M, uint32_t tab,
                                                 SelScratch &X, SelPre<NG> &pf, bool nslot, uint32_t nkey,
                                                 uint32_t nloc) {
    constexpr int kSelRegGroups = NG, kSelRegCuts = NG / 2;
    const int K = A.K;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    uint32_t kmin = 0xffffffffu, kmax = 0u, nreal = 0u, mcut = 0u;
#pragma unroll
    for (int u = 0; u < kSelRegGroups; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * ((int)threadIdx.x + u * kSelThreads) + e;
            uint32_t &key = u4_at(pf.k[u], e);
            key = j < M ? key : 0u;
            if (nslot && j == M - 1) {
                key = nkey;
                pf.l[u] = (pf.l[u] & ~(0xffu << (8 * e))) | (nloc << (8 * e));
            }
            if (key != 0u) {
                kmin = min(kmin, key);
                kmax = max(kmax, key);
                ++nreal;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kSelRegCuts; ++u)
        if ((int)threadIdx.x + u * kSelThreads < nch) mcut = max(mcut, pf.c[u]);
    for (int b = threadIdx.x; b < kSelBins; b += kSelThreads) X.hist[b] = 0u;
    {
        const uint32_t w_mn = wave_min_u32(kmin), w_mx = wave_max_u32(kmax), w_mc = wave_max_u32(mcut);
        const uint32_t w_n = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(nreal), kWave - 1);
        if (lane == 0) {
            X.red[0][wave] = w_mn;
            X.red[1][wave] = w_mx;
            X.red[2][wave] = w_n;
            X.red[3][wave] = w_mc;
        }
    }
    __syncthreads();                                                      // 1
    kmin = X.red[0][0];
    kmax = X.red[1][0];
    nreal = X.red[2][0];
    mcut = X.red[3][0];
#pragma unroll
    for (int w = 1; w < kWgWaves; ++w) {
        kmin = min(kmin, X.red[0][w]);
        kmax = max(kmax, X.red[1][w]);
        nreal += X.red[2][w];
        mcut = max(mcut, X.red[3][w]);
    }
    if (!(nreal >= (uint32_t)K && mcut < kmax)) {     // cannot certify (uniform)
        __syncthreads();
        return false;
    }
    uint32_t T, need_eq;
    if (kmin == kmax) {
        T = kmin;
        need_eq = (uint32_t)K;
    } else {
        // A certified threshold exceeds every cutoff, so only keys from
        // lo = max(kmin, mcut + 1) up can be it (a whole short chunk can list
        // keys far below the rest, which would crowd coarse bins).  1024 bins
        // linear in the key: bin = (key - lo) >> sh <= 1023.
        const uint32_t lo = max(kmin, mcut + 1u);
        const uint32_t span = kmax - lo;
        const int sh = span < (uint32_t)kSelBins ? 0 : (32 - __builtin_clz(span)) - 10;
#pragma unroll
        for (int u = 0; u < kSelRegGroups; ++u) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t key = u4_at(pf.k[u], e);
                if (key >= lo) atomicAdd(&X.hist[(key - lo) >> sh], 1u);
            }
        }
        __syncthreads();                                                  // 2
        // every wave finds the bin of the K-th largest: lane l owns the 16
        // bins 1023 - 16 l down to 1008 - 16 l (the top bins first)
        const uint4 *h4 = reinterpret_cast<const uint4 *>(X.hist);
        uint32_t hb[16], own = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = h4[kSelBins / 4 - 1 - 4 * lane - q];
            hb[4 * q + 0] = v.w;
            hb[4 * q + 1] = v.z;
            hb[4 * q + 2] = v.y;
            hb[4 * q + 3] = v.x;
            own += (v.x + v.y) + (v.z + v.w);
        }
        const uint32_t incl = wave_incl_scan(own);
        const uint32_t above = incl - own;
        const bool hit = above < (uint32_t)K && (uint32_t)K <= incl;
        const uint64_t hm = __ballot(hit);
        if (hm == 0u) {                               // fewer than K keys above the cutoffs (uniform)
            __syncthreads();
            return false;
        }
        const int hl = (int)__builtin_ctzll(hm);
        const int top = kSelBins - 1 - 16 * lane;
        uint32_t tb_l = 0u, need_l = 0u, nbin_l = 0u, a = above;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (a < (uint32_t)K && (uint32_t)K <= a + hb[e]) {
                tb_l = (uint32_t)(top - e);
                need_l = (uint32_t)K - a;
                nbin_l = hb[e];
            }
            a += hb[e];
        }
        const uint32_t tb = (uint32_t)__builtin_amdgcn_readlane((int)tb_l, hl);
        const uint32_t need = (uint32_t)__builtin_amdgcn_readlane((int)need_l, hl);
        const uint32_t nbin = (uint32_t)__builtin_amdgcn_readlane((int)nbin_l, hl);
        if (nbin > (uint32_t)kSelBinCand) {           // crowded bin: the whole row decides (uniform)
            __syncthreads();
            return false;
        }
        // the bin's keys, compacted per wave in ascending order (ballots)
        uint32_t wcnt = 0u;
#pragma unroll
        for (int u = 0; u < kSelRegGroups; ++u) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t key = u4_at(pf.k[u], e);
                const bool in = key >= lo && ((key - lo) >> sh) == tb;
                const uint64_t m = __ballot(in);
                if (in) X.bcw[wave][wcnt + list_lanes_below(m)] = key;
                wcnt += (uint32_t)__builtin_popcountll(m);
            }
        }
        if (lane == 0) X.bcn[wave] = wcnt;
        __syncthreads();                                                  // 3
        // every wave ranks them: lane l < nbin holds key l of the union
        const uint32_t o1 = X.bcn[0], o2 = o1 + X.bcn[1], o3 = o2 + X.bcn[2];
        const uint32_t ul = (uint32_t)lane;
        const int w = ul < o1 ? 0 : ul < o2 ? 1 : ul < o3 ? 2 : 3;
        const uint32_t off = w == 0 ? 0u : w == 1 ? o1 : w == 2 ? o2 : o3;
        const bool mine = ul < nbin;
        const uint32_t key = mine ? X.bcw[w][ul - off] : 0u;
        uint32_t gt = 0u, eq = 0u;
        for (int j = 0; j < (int)nbin; ++j) {
            const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)key, j);
            gt += o > key ? 1u : 0u;
            eq += o == key ? 1u : 0u;
        }
        const bool h2 = mine && gt < need && need <= gt + eq;
        const int l2 = (int)__builtin_ctzll(__ballot(h2));
        T = (uint32_t)__builtin_amdgcn_readlane((int)key, l2);
        need_eq = (uint32_t)__builtin_amdgcn_readlane((int)(need - gt), l2);
    }
    if (!(T != 0u && mcut < T)) {
        __syncthreads();
        return false;
    }
    // ordered emit: per (u, wave) the packed counts (gt << 16 | eq) of the
    // entries before each lane, and the four waves' totals through LDS
    uint32_t pre[kSelRegGroups];
#pragma unroll
    for (int u = 0; u < kSelRegGroups; ++u) {
        uint32_t c = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t key = u4_at(pf.k[u], e);
            c += key > T ? 0x10000u : 0u;
            c += key == T ? 1u : 0u;
        }
        const uint32_t incl = wave_incl_scan(c);
        pre[u] = incl - c;
        const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
        if (lane == 0) X.tot[u][wave] = tot;
    }
    __syncthreads();                                                      // 4
    // chunk of entry j: j / kk by a multiply (j < 2^13, 8 <= kk <= 64:
    // j * magic / 2^20 exceeds j / kk by less than j / 2^20 < 1 / kk, so the
    // floor is exact)
    const uint32_t magic = (1u << 20) / (uint32_t)kk + 1u;
    uint32_t base = 0u;
#pragma unroll
    for (int u = 0; u < kSelRegGroups; ++u) {
        uint32_t b = base;
#pragma unroll
        for (int w = 0; w < kWgWaves; ++w) {
            const uint32_t t = X.tot[u][w];
            b += w < wave ? t : 0u;
            base += t;
        }
        b += pre[u];
        uint32_t gb = b >> 16, eb = b & 0xffffu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t key = u4_at(pf.k[u], e);
            const uint32_t isgt = key > T ? 1u : 0u, iseq = key == T ? 1u : 0u;
            const bool take = isgt != 0u || (iseq != 0u && eb < need_eq);
            const uint32_t pos = gb + (isgt != 0u ? min(eb, need_eq) : eb);
            gb += isgt;
            eb += iseq;
            const uint32_t j = 4u * (threadIdx.x + (uint32_t)(u * kSelThreads)) + (uint32_t)e;
            const int32_t blk = (int32_t)(((j * magic) >> 20) * kListChunk + ((pf.l[u] >> (8 * e)) & 0xffu));
            if (take) *(lds_i32_t *)(uintptr_t)(tab + 4u * pos) = blk;
        }
    }
    (void)nch;
    __syncthreads();                                                      // 5
    return true;
}

// The selection paths taken rarely: lists of more than kSelRegEntries
// entries (staged in the ring's LDS), and the whole score row when the lists
// cannot decide (staged in LDS when it fits).  The caller has emptied the
// ring (no query rows in flight).  Fills LDS table slots 0 .. K-1 with
// logical block ids and ends with a barrier.
template <int D, int kSelRegEntries>
__device__ __forceinline__ void select_slow(const uint32_t *__restrict__ gk, const uint8_t *__restrict__ gl,
                                            const uint32_t *__restrict__ gc, const float *__restrict__ row, int64_t nb,
                                            int K, int kk, int nch, int M, uint32_t tab, uint8_t *ring_lds,
                                            bool nslot, uint32_t nkey, uint32_t nloc) {
    SelScratch &X = *reinterpret_cast<SelScratch *>(ring_lds);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    constexpr int cap = ((kWgWaves * D * kSlotBytes - kSelScratchBytes) / 5) & ~3;
    uint32_t *keys = reinterpret_cast<uint32_t *>(ring_lds + kSelScratchBytes);
    uint8_t *locs = reinterpret_cast<uint8_t *>(keys + cap);
    uint32_t T = 0, need_eq = 0, total_eq = 0;
    bool done = false;
    if (M > kSelRegEntries && M <= cap) {
        uint32_t kmin = 0xffffffffu, kmax = 0u, nreal = 0u, mcut = 0u;
        for (int j0 = threadIdx.x; j0 < M; j0 += 4 * kSelThreads) {
            uint32_t k[4], l[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * kSelThreads;
                const bool nj = nslot && j == M - 1;
                k[u] = j < M ? (nj ? nkey : gk[j]) : 0u;
                l[u] = j < M ? (nj ? nloc : gl[j]) : 0u;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * kSelThreads;
                if (j < M) {
                    keys[j] = k[u];
                    locs[j] = (uint8_t)l[u];
                    if (k[u] != 0u) {
                        kmin = min(kmin, k[u]);
                        kmax = max(kmax, k[u]);
                        ++nreal;
                    }
                }
            }
        }
        for (int cc = threadIdx.x; cc < nch; cc += kSelThreads) mcut = max(mcut, gc[cc]);
        for (int b = threadIdx.x; b < kSelBins; b += kSelThreads) X.hist[b] = 0u;
        {
            const uint32_t w_mn = wave_min_u32(kmin), w_mx = wave_max_u32(kmax), w_mc = wave_max_u32(mcut);
            const uint32_t w_n = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(nreal), kWave - 1);
            if (lane == 0) {
                X.red[0][wave] = w_mn;
                X.red[1][wave] = w_mx;
                X.red[2][wave] = w_n;
                X.red[3][wave] = w_mc;
            }
            __syncthreads();
            kmin = X.red[0][0];
            kmax = X.red[1][0];
            nreal = X.red[2][0];
            mcut = X.red[3][0];
#pragma unroll
            for (int w = 1; w < kWgWaves; ++w) {
                kmin = min(kmin, X.red[0][w]);
                kmax = max(kmax, X.red[1][w]);
                nreal += X.red[2][w];
                mcut = max(mcut, X.red[3][w]);
            }
            __syncthreads();                                 // X.red is reused below
        }
        if (nreal >= (uint32_t)K && mcut < kmax) {
            const uint32_t *kl = keys;
            T = sel_radix([kl](int64_t j) { return kl[j]; }, (int64_t)M, (uint32_t)K, kmin, kmax, X, need_eq,
                          total_eq);
            if (T != 0u && mcut < T) {
                sel_emit([keys](int64_t j) { return keys[j]; },
                         [locs, kk](int64_t j) { return (int32_t)(((int)j / kk) * kListChunk + locs[j]); },
                         (int64_t)M, T, need_eq, tab, X);
                done = true;
            }
        }
        __syncthreads();
    }
    if (!done) {
        // the whole score row, exactly: staged in the ring's LDS when it fits
        // (one pass of coalesced loads, 16 in flight per thread), else read
        // from the score row on every pass
        auto rkey = [row](int64_t j) {
            const uint32_t u = __float_as_uint(row[j]);
            return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
        };
        constexpr int row_cap = (kWgWaves * D * kSlotBytes - kSelScratchBytes) / 4;
        const bool staged = nb <= row_cap;
        uint32_t *rk = keys;
        uint32_t kmin = 0xffffffffu, kmax = 0u;
        if (staged) {
            for (int j0 = 0; j0 < (int)nb; j0 += 16 * kSelThreads) {
                uint32_t v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int j = j0 + u * kSelThreads + (int)threadIdx.x;
                    v[u] = j < (int)nb ? rkey(j) : 0u;
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int j = j0 + u * kSelThreads + (int)threadIdx.x;
                    if (j < (int)nb) {
                        rk[j] = v[u];
                        kmin = min(kmin, v[u]);
                        kmax = max(kmax, v[u]);
                    }
                }
            }
        } else {
            for (int64_t j = threadIdx.x; j < nb; j += kSelThreads) {
                const uint32_t k = rkey(j);
                kmin = min(kmin, k);
                kmax = max(kmax, k);
            }
        }
        {
            const uint32_t w_mn = wave_min_u32(kmin), w_mx = wave_max_u32(kmax);
            if (lane == 0) {
                X.red[0][wave] = w_mn;
                X.red[1][wave] = w_mx;
            }
            __syncthreads();
            kmin = X.red[0][0];
            kmax = X.red[1][0];
#pragma unroll
            for (int w = 1; w < kWgWaves; ++w) {
                kmin = min(kmin, X.red[0][w]);
                kmax = max(kmax, X.red[1][w]);
            }
            __syncthreads();
        }
        auto ident = [](int64_t j) { return (int32_t)j; };
        if (staged) {
            auto lkey = [rk](int64_t j) { return rk[j]; };
            T = sel_radix(lkey, nb, (uint32_t)K, kmin, kmax, X, need_eq, total_eq);
            sel_emit(lkey, ident, nb, T, need_eq, tab, X);
        } else {
            T = sel_radix(rkey, nb, (uint32_t)K, kmin, kmax, X, need_eq, total_eq);
            sel_emit(rkey, ident, nb, T, need_eq, tab, X);
        }
        __syncthreads();
    }
    (void)total_eq;
}

// Fill LDS table slots [p_beg, p_end) with query i's selected block ids
// (physical when paged; nb > 0 visible blocks) and, for the designated
// workgroup, write the idx row.  The selection is built as logical ids in
// slots 0 .. K-1; a last pass copies the row out and translates the part.
// `q_in_ring`: the query rows' loads into the ring's last slots are in
// flight; a path that uses the whole ring waits for them and clears it.
template <int D, int NG>
__device__ __forceinline__ void select_part(const AttnArgs &A, int64_t i, int seq, int64_t L, int p_beg, int p_end,
                                            bool designated, uint32_t tab, uint8_t *ring_lds, SelPre<NG> &pf,
                                            bool &q_in_ring) {
    const int64_t nb = L >> A.log2r;
    SelScratch &X = *reinterpret_cast<SelScratch *>(ring_lds);
    const int K = A.K;
    int32_t *row_out = designated ? A.idx_out + i * (int64_t)K : nullptr;
    if (nb <= K) {                                           // dense regime: identity
        for (int j = threadIdx.x; j < K; j += kSelThreads) {
            const int32_t v = j < nb ? j : -1;
            if (row_out) row_out[j] = v;
            if (j >= p_beg && j < p_end)
                *(lds_i32_t *)(uintptr_t)(tab + 4u * (uint32_t)j) =
                    A.pm.table ? slot_phys(v, A.pm, seq, nb, A.log2r) : v;
        }
        __syncthreads();
        return;
    }
    const int kk = list_len(nb, K);
    const int nch = (int)((nb + kListChunk - 1) / kListChunk);
    const int M = nch * kk;
    static_assert(kSelScratchBytes <= kSlotBytes, "the selection scratch stays clear of the query rows' slots");
    // the last entry of a row whose newest token completed a block is that
    // block, scored by the append (its chunk left the slot)
    const bool nslot = list_new_block_slot(pf.mode, L, A.log2r);
    const uint32_t nkey = nslot ? list_order_key(A.scores[i * A.ld + nb - 1]) : 0u;
    const uint32_t nloc = (uint32_t)((nb - 1) & (kListChunk - 1));
    bool done = false;
    if (M <= sel_reg_entries(NG)) done = select_part_regs<NG>(A, kk, nch, M, tab, X, pf, nslot, nkey, nloc);
    if (!done) {
        if (q_in_ring) {                                      // the slow paths use the whole ring
            wait_vmcnt<0>();                                  // this wave's query loads landed,
            __syncthreads();                                  // and every other wave's
            q_in_ring = false;
        }
        select_slow<D, sel_reg_entries(NG)>(A.la.keys + i * A.la.stride, A.la.loc + i * A.la.stride,
                                            A.la.cut + i * A.la.cstride,
                       A.scores + i * A.ld, nb, K, kk, nch, M, tab, ring_lds, nslot, nkey, nloc);
    }
    // slots 0 .. K-1 hold the selection (nb > K): the idx row, and the part
    // translated to pool blocks when paged (each slot read and written by
    // one thread)
    for (int j = threadIdx.x; j < K; j += kSelThreads) {
        lds_i32_t *slot = (lds_i32_t *)(uintptr_t)(tab + 4u * (uint32_t)j);
        if (row_out) row_out[j] = *slot;
        if (A.pm.table && j >= p_beg && j < p_end) *slot = slot_phys(*slot, A.pm, seq, nb, A.log2r);
    }
    if (A.pm.table) __syncthreads();
}

// Decode attention of one wave on the matrix cores.  Per 16-token step:
//  QK: S[t][n] = K[t,:] . q_n for the 16 tokens t (M) and up to 16 query
//      heads n of the KV head (N; heads >= G are zero columns), four
//      v_mfma_f32_16x16x32_bf16 over the 128 dims.  Lane l gets S for head
//      n = l%16 and tokens 4(l/16)..+3.
//  softmax: online, fp32, exp2 domain; the running max of head n is shared
//      by the four lanes that hold it (permlane swaps).
//  PV: O^T[d][n] += V^T[d][t] P[t][n] as eight v_mfma_f32_16x16x16_bf16
//      tiles of 16 dims (M) by the 16 heads (N) over the 16 tokens (K).  The
//      B operand P[t][n] (4 tokens of head n per lane) is exactly what the
//      QK tile left in the lane.  P is fed as two bf16 terms, hi = P with the
//      low 16 bits cleared and lo = bf16(P - hi), so the weights carry 16
//      significant bits (relative error <= 2^-16) instead of bf16's 8; V is
//      bf16 data and enters unchanged.  The V^T operand is read with the
//      gfx950 transposed LDS load (ds_read_b64_tr_b16: lane i of each 16-lane
//      group gets column i of the four rows its group points at).
//  Lane l accumulates O^T for head l%16, dims 16m + 4(l/16) + 0..3, m < 8.
template <int D, bool BIG, bool SELECT, int NG = 4>
__device__ __forceinline__ void attn_decode_mfma_body(const AttnArgs &A, int G) {
    static_assert(BIG || !SELECT, "the in-kernel selection fills an LDS slot table");
    extern __shared__ __align__(16) uint8_t dyn_lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // workgroup = (query i, KV head g, part c); its 4 waves split the part.
    // 32-bit index arithmetic: the grid, K and the part sizes are below 2^31
    // (the launcher's grid is a 32-bit count), and 64-bit division by a
    // runtime divisor is a long dependent sequence at the head of every wave.
    const uint32_t wg = blockIdx.x;
    const int g = (int)(wg % (uint32_t)A.hkv);
    const uint32_t t2 = wg / (uint32_t)A.hkv;
    const int c = (int)(t2 % (uint32_t)A.n_part);
    const int64_t i = (int64_t)(t2 / (uint32_t)A.n_part);
    if (i >= A.total_q) return;                      // uniform over the workgroup
    const int qh0 = g * G;
    uint8_t *ring = dyn_lds + wave * (D * kSlotBytes);
    const uint32_t ring_addr = lds_addr(ring);
    // Query rows (G x 256 contiguous bytes) travel through the last ring slot,
    // which the prologue leaves free (a compiler-visible load would make the
    // compiler wait for it, and so for the whole ring, inside the loop).
    auto load_q = [&]() {
        const uint32_t qslot = ring_addr + (D - 1) * kSlotBytes;
        const uint16_t *qsrc = static_cast<const uint16_t *>(A.q) + (i * A.hq + qh0) * kD;
        const int nq = (G * kD * 2 + 1023) / 1024;        // 1 KB per load, G <= 16
        for (int j = 0; j < nq; ++j) {
            const int e = (j * kWave + lane) * 8;          // bf16 element of this lane
            dma16(qsrc + (e < G * kD ? e : 0), qslot + j * 1024);
        }
    };
    // SELECT: the lists and the query rows are requested first; neither
    // depends on the query's length, so their latency overlaps the offsets'.
    SelPre<NG> pf;
    bool q_in_ring = false;
    if constexpr (SELECT) {
        sel_prefetch<NG>(A, i, pf);
        load_q();
        q_in_ring = true;
    }

    // This wave's share [s_beg, s_end) of the query's nsel selected blocks.
    auto split = [&](int nsel_, int64_t &sb, int64_t &se) {
        const int per = (nsel_ + A.n_part - 1) / A.n_part;
        const int p_beg = min(c * per, nsel_);
        const int p_end = min(p_beg + per, nsel_);
        const int sub = (p_end - p_beg + kWgWaves - 1) / kWgWaves;
        sb = min(p_beg + wave * sub, p_end);
        se = min((int)sb + sub, p_end);
    };
    // The slot table (this wave's selected block ids) is requested before
    // the query's length is known, for the common case of a row with at least
    // K blocks (nsel = K), so its latency overlaps that of the offsets; a
    // shorter row loads it again below.
    int64_t s_beg, s_end;
    split(A.K, s_beg, s_end);
    const int32_t *sel = A.idx + i * (int64_t)A.K + s_beg;
    int nslot = (int)(s_end - s_beg);
    uint32_t tab0 = 0, tab1 = 0;
    if constexpr (!BIG) {
        tab0 = (uint32_t)(lane < nslot ? sel[lane] : -1);
        tab1 = (uint32_t)(kWave + lane < nslot ? sel[kWave + lane] : -1);
    }

    const QueryPos qp = query_pos(A.kv_off, nullptr, A.q_off, A.num_seqs, i);
    const int64_t nb = qp.L >> A.log2r;
    const int64_t nsel = nb < A.K ? nb : (int64_t)A.K;
    if (nsel < A.K) {                                // wave-uniform
        split((int)nsel, s_beg, s_end);
        sel = A.idx + i * (int64_t)A.K + s_beg;
        nslot = (int)(s_end - s_beg);
        if constexpr (!BIG) {
            tab0 = (uint32_t)(lane < nslot ? sel[lane] : -1);
            tab1 = (uint32_t)(kWave + lane < nslot ? sel[kWave + lane] : -1);
        }
    }
    // BIG: the whole share (at most kBigTabSlots slots) into this wave's LDS
    // table, block ids translated to pool blocks when paged, -1 past the end.
    // SELECT: one table of the whole selection (slot p = position p) over the
    // four waves' regions, filled by the selection; each wave reads its share
    // from its first position (the part's slots translated when paged).
    uint32_t big_tab = lds_addr(dyn_lds + kWgWaves * D * kSlotBytes + wave * kBigTabBytes);
    if constexpr (SELECT) {
        const int per = ((int)nsel + A.n_part - 1) / A.n_part;
        const int p_beg = min(c * per, (int)nsel);
        const int p_end = min(p_beg + per, (int)nsel);
        const uint32_t sel_tab = lds_addr(dyn_lds + kWgWaves * D * kSlotBytes);   // slot p = position p
        if (nb > 0)
            select_part<D, NG>(A, i, qp.seq, qp.L, p_beg, p_end, g == 0 && c == 0, sel_tab, dyn_lds, pf, q_in_ring);
        else if (g == 0 && c == 0)
            for (int j = threadIdx.x; j < A.K; j += kSelThreads) A.idx_out[i * (int64_t)A.K + j] = -1;
        big_tab = sel_tab + 4u * (uint32_t)s_beg;
    }
    if constexpr (BIG && !SELECT) {
        int32_t v[kBigTabSlots / kWave];
#pragma unroll
        for (int j = 0; j < kBigTabSlots / kWave; ++j)
            v[j] = j * kWave + lane < nslot ? sel[j * kWave + lane] : -1;
#pragma unroll
        for (int j = 0; j < kBigTabSlots / kWave; ++j) {
            const int32_t b = A.pm.table ? slot_phys(v[j], A.pm, qp.seq, nb, A.log2r) : v[j];
            *(lds_i32_t *)(uintptr_t)(big_tab + 4u * (uint32_t)(j * kWave + lane)) = b;
        }
    }
    const bool owns_tail = c == A.n_part - 1 && wave == kWgWaves - 1;
    WaveWork W;
    W.sel = sel;
    W.nslot = nslot;
    W.log2r = A.log2r;
    W.nblk_tok = W.nslot << A.log2r;
    W.tail0 = nb << A.log2r;
    W.nb = nb;
    W.ntok = W.nblk_tok + (owns_tail ? (int)(qp.L - W.tail0) : 0);
    if (A.pm.table) {                                // paged pools: physical block ids and rows
        page_wave(W, A.pm, qp.seq, qp.L);
        if constexpr (!BIG) {
            tab0 = (uint32_t)slot_phys((int)tab0, A.pm, qp.seq, nb, A.log2r);
            tab1 = (uint32_t)slot_phys((int)tab1, A.pm, qp.seq, nb, A.log2r);
        }
    }
    const int64_t row0 = A.pm.table ? 0 : qp.kv_row0;

    const int n = lane & 15;                        // head column of this lane
    const int gq = lane >> 4;                       // 16-lane group
    const uint32_t row_bytes = (uint32_t)A.hkv * kD * 2;
    const uint16_t *__restrict__ kbase = static_cast<const uint16_t *>(A.k) + (row0 * A.hkv + g) * kD;
    const uint16_t *__restrict__ vbase = static_cast<const uint16_t *>(A.v) + (row0 * A.hkv + g) * kD;

    const int nsteps = (W.ntok + kStep - 1) / kStep;
    // the query rows are requested together with the slot table, so the two
    // latencies overlap (SELECT requested them at the start)
    if (nsteps > 0 && !q_in_ring) load_q();
    // a wave with no steps lets its early query loads land before the merge
    // below reuses its ring
    if (nsteps == 0 && q_in_ring) wait_vmcnt<0>();
    // The ring loads are invisible to the compiler, so it would place the
    // wait for the slot table inside the prologue loop below (waiting for the
    // ring loads as well); consuming the table here puts that wait up front.
    asm volatile("" ::"v"(tab0), "v"(tab1));

    uint64_t fifo = 0;                               // valid masks of issued steps
    int pending = 0;
    int slot_in = 0, slot_out = 0;
    auto issue = [&](int s) {
        uint32_t m;
        if constexpr (BIG)
            m = issue_step_lds_tab(W, s, lane, big_tab, kbase, vbase, row_bytes, ring_addr + slot_in * kSlotBytes);
        else
            m = issue_step_lds(W, s, lane, tab0, tab1, kbase, vbase, row_bytes, ring_addr + slot_in * kSlotBytes);
        fifo |= (uint64_t)m << (16 * pending);
        ++pending;
        slot_in = slot_in + 1 == D ? 0 : slot_in + 1;
    };

    const int npro = nsteps < D - 1 ? nsteps : D - 1;
    for (int s = 0; s < npro; ++s) issue(s);

    bf16x8_t qb[4];                                  // B operand: q_n, dims 32k + 8gq ..
    if (nsteps > 0) {
        if (nsteps < D - 1) wait_drain<D>(npro);
        else wait_drain<D>(D - 1);                   // the query loads are older than the steps
        __builtin_amdgcn_sched_barrier(0);
        const uint4 *qs = reinterpret_cast<const uint4 *>(ring + (D - 1) * kSlotBytes);
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            const uint4 x = n < G ? qs[n * 16 + 4 * k4 + gq] : make_uint4(0u, 0u, 0u, 0u);
            qb[k4] = __builtin_bit_cast(bf16x8_t, x);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): read out before the slot is refilled
        __builtin_amdgcn_sched_barrier(0);
    }

    f32x4_t o[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) o[m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;

    for (int st = 0; st < nsteps; ++st) {
        __builtin_amdgcn_sched_barrier(0);
        if (st + D - 1 < nsteps) {
            issue(st + D - 1);
            wait_vmcnt<8 * (D - 1)>();
        } else {
            wait_drain<D>(nsteps - 1 - st);
        }
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t valid = (uint32_t)(fifo & 0xffffu);
        fifo >>= 16;
        --pending;
        const uint8_t *slot = ring + slot_out * kSlotBytes;
        slot_out = slot_out + 1 == D ? 0 : slot_out + 1;

        // ---- QK: token n of the tile (row of A), dims 32k + 8gq .. +8
        const uint4 *kt = reinterpret_cast<const uint4 *>(slot);
        f32x4_t sacc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            const uint4 a = kt[n * 16 + ((4 * k4 + gq) ^ n)];
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), qb[k4], sacc,
                                                           0, 0, 0);
        }
        // ---- V^T operands (transposed reads), issued before the softmax
        s16x4_t va[8];
        {
            // lanes 4a+c of group gq point at token 4gq + a, dims 16m + 4c
            const int tv = 4 * gq + ((lane & 15) >> 2);
            const int cc = lane & 3;
            typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
            const uint32_t vrow = lds_addr(slot + 4096 + tv * 256);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int ch = 2 * m + (cc >> 1);
                const uint32_t addr = vrow + ((ch ^ tv) << 4) + ((cc & 1) << 3);
                va[m] = __builtin_bit_cast(s16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                        (lds_s16x4 *)(uintptr_t)addr));
            }
        }
        // ---- online softmax for head n over tokens 4gq .. 4gq+3
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            x[e] = ((valid >> (4 * gq + e)) & 1u) ? sacc[e] * A.c : -INFINITY;
        // The reference max m_run is raised only when a score exceeds it by
        // more than 8 (log2 domain): weights relative to a stale reference are
        // at most 2^8, which fp32 and the bf16 terms below hold easily, and the
        // common factor cancels in o / l.  Rescales thus happen a few times
        // per part instead of at nearly every step.
        const float mloc = quad_group_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const bool raise = mloc > m_run + 8.0f;
        if (__ballot(raise) != 0) {
            const float m_new = raise ? mloc : m_run;
            const float alpha = raise ? exp2f(m_run - m_new) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int m = 0; m < 8; ++m) o[m] *= alpha;
            m_run = m_new;
        }
        const float m_safe = m_run == -INFINITY ? 0.0f : m_run;
        float pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[e] = exp2f(x[e] - m_safe);
        l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        // ---- P as hi + lo bf16 terms
        s16x4_t ph, pl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t u = __float_as_uint(pr[e]);
            const float hi = __uint_as_float(u & 0xffff0000u);
            ph[e] = (short)(u >> 16);
            pl[e] = (short)bf16_rne_bits(pr[e] - hi);
        }
        // ---- PV
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[m], ph, o[m], 0, 0, 0);
            o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[m], pl, o[m], 0, 0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- merge the 4 waves of the workgroup through LDS (each wave writes
    // its fragments into its own, now idle, ring region), then wave w
    // finishes dims tiles 2w and 2w+1 of every head.
    const float l_tot = quad_group_sum(l_run);
    {
        f32x4_t *frag = reinterpret_cast<f32x4_t *>(ring);             // [8][64]
        float *ml = reinterpret_cast<float *>(ring + 8 * kWave * 16);  // [64][2]
#pragma unroll
        for (int m = 0; m < 8; ++m) frag[m * kWave + lane] = o[m];
        ml[2 * lane] = m_run;
        ml[2 * lane + 1] = l_tot;
    }
    __syncthreads();
    float mv[kWgWaves], lv[kWgWaves];
#pragma unroll
    for (int v = 0; v < kWgWaves; ++v) {
        const float *ml = reinterpret_cast<const float *>(dyn_lds + v * (D * kSlotBytes) + 8 * kWave * 16);
        mv[v] = ml[2 * lane];
        lv[v] = ml[2 * lane + 1];
    }
    float M = mv[0];
#pragma unroll
    for (int v = 1; v < kWgWaves; ++v) M = fmaxf(M, mv[v]);
    const float Ms = M == -INFINITY ? 0.0f : M;
    float wv[kWgWaves], L = 0.0f;
#pragma unroll
    for (int v = 0; v < kWgWaves; ++v) {
        wv[v] = exp2f(mv[v] - Ms);
        L += wv[v] * lv[v];
    }
    if (n >= G) return;
    const int h = qh0 + n;
    const int64_t slotp = (i * A.hq + h) * A.n_part + c;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
        const int m = 2 * wave + k2;
        f32x4_t acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int v = 0; v < kWgWaves; ++v) {
            const f32x4_t *frag = reinterpret_cast<const f32x4_t *>(dyn_lds + v * (D * kSlotBytes));
            acc += wv[v] * frag[m * kWave + lane];
        }
        const int d0 = 16 * m + 4 * gq;
        if (A.n_part == 1) {
            const float inv = L > 0.0f ? 1.0f / L : 0.0f;
            uint2 w2;
            w2.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
            w2.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(A.out) + (i * A.hq + h) * kD + d0) = w2;
        } else {
            *reinterpret_cast<f32x4_t *>(A.ws_o + slotp * kD + d0) = acc;
        }
    }
    if (A.n_part > 1 && wave == 0 && gq == 0) {
        A.ws_ml[slotp * 2 + 0] = M;
        A.ws_ml[slotp * 2 + 1] = L;
    }
}

template <int D, bool BIG, bool SELECT, int NG = 4>
__global__ __launch_bounds__(kWgWaves * kWave) void attn_decode_mfma_kernel(AttnArgs A, int G, LayerPtrs Lp) {
    if (gridDim.y > 1) {
        const int l = blockIdx.y;
        A.q = Lp.q[l]; A.k = Lp.k[l]; A.v = Lp.v[l]; A.out = Lp.out[l]; A.c = Lp.c[l];
        A.ws_o += l * Lp.ws_stride;
        if (A.ws_ml) A.ws_ml += l * Lp.ws_stride;
    }
    attn_decode_mfma_body<D, BIG, SELECT, NG>(A, G);
}

// Merge part partials: one wave per (query, head); lane s < n_part reads
// partial s's (m, l), the wave forms the weights (DPP reductions), then every
// lane accumulates dims 2p, 2p+1 over the partials (all partial loads issued
// together, so the kernel costs one memory round trip).
constexpr int kMaxGroups = 32;

template <bool BF16>
__global__ __launch_bounds__(kWgWaves * kWave) void attn_combine_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_ml, int n_part, int64_t rows,
    void *__restrict__ out, LayerPtrs Lp) {
    if (gridDim.y > 1) {
        const int l = blockIdx.y;
        ws_o += l * Lp.ws_stride;
        ws_ml += l * Lp.ws_stride;
        out = Lp.out[l];
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t r = (int64_t)blockIdx.x * kWgWaves + wave;   // query*hq + head
    if (r >= rows) return;
    const float *ml = ws_ml + r * n_part * 2;
    float2 os[kMaxGroups];
#pragma unroll
    for (int s = 0; s < kMaxGroups; ++s)
        if (s < n_part) os[s] = reinterpret_cast<const float2 *>(ws_o + (r * n_part + s) * kD)[lane];
    const float m_s = lane < n_part ? ml[2 * lane] : -INFINITY;
    const float l_s = lane < n_part ? ml[2 * lane + 1] : 0.0f;
    const float mmax = wave_max_f32(m_s);
    const float msafe = mmax == -INFINITY ? 0.0f : mmax;
    const float w_s = l_s > 0.0f ? exp2f(m_s - msafe) : 0.0f;
    const float l = wave_sum_f32(w_s * l_s);
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxGroups; ++s) {
        if (s < n_part) {
            const float wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_s), s));
            o0 = __builtin_fmaf(wgt, os[s].x, o0);
            o1 = __builtin_fmaf(wgt, os[s].y, o1);
        }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if constexpr (BF16) {
        reinterpret_cast<uint32_t *>(out)[r * (kD / 2) + lane] = pack_bf16x2(o0 * inv, o1 * inv);
    } else {
        reinterpret_cast<float2 *>(out)[r * (kD / 2) + lane] = make_float2(o0 * inv, o1 * inv);
    }
}

// Ring depth of the decode kernel: as deep as the LDS of one CU allows for
// the workgroups that share it (4 waves x D slots x 8 KB per workgroup, two
// or more workgroups per CU get D = 2).
int cu_count() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Workgroups per CU the decode split aims for: a random gather of 256-byte
// rows needs at least 8 waves per CU to approach the HBM limit (measured:
// about 2.9 TB/s with 4 waves per CU, 4.7-5.6 TB/s with 8).
constexpr int kDecodeWgPerCu = 2;

int ring_depth(int64_t workgroups) { return workgroups <= cu_count() ? 4 : 2; }

template <int D, bool BIG, bool SELECT = false, int NG = 4>
hipError_t launch_decode_mfma(const AttnArgs &A, int G, dim3 grid, const LayerPtrs &Lp, hipStream_t st) {
    // SELECT: the table holds the whole selection (slot p = position p) and a
    // wave reads up to kBigTabSlots slots past its first one
    const size_t lds = (size_t)kWgWaves * (D * kSlotBytes + (BIG ? kBigTabBytes : 0)) + (SELECT ? kBigTabBytes : 0);
    const hipError_t attr = enable_dyn_lds((const void *)attn_decode_mfma_kernel<D, BIG, SELECT, NG>, (int)lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((attn_decode_mfma_kernel<D, BIG, SELECT, NG>), grid, dim3(kWgWaves * kWave), lds, st, A, G,
                       Lp);
    return hipGetLastError();
}

// Largest share of one wave, in slots: ceil(ceil(K / n_part) / kWgWaves).
// Past 2 * kWave the registers tab0 / tab1 cannot hold the share and the
// kernel keeps the slot table in LDS.
bool big_table(const AttnArgs &A) {
    const int per = (A.K + A.n_part - 1) / A.n_part;
    return (per + kWgWaves - 1) / kWgWaves > 2 * kWave;
}

template <bool BF16>
hipError_t launch_attn_t(const AttnArgs &A, int G, bool mfma, hipStream_t st, const LayerPtrs &Lp,
                         int n_layers = 1) {
    const int64_t waves = A.total_q * A.n_part * A.hkv;
    dim3 grid((unsigned)((waves + kWgWaves - 1) / kWgWaves));
    dim3 block(kWgWaves * kWave);
    hipError_t e = hipSuccess;
    if constexpr (BF16) {
        if (mfma) {
            // one workgroup per (query, KV head, part) [x layer]
            grid = dim3((unsigned)(A.total_q * A.hkv * A.n_part), (unsigned)n_layers);
            const int D = ring_depth((int64_t)grid.x * n_layers);
            const bool big = big_table(A);
            trace("attn decode lds ring D=%d workgroups=%u layers=%d lds_table=%d", D, grid.x, n_layers, (int)big);
            if (big)
                e = D == 4 ? launch_decode_mfma<4, true>(A, G, grid, Lp, st)
                           : launch_decode_mfma<2, true>(A, G, grid, Lp, st);
            else
                e = D == 4 ? launch_decode_mfma<4, false>(A, G, grid, Lp, st)
                           : launch_decode_mfma<2, false>(A, G, grid, Lp, st);
        } else {
            switch (G) {
            case 1: hipLaunchKernelGGL((attn_kernel_w3<BF16, 1>), grid, block, 0, st, A); break;
            case 2: hipLaunchKernelGGL((attn_kernel_w3<BF16, 2>), grid, block, 0, st, A); break;
            case 4: hipLaunchKernelGGL((attn_kernel_w3<BF16, 4>), grid, block, 0, st, A); break;
            case 8: hipLaunchKernelGGL((attn_kernel<BF16, 8>), grid, block, 0, st, A); break;
            default: hipLaunchKernelGGL((attn_kernel<BF16, 16>), grid, block, 0, st, A); break;
            }
            e = hipGetLastError();
        }
    } else {
        switch (G) {
        case 1: hipLaunchKernelGGL((attn_kernel<BF16, 1>), grid, block, 0, st, A); break;
        case 2: hipLaunchKernelGGL((attn_kernel<BF16, 2>), grid, block, 0, st, A); break;
        case 4: hipLaunchKernelGGL((attn_kernel<BF16, 4>), grid, block, 0, st, A); break;
        case 8: hipLaunchKernelGGL((attn_kernel<BF16, 8>), grid, block, 0, st, A); break;
        default: hipLaunchKernelGGL((attn_kernel<BF16, 16>), grid, block, 0, st, A); break;
        }
        e = hipGetLastError();
    }
    if (e != hipSuccess || A.n_part == 1) return e;
    const int64_t rows = A.total_q * A.hq;
    dim3 cgrid((unsigned)((rows + kWgWaves - 1) / kWgWaves), (unsigned)n_layers);
    hipLaunchKernelGGL((attn_combine_kernel<BF16>), cgrid, block, 0, st, A.ws_o, A.ws_ml, A.n_part,
                       rows, A.out, Lp);
    return hipGetLastError();
}

}  // namespace

#ifndef QSA_ATTN_WIDE_TU
int attn_num_splits(const qsa_batch &b, const qsa_attn &a, int budget, int ratio, bool decode) {
    (void)b; (void)a;
    // Parts per query of the register-staged kernel (fp32, or bf16 rows past
    // 32-bit offsets): decode cuts the K selected blocks into runs of 32 (at
    // most 16 runs); prefill keeps one part per (query, KV head).  This is
    // also the most parts any decode launch uses, so it sizes the workspace.
    if (!decode) return 1;
    const int K = budget / ratio;
    int s = K / 32;
    if (s > 16) s = 16;
    if (s < 1) s = 1;
    return s;
}

#endif  // QSA_ATTN_WIDE_TU

namespace {
// Parts per (query, KV head) of the matrix-core decode kernel: enough
// workgroups for about one per CU, each part keeping at least 256 tokens
// (4 waves x 4 steps); at most the register kernel's count, so the
// workspace bound holds.  Depends on the batch size, so a query's output
// may differ in the last bits between batch sizes (the split of its
// reduction changes), never between runs of the same batch.
int mfma_decode_parts(const qsa_batch &b, const qsa_attn &a, int budget, int ratio) {
    const int64_t units = b.total_q * (int64_t)a.hkv;
    const int64_t want = (kDecodeWgPerCu * cu_count() + units - 1) / (units > 0 ? units : 1);
    const int64_t cap_tokens = ((int64_t)budget) / 256;
    int64_t p = want < cap_tokens ? want : cap_tokens;
    const int reg_parts = attn_num_splits(b, a, budget, ratio, true);
    if (p > reg_parts) p = reg_parts;
    return p < 1 ? 1 : (int)p;
}
}  // namespace

#ifndef QSA_ATTN_WIDE_TU
size_t attn_workspace_bytes(const qsa_batch &b, const qsa_attn &a, int budget, int ratio) {
    const int parts = attn_num_splits(b, a, budget, ratio, true);
    if (parts <= 1) return 0;
    const size_t rows = (size_t)b.total_q * (size_t)a.hq * (size_t)parts;
    return rows * (kD + 2) * sizeof(float) + 256;
}

#endif  // QSA_ATTN_WIDE_TU

namespace {
// Kernel arguments of one attention call; returns whether the matrix-core
// kernel runs it.
bool attn_args(const qsa_attn &a, const int32_t *idx, int budget, int ratio, const qsa_batch &b, void *out,
               void *ws, bool decode, const qsa_paged_kv *pg, AttnArgs &A) {
    A.q = a.q; A.k = a.k; A.v = a.v; A.idx = idx;
    A.kv_off = b.kv_offsets; A.q_off = b.q_offsets;
    A.num_seqs = b.num_seqs; A.hq = a.hq; A.hkv = a.hkv;
    A.log2r = __builtin_ctz((unsigned)ratio);
    A.K = budget / ratio;
    // The matrix-core decode kernel addresses a sequence's K/V rows with
    // 32-bit byte offsets; longer sequences (larger pools) take the register-staged kernel.
    // With paged K/V the offsets address the whole pool.
    const uint64_t span_rows = pg ? (uint64_t)pg->num_pages * (uint64_t)pg->page_size : (uint64_t)b.max_kv_len;
    const bool rows32 = span_rows * (uint64_t)a.hkv * kD * 2 < (1ull << 32);
    A.pm = page_map(pg);
    // bf16 decode and prefill both run on the matrix-core kernel; prefill
    // keeps one part per (query, KV head), so its result never depends on
    // the rest of the batch (chunked prefill equals single-shot bit for bit).
    const bool mfma_path = a.dtype == QSA_BF16 && rows32;
    A.n_part = mfma_path ? (decode ? mfma_decode_parts(b, a, budget, ratio) : 1)
                         : attn_num_splits(b, a, budget, ratio, decode);
    A.c = a.softmax_scale * kLog2e;
    A.total_q = b.total_q;
    A.out = out;
    const size_t rows = (size_t)b.total_q * (size_t)a.hq * (size_t)A.n_part;
    A.ws_o = static_cast<float *>(ws);
    A.ws_ml = A.n_part > 1 ? static_cast<float *>(ws) + rows * kD : nullptr;
    return mfma_path;
}
// Decode attention that selects from the lists, with NG register groups.
template <int NG>
hipError_t attn_select_impl(const qsa_attn &a, int budget, int ratio, const qsa_batch &b, const ListArgs &la,
                            const float *scores, int64_t ld, int32_t *idx, void *out, void *ws,
                            const qsa_paged_kv *pg, hipStream_t st) {
    if (b.total_q == 0) return hipSuccess;
    AttnArgs A{};
    if (!attn_args(a, idx, budget, ratio, b, out, ws, true, pg, A)) return hipErrorNotSupported;
    A.la = la;
    A.scores = scores;
    A.ld = ld;
    A.idx_out = idx;
    // only the entries a row of at most max_kv_len tokens can list are
    // requested before the row's length is known
    const int64_t pref = list_max_entries(b.max_kv_len / ratio, la.K);
    A.sel_pref = (int32_t)(pref < sel_reg_entries(NG) ? pref : sel_reg_entries(NG));
    const int G = a.hq / a.hkv;
    const dim3 grid((unsigned)(A.total_q * A.hkv * A.n_part));
    const int D = ring_depth((int64_t)grid.x);
    trace("attn decode with selection D=%d workgroups=%u parts=%d groups=%d", D, grid.x, A.n_part, NG);
    const LayerPtrs none{};
    hipError_t e = D == 4 ? launch_decode_mfma<4, true, true, NG>(A, G, grid, none, st)
                          : launch_decode_mfma<2, true, true, NG>(A, G, grid, none, st);
    if (e != hipSuccess || A.n_part == 1) return e;
    const int64_t rows = A.total_q * A.hq;
    dim3 cgrid((unsigned)((rows + kWgWaves - 1) / kWgWaves));
    hipLaunchKernelGGL((attn_combine_kernel<true>), cgrid, dim3(kWgWaves * kWave), 0, st, A.ws_o, A.ws_ml, A.n_part,
                       rows, A.out, none);
    return hipGetLastError();
}
}  // namespace

#ifndef QSA_ATTN_WIDE_TU
hipError_t launch_attn(const qsa_attn &a, const int32_t *idx, int budget, int ratio,
                       const qsa_batch &b, void *out, void *ws, bool decode, const qsa_paged_kv *pg,
                       hipStream_t st) {
    if (b.total_q == 0) return hipSuccess;
    AttnArgs A{};
    const bool mfma_path = attn_args(a, idx, budget, ratio, b, out, ws, decode, pg, A);
    const int G = a.hq / a.hkv;
    trace("attn total_q=%lld hkv=%d G=%d parts=%d dtype=%d", (long long)b.total_q, a.hkv, G,
          A.n_part, a.dtype);
    const LayerPtrs none{};
    return a.dtype == QSA_BF16 ? launch_attn_t<true>(A, G, mfma_path, st, none)
                                : launch_attn_t<false>(A, G, false, st, none);
}

// ---------------------------------------------------------------------------
// Decode attention without a caller workspace, for callers that cannot
// allocate: the split partials live in `scratch`, a file-scope device array
// that every GPU the library runs on holds until the process ends.  Host
// code never passes the array's name to a kernel (in host code it is only a
// stand-in for the symbol); the device address is resolved once per device
// with hipGetSymbolAddress and kept.  All calls on one GPU share the array,
// so calls that overlap on one GPU race.
static __device__ __align__(256) uint8_t scratch[kAttnStaticScratchBytes];

hipError_t attn_static_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    static std::mutex mu;
    static void *addr[kMaxScratchDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

bool attn_select_supported(const qsa_batch &b, const qsa_attn &a, const qsa_paged_kv *pg) {
    const uint64_t span_rows = pg ? (uint64_t)pg->num_pages * (uint64_t)pg->page_size : (uint64_t)b.max_kv_len;
    return a.dtype == QSA_BF16 && span_rows * (uint64_t)a.hkv * kD * 2 < (1ull << 32);
}

hipError_t launch_attn_select(const qsa_attn &a, int budget, int ratio, const qsa_batch &b, const ListArgs &la,
                              const float *scores, int64_t ld, int32_t *idx, void *out, void *ws,
                              const qsa_paged_kv *pg, hipStream_t st) {
    // batches whose rows of the longest length list more than 4096 entries
    // (32768 blocks at K = 2048) take the 8-group register path, built in a
    // translation unit of its own: instantiated here, the 8-group kernels
    // changed the register allocation of the 4-group ones (a third more
    // scalar spills).  The count is not monotone in the length, so shorter
    // rows can list more than the longest (up to 6656 entries for rows under
    // 32768 blocks at K = 512); those take the LDS path of either kernel.
    const int64_t nb_max = b.max_kv_len / ratio;
    const int64_t m_max = nb_max > la.K ? (nb_max + kListChunk - 1) / kListChunk * list_len(nb_max, la.K) : 0;
    if (m_max > sel_reg_entries(4))
        return launch_attn_select_wide(a, budget, ratio, b, la, scores, ld, idx, out, ws, pg, st);
    return attn_select_impl<4>(a, budget, ratio, b, la, scores, ld, idx, out, ws, pg, st);
}

size_t attn_layer_stride_bytes(const qsa_batch &b, const qsa_attn &a, int budget, int ratio) {
    return (attn_workspace_bytes(b, a, budget, ratio) + 255) & ~(size_t)255;
}

hipError_t launch_attn_layers(const qsa_attn *layers, int n_layers, const int32_t *idx, int budget, int ratio,
                              const qsa_batch &b, void *const *outs, void *ws, const qsa_paged_kv *pg,
                              hipStream_t st) {
    if (b.total_q == 0) return hipSuccess;
    const size_t stride = attn_layer_stride_bytes(b, layers[0], budget, ratio);
    AttnArgs A{};
    const bool mfma_path = attn_args(layers[0], idx, budget, ratio, b, outs[0], ws, true, pg, A);
    const int G = layers[0].hq / layers[0].hkv;
    if (!mfma_path || n_layers == 1) {   // one launch per layer
        for (int l = 0; l < n_layers; ++l) {
            hipError_t e = launch_attn(layers[l], idx, budget, ratio, b, outs[l],
                                       static_cast<uint8_t *>(ws) + l * stride, true, pg, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    LayerPtrs Lp{};
    for (int l = 0; l < n_layers; ++l) {
        Lp.q[l] = layers[l].q; Lp.k[l] = layers[l].k; Lp.v[l] = layers[l].v; Lp.out[l] = outs[l];
        Lp.c[l] = layers[l].softmax_scale * kLog2e;
    }
    Lp.ws_stride = (int64_t)(stride / sizeof(float));
    trace("attn layers=%d total_q=%lld hkv=%d G=%d parts=%d", n_layers, (long long)b.total_q,
          layers[0].hkv, G, A.n_part);
    return launch_attn_t<true>(A, G, true, st, Lp, n_layers);
}

#endif  // QSA_ATTN_WIDE_TU

}  // namespace qsa
