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
// Work decomposition: one wave per (query, KV head, split); a split owns a
// contiguous range of selected slots (the last split also owns the tail).
// The G = hq/hkv query heads of the KV head share every K/V load.  Tokens are
// processed 16 at a time:
//  * QK: lane (tk = lane/8, ds = lane%8) loads dims ds*16..+16 of tokens tk
//    and tk+8 straight from HBM and forms partial dots for all G heads
//    (bf16: v_dot2_f32_bf16); a transpose-reduce across the 8 ds lanes leaves
//    each lane with full dots of G/8 heads (or a shared head for G < 8).
//  * online softmax in fp32 (exp2 domain), one running max per head.
//  * PV: lane p owns dims 2p, 2p+1 of every head; V rows are read as one
//    coalesced row per token; fp32 probabilities come through a small
//    per-wave LDS slot and meet fp32-widened V in plain FMAs.  (Rounding the
//    probabilities to bf16 for a packed dot would cost up to 2^-8 relative per
//    weight, which is visible when only a few tokens carry the softmax.)
// With more than one split, unnormalised (m, l, o) partials go to the
// workspace and a combine kernel merges them.
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {
namespace {

constexpr int kD = 128;
constexpr int kAttnWaves = 4;
constexpr int kStep = 16;               // tokens per step
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
    const void *q, *k, *v;
    const int32_t *idx;
    const int64_t *kv_off, *q_off;
    int num_seqs, hq, hkv, log2r, K, n_split;
    float c;                 // softmax_scale * log2(e)
    int64_t total_q;
    void *out;
    float *ws_o;             // [total_q, hq, n_split, D]
    float *ws_ml;            // [total_q, hq, n_split, 2]
};

// log2 of a power of two known at compile time
template <int G>
constexpr int ilog2() { return G <= 1 ? 0 : 1 + ilog2<G / 2>(); }

// One step of the transpose-reduce: keep half of the array (upper half when
// `upper`), add the partner's copy of that half.
template <int N>
__device__ __forceinline__ void tr_step(const float (&a)[N], float (&o)[N / 2], bool upper, int xm) {
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
        const float mine = upper ? a[N / 2 + j] : a[j];
        const float send = upper ? a[j] : a[N / 2 + j];
        o[j] = mine + __shfl_xor(send, xm, kWave);
    }
}

// Reduce G partial sums over the 8 ds-lanes; returns NH = max(1, G/8) sums.
template <int G>
__device__ __forceinline__ void transpose_reduce(const float (&p)[G], float (&r)[(G >= 8 ? G / 8 : 1)],
                                                 int ds) {
    if constexpr (G >= 8) {
        float a4[G / 2], a2[G / 4];
        tr_step<G>(p, a4, ds & 4, 4);
        tr_step<G / 2>(a4, a2, ds & 2, 2);
        tr_step<G / 4>(a2, r, ds & 1, 1);
    } else if constexpr (G == 4) {
        float a4[2], a2[1];
        tr_step<4>(p, a4, ds & 4, 4);
        tr_step<2>(a4, a2, ds & 2, 2);
        r[0] = a2[0] + __shfl_xor(a2[0], 1, kWave);
    } else if constexpr (G == 2) {
        float a4[1];
        tr_step<2>(p, a4, ds & 4, 4);
        float x = a4[0] + __shfl_xor(a4[0], 2, kWave);
        r[0] = x + __shfl_xor(x, 1, kWave);
    } else {
        float x = p[0] + __shfl_xor(p[0], 4, kWave);
        x = x + __shfl_xor(x, 2, kWave);
        r[0] = x + __shfl_xor(x, 1, kWave);
    }
}

template <int G>
__device__ __forceinline__ int head_base(int ds) {
    if constexpr (G >= 8) return ds * (G / 8);
    else return ds >> (3 - ilog2<G>());
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Token position of flat token t of this split (-1 if t is past the end).
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
    const int32_t *__restrict__ sel;  // idx row + first slot of this split
    int nslot;                        // selected slots of the split
    int nblk_tok;                     // tokens from selected blocks
    int ntok;                         // + tail tokens
    int64_t tail0;                    // first tail position (ratio * nb)
    int64_t nb;                       // complete blocks visible to the query
    int log2r;
};

// Issue the loads of step `st`.  Lane t < 16 resolves token t0+t to a row of
// the sequence (a selected block id from the slot table held one slot per
// lane, or a tail position; malformed ids and positions past the end give
// "no token" and read row 0).  K rows reach the QK lanes by a cross-lane
// permute; V rows become wave-uniform addresses, so each V row is one
// coalesced scalar-based load.
template <bool BF16>
__device__ __forceinline__ void issue_step(const WaveWork &W, int st, int lane, int tk, int ds,
                                           uint32_t slot_tab, int tab_base,
                                           const typename KVTypes<BF16>::elem *__restrict__ kbase,
                                           const typename KVTypes<BF16>::elem *__restrict__ vbase,
                                           int64_t row_stride, StepBuf<BF16> &B) {
    using T = typename KVTypes<BF16>::elem;
    constexpr int KW = StepBuf<BF16>::KW;
    const int t = st * kStep + (lane & (kStep - 1));
    // The permute runs with every lane active: a lane that is switched off
    // does not supply its value to the others.
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
    // K: lane (tk, ds) takes tokens tk and tk+8
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
    // V: one coalesced row per token, wave-uniform base address
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

template <bool BF16, int G>
struct AttnState {
    static constexpr int NH = G >= 8 ? G / 8 : 1;
    float m_run[NH], l_run[NH];
    float o[G][2];
};

// Consume one step: QK, online softmax, PV.
template <bool BF16, int G>
__device__ __forceinline__ void compute_step(const StepBuf<BF16> &B,
                                             const uint32_t (&qr)[G][KVTypes<BF16>::kDwordsPerLaneK],
                                             float c, int tk, int ds, int hb,
                                             float (*sh_p)[G], float *sh_alpha,
                                             AttnState<BF16, G> &S) {
    constexpr int NH = AttnState<BF16, G>::NH;
    constexpr int KW = KVTypes<BF16>::kDwordsPerLaneK;
    // ---- QK partial dots over this lane's 16 dims
    float dA[G], dB[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float a = 0.0f, b = 0.0f;
        if constexpr (BF16) {
            typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int e = 0; e < KW; ++e) {
                const bf2 qv = __builtin_bit_cast(bf2, qr[h][e]);
                a = __builtin_amdgcn_fdot2_f32_bf16(qv, __builtin_bit_cast(bf2, B.kA[e]), a, false);
                b = __builtin_amdgcn_fdot2_f32_bf16(qv, __builtin_bit_cast(bf2, B.kB[e]), b, false);
            }
        } else {
#pragma unroll
            for (int e = 0; e < KW; ++e) {
                const float qv = __uint_as_float(qr[h][e]);
                a = __builtin_fmaf(qv, __uint_as_float(B.kA[e]), a);
                b = __builtin_fmaf(qv, __uint_as_float(B.kB[e]), b);
            }
        }
        dA[h] = a;
        dB[h] = b;
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
        float mx = fmaxf(xa, xb);
        mx = fmaxf(mx, __shfl_xor(mx, 8, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
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
    wave_lds_sync();
}

template <bool BF16, int G>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_kernel(AttnArgs A) {
    using T = typename KVTypes<BF16>::elem;
    constexpr int NH = AttnState<BF16, G>::NH;
    constexpr int KW = KVTypes<BF16>::kDwordsPerLaneK;
    __shared__ float sh_p[kAttnWaves][kStep][G];   // probabilities [token][head]
    __shared__ float sh_alpha[kAttnWaves][G];
    __shared__ float sh_l[kAttnWaves][G];

    const int lane = threadIdx.x & (kWave - 1);
    // The wave index is uniform across the wave; saying so keeps everything
    // derived from it (query, split, positions) in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t wid = (int64_t)blockIdx.x * kAttnWaves + wave;
    const int g = (int)(wid % A.hkv);
    const int64_t t2 = wid / A.hkv;
    const int c = (int)(t2 % A.n_split);
    const int64_t i = t2 / A.n_split;
    if (i >= A.total_q) return;

    const QueryPos qp = query_pos(A.kv_off, nullptr, A.q_off, A.num_seqs, i);
    const int64_t nb = qp.L >> A.log2r;
    const int64_t nsel = nb < A.K ? nb : (int64_t)A.K;
    const int64_t per = (nsel + A.n_split - 1) / A.n_split;
    const int64_t s_beg = imin64((int64_t)c * per, nsel);
    const int64_t s_end = imin64(s_beg + per, nsel);
    WaveWork W;
    W.sel = A.idx + i * (int64_t)A.K + s_beg;
    W.nslot = (int)(s_end - s_beg);
    W.log2r = A.log2r;
    W.nblk_tok = W.nslot << A.log2r;
    W.tail0 = nb << A.log2r;
    W.nb = nb;
    W.ntok = W.nblk_tok + ((c == A.n_split - 1) ? (int)(qp.L - W.tail0) : 0);

    const int tk = lane >> 3, ds = lane & 7;
    const int hb = head_base<G>(ds);
    const int qh0 = g * G;                          // first query head of this KV head
    const int64_t row_stride = (int64_t)A.hkv * kD; // elements between consecutive tokens
    const T *__restrict__ kbase = static_cast<const T *>(A.k) + (qp.kv_row0 * A.hkv + g) * kD;
    const T *__restrict__ vbase = static_cast<const T *>(A.v) + (qp.kv_row0 * A.hkv + g) * kD;

    // q slice for the QK lane mapping: heads qh0..qh0+G-1, dims ds*16..+16
    uint32_t qr[G][KW];
    {
        const T *qp_ = static_cast<const T *>(A.q) + (i * A.hq + qh0) * kD + ds * 16;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint4 *src = reinterpret_cast<const uint4 *>(qp_ + h * kD);
#pragma unroll
            for (int c4 = 0; c4 < KW / 4; ++c4) {
                const uint4 x = src[c4];
                qr[h][4 * c4 + 0] = x.x; qr[h][4 * c4 + 1] = x.y;
                qr[h][4 * c4 + 2] = x.z; qr[h][4 * c4 + 3] = x.w;
            }
        }
    }

    AttnState<BF16, G> S;
#pragma unroll
    for (int h = 0; h < NH; ++h) { S.m_run[h] = -INFINITY; S.l_run[h] = 0.0f; }
#pragma unroll
    for (int h = 0; h < G; ++h) { S.o[h][0] = 0.0f; S.o[h][1] = 0.0f; }

    // Slot table: lane j holds selected block id of slot tab_base + j.
    int tab_base = 0;
    uint32_t slot_tab = (uint32_t)(lane < W.nslot ? W.sel[lane] : -1);
    const int nsteps = (W.ntok + kStep - 1) / kStep;
    // slots a step touches: [ (16*st) >> log2r, (16*st + 15) >> log2r ]
    auto ensure_table = [&](int st) {
        const int first = (st * kStep) >> W.log2r;
        const int last = (st * kStep + kStep - 1) >> W.log2r;
        if (st * kStep < W.nblk_tok && (first < tab_base || last >= tab_base + kWave)) {
            tab_base = first;
            slot_tab = (uint32_t)(tab_base + lane < W.nslot ? W.sel[tab_base + lane] : -1);
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
        compute_step<BF16, G>(b0, qr, A.c, tk, ds, hb, sh_p[wave], sh_alpha[wave], S);
        if (st + 1 >= nsteps) break;
        if (st + 2 < nsteps) {
            ensure_table(st + 2);
            issue_step<BF16>(W, st + 2, lane, tk, ds, slot_tab, tab_base, kbase, vbase, row_stride, b0);
        }
        compute_step<BF16, G>(b1, qr, A.c, tk, ds, hb, sh_p[wave], sh_alpha[wave], S);
    }

    // ---- denominators: sum the per-lane partials over the 8 token lanes
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        float l = S.l_run[h];
        l = l + __shfl_xor(l, 8, kWave);
        l = l + __shfl_xor(l, 16, kWave);
        l = l + __shfl_xor(l, 32, kWave);
        if (tk == 0) {
            sh_l[wave][hb + h] = l;
            sh_alpha[wave][hb + h] = S.m_run[h];    // reuse slot for the running max
        }
    }
    wave_lds_sync();

    if (A.n_split == 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float l = sh_l[wave][h];
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            const float r0 = S.o[h][0] * inv, r1 = S.o[h][1] * inv;
            const int64_t off = (i * A.hq + qh0 + h) * kD + 2 * lane;
            if constexpr (BF16) {
                reinterpret_cast<uint32_t *>(A.out)[off >> 1] = pack_bf16x2(r0, r1);
            } else {
                reinterpret_cast<float2 *>(A.out)[off >> 1] = make_float2(r0, r1);
            }
        }
    } else {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const int64_t slot = (i * A.hq + qh0 + h) * A.n_split + c;
            reinterpret_cast<float2 *>(A.ws_o + slot * kD)[lane] = make_float2(S.o[h][0], S.o[h][1]);
            if (lane == 0) {
                A.ws_ml[slot * 2 + 0] = sh_alpha[wave][h];
                A.ws_ml[slot * 2 + 1] = sh_l[wave][h];
            }
        }
    }
}

// Merge split partials: one wave per (query, head); lane s < n_split reads
// split s's (m, l), the wave forms the weights, then every lane accumulates
// dims 2p, 2p+1 over the splits (all partial loads issued together).
constexpr int kMaxSplits = 16;

template <bool BF16>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_combine_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_ml, int n_split, int64_t rows,
    void *__restrict__ out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t r = (int64_t)blockIdx.x * kAttnWaves + wave;   // query*hq + head
    if (r >= rows) return;
    const float *ml = ws_ml + r * n_split * 2;
    float2 os[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
        if (s < n_split) os[s] = reinterpret_cast<const float2 *>(ws_o + (r * n_split + s) * kD)[lane];
    const float m_s = lane < n_split ? ml[2 * lane] : -INFINITY;
    const float l_s = lane < n_split ? ml[2 * lane + 1] : 0.0f;
    const float mmax = wave_max(m_s);
    const float msafe = mmax == -INFINITY ? 0.0f : mmax;
    const float w_s = l_s > 0.0f ? exp2f(m_s - msafe) : 0.0f;
    const float l = wave_sum(w_s * l_s);
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
        if (s < n_split) {
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

template <bool BF16>
hipError_t launch_attn_t(const AttnArgs &A, int G, hipStream_t st) {
    const int64_t waves = A.total_q * A.n_split * A.hkv;
    dim3 grid((unsigned)((waves + kAttnWaves - 1) / kAttnWaves));
    dim3 block(kAttnWaves * kWave);
    switch (G) {
    case 1: hipLaunchKernelGGL((attn_kernel<BF16, 1>), grid, block, 0, st, A); break;
    case 2: hipLaunchKernelGGL((attn_kernel<BF16, 2>), grid, block, 0, st, A); break;
    case 4: hipLaunchKernelGGL((attn_kernel<BF16, 4>), grid, block, 0, st, A); break;
    case 8: hipLaunchKernelGGL((attn_kernel<BF16, 8>), grid, block, 0, st, A); break;
    default: hipLaunchKernelGGL((attn_kernel<BF16, 16>), grid, block, 0, st, A); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || A.n_split == 1) return e;
    const int64_t rows = A.total_q * A.hq;
    dim3 cgrid((unsigned)((rows + kAttnWaves - 1) / kAttnWaves));
    hipLaunchKernelGGL((attn_combine_kernel<BF16>), cgrid, block, 0, st, A.ws_o, A.ws_ml,
                       A.n_split, rows, A.out);
    return hipGetLastError();
}

}  // namespace

int attn_num_splits(const qsa_batch &b, const qsa_attn &a, int budget, int ratio, bool decode) {
    (void)b; (void)a;
    // The split count depends on K alone (decode) or is 1 (prefill), never on
    // how many queries share the launch: a query's fp32 accumulation order is
    // then the same in any batch, so chunked prefill equals single-shot
    // prefill bit for bit.  Decode splits the K selected blocks into runs of
    // 32 (at most 16 runs); prefill has enough queries to fill the chip.
    if (!decode) return 1;
    const int K = budget / ratio;
    int s = K / 32;
    if (s > 16) s = 16;
    if (s < 1) s = 1;
    return s;
}

size_t attn_workspace_bytes(const qsa_batch &b, const qsa_attn &a, int budget, int ratio) {
    const int s = attn_num_splits(b, a, budget, ratio, true);
    if (s <= 1) return 0;
    const size_t rows = (size_t)b.total_q * (size_t)a.hq * (size_t)s;
    return rows * (kD + 2) * sizeof(float) + 256;
}

hipError_t launch_attn(const qsa_attn &a, const int32_t *idx, int budget, int ratio,
                       const qsa_batch &b, void *out, void *ws, bool decode, hipStream_t st) {
    if (b.total_q == 0) return hipSuccess;
    AttnArgs A;
    A.q = a.q; A.k = a.k; A.v = a.v; A.idx = idx;
    A.kv_off = b.kv_offsets; A.q_off = b.q_offsets;
    A.num_seqs = b.num_seqs; A.hq = a.hq; A.hkv = a.hkv;
    A.log2r = __builtin_ctz((unsigned)ratio);
    A.K = budget / ratio;
    A.n_split = attn_num_splits(b, a, budget, ratio, decode);
    A.c = a.softmax_scale * kLog2e;
    A.total_q = b.total_q;
    A.out = out;
    const size_t rows = (size_t)b.total_q * (size_t)a.hq * (size_t)A.n_split;
    A.ws_o = static_cast<float *>(ws);
    A.ws_ml = A.n_split > 1 ? static_cast<float *>(ws) + rows * kD : nullptr;
    const int G = a.hq / a.hkv;
    trace("attn total_q=%lld hkv=%d G=%d splits=%d dtype=%d", (long long)b.total_q, a.hkv, G,
          A.n_split, a.dtype);
    return a.dtype == QSA_BF16 ? launch_attn_t<true>(A, G, st) : launch_attn_t<false>(A, G, st);
}

}  // namespace qsa
