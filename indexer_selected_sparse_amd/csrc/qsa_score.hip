// Indexer scores, canonical (bit-defined) form.
//
// s_b = sum_h w_h * ReLU(q_idx[h] . kc_b)  — "Agentic shootout" page, "PR 16
// review" section (a): a 4Q+1K indexer with a relu score over 4-token
// mean-pooled blocks; the single key head is the vLLM report's validator
// (indexer kv heads == 1, section (a)1).  For e4m3 keys the dot runs over the
// code values and is then multiplied by the block's fp32 scale.  For fp4 keys
// ("ATOM Model Support Guide" page, DeepSeek-V4.1: E2M1 values with E8M0
// scales) each key value is its code value times its 32-dim group's power of
// two, exact in fp32, and the dot runs over those values.
//
// The score decides an integer (the selection), so it is evaluated in one
// fixed fp32 order that the CPU oracle follows too: for each head, a
// left-to-right sum over d of rounded products; ReLU; then a left-to-right
// sum over heads of rounded w_h * r_h.  A product of bf16 by bf16 (or by an
// e4m3 code) is exact in fp32, so a fused multiply-add there gives the same
// bits as multiply-then-add; fp32 inputs use a separate multiply and add.
//
// Decode is a GEMV per query.  One lane owns one block (a compressed key
// row); the query's H x D values are wave-uniform and reach the FMAs through
// the scalar unit.  Workgroup = 256 blocks of one query; blocks that are not
// yet visible to the query (b >= floor(L/ratio)) are skipped.  With bf16
// queries and bf16 / e4m3 keys the arithmetic is H*D fused multiply-adds per
// block on the vector ALU (the canonical order admits no packed or matrix
// form), which for decode batches takes about as long as reading the keys.
#include <type_traits>

#include "qsa_device.hpp"
#include "qsa_ingest.hpp"
#include "qsa_internal.hpp"
#include "qsa_lists.hpp"

namespace qsa {
namespace {

constexpr int kScoreThreads = 256;

// fp4 index plane: a byte holds two E2M1 codes (tag type of the key row).
struct Fp4x2 {
    uint8_t v;
};
template <typename KT>
struct KeyBits {
    static constexpr int value = 8 * (int)sizeof(KT);
};
template <>
struct KeyBits<Fp4x2> {
    static constexpr int value = 4;
};

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

// At least one fp32 operand: products are rounded, so multiply and add are
// separate operations.  The key row is widened once to fp32 and kept in
// registers; the query values are wave-uniform and come through the scalar
// unit.
template <typename QT, typename KT, int D, int H>
__global__ __launch_bounds__(kScoreThreads) void score_rounded_kernel(
    const QT *__restrict__ q_idx, const float *__restrict__ w, const KT *__restrict__ kc,
    const float *__restrict__ kc_scale, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ blk_off, const int64_t *__restrict__ q_off, int num_seqs,
    int log2r, float *__restrict__ scores, int64_t ld, PageMap pm, ListArgs la) {
    constexpr bool kE4M3 = std::is_same<KT, uint8_t>::value;
    const int64_t i = blockIdx.x;
    if (la.mode && i == 0 && blockIdx.y == 0 && threadIdx.x == 0) *la.mode = 0u;   // plain lists
    const QueryPos qp = query_pos(kv_off, blk_off, q_off, num_seqs, i);
    const int64_t nb = qp.L >> log2r;
    const int64_t b = (int64_t)blockIdx.y * kScoreThreads + threadIdx.x;
    if ((int64_t)blockIdx.y * kScoreThreads >= nb) return;   // whole workgroup invisible
    const bool active = b < nb;
    const int64_t row = pm.table ? paged_row(pm, qp.seq, active ? b : 0, pm.log2_page - log2r)
                                 : qp.blk_row0 + (active ? b : 0);

    const float sc = kE4M3 ? kc_scale[row] : 1.0f;
    const float *__restrict__ wi = w + i * (int64_t)H;
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
    float s = 0.0f;
#pragma unroll 1
    for (int h = 0; h < H; ++h) {
        float dot = 0.0f;
#pragma unroll
        for (int d0 = 0; d0 < D; d0 += 32) {
            float qv[32];
            load_q<32>(q, h * D + d0, qv);
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const float p = qv[e] * kf[d0 + e];
                dot = dot + p;
            }
        }
        if constexpr (kE4M3) dot = dot * sc;
        const float r = dot > 0.0f ? dot : 0.0f;
        const float t = wi[h] * r;
        s = s + t;
    }
    if (active) scores[i * ld + b] = s;
    if (la.keys) emit_chunk_list(la, i, nb, b - (threadIdx.x & (kWave - 1)), active, s, threadIdx.x & (kWave - 1));
}

// Exact products (bf16 query; bf16 or e4m3 keys).  One lane owns one block;
// its whole key row is requested at once (the loads of a row go out back to
// back, so the L1 still holds each line for the later pieces of it), and the
// row is widened and used chunk by chunk (kExactChunk dims) as it lands: the
// H per-head sums advance together chunk by chunk, each in ascending d, so
// every head's chain of fused multiply-adds is the canonical one.  Widening
// one chunk at a time keeps the register footprint at one raw row, one
// widened chunk and H sums, so every workgroup of a decode batch is resident
// at once; with the whole row widened up front (128 registers for it alone)
// three workgroups fit per CU and the fourth ran as a second round on an
// otherwise idle chip.  The query values are wave-uniform: with at most 32
// (chunk, head) steps they arrive with the wave's first vector loads and
// enter the multiply-adds through DPP row broadcasts (QueryVec); longer
// query rows go through the scalar unit, one step ahead.  Measured on one
// MI355X, per-step scalar loads had put a scalar-cache miss (microseconds
// under the key traffic) in front of every step.
constexpr int kExactChunk = 32;
constexpr int kExactThreads = 256;

// The key loads and the query loads of this kernel are written as
// instructions with explicit waits.  Left to itself the compiler issues the
// chunk loads out of order (loads complete in issue order, so a wait for
// chunk 0 then also waits for later chunks) and hoists the query loads of all
// (chunk, head) steps ahead of their use until scalar registers spill.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

// One 16-byte load at byte offset OFF (key rows; query dwords).
template <int OFF>
__device__ __forceinline__ u32x4 key_load16(const void *row) {
    u32x4 r;
    asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "=v"(r) : "v"(row), "n"(OFF) : "memory");
    return r;
}
// Wait until at most N vector loads are outstanding; the registers of the
// chunk that is about to be used are tied to the wait so that nothing reads
// them earlier.
template <int N, int L>
__device__ __forceinline__ void key_wait(u32x4 (&u)[L]) {
    static_assert(L == 1 || L == 2 || L == 4, "chunk of 1, 2 or 4 loads");
    if constexpr (L == 1)
        asm volatile("s_waitcnt vmcnt(%1)" : "+v"(u[0]) : "n"(N));
    else if constexpr (L == 2)
        asm volatile("s_waitcnt vmcnt(%2)" : "+v"(u[0]), "+v"(u[1]) : "n"(N));
    else
        asm volatile("s_waitcnt vmcnt(%4)" : "+v"(u[0]), "+v"(u[1]), "+v"(u[2]), "+v"(u[3]) : "n"(N));
}
// On the scalar query path, 16 wave-uniform dwords per (chunk, head) step go
// through the scalar unit into scalar registers one step ahead: a step's
// wait and the next step's load are one statement, so the load is in flight
// while the step's FMAs run.  The wait is also tied to the sum the previous step wrote
// (so that step is finished and only two steps' values are live).  Scalar
// loads may complete out of order, hence lgkmcnt(0).
template <int OFF>
__device__ __forceinline__ u32x16 query_load16(const uint32_t *p) {
    u32x16 r;
    asm volatile("s_load_dwordx16 %0, %1, %2" : "=s"(r) : "s"(p), "n"(OFF) : "memory");
    return r;
}
template <int OFF>
__device__ __forceinline__ u32x16 query_wait_load16(u32x16 &cur, float &prev, const uint32_t *p) {
    u32x16 nxt;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_load_dwordx16 %0, %3, %4"
                 : "=&s"(nxt), "+s"(cur), "+v"(prev) : "s"(p), "n"(OFF) : "memory");
    return nxt;
}
template <int OFF>
__device__ __forceinline__ u32x16 query_wait_load16(u32x16 &cur, const uint32_t *p) {
    u32x16 nxt;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_load_dwordx16 %0, %2, %3"
                 : "=&s"(nxt), "+s"(cur) : "s"(p), "n"(OFF) : "memory");
    return nxt;
}
__device__ __forceinline__ void query_wait(u32x16 &u, float &prev) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(u), "+v"(prev));
}

// The E8M0 scale bytes of this lane's fp4 row (D/32 of them), requested
// before the key loads so that the wait for the first chunk covers them.
template <int D>
__device__ __forceinline__ uint32_t fp4_scale_load(const uint8_t *p) {
    uint32_t r;
    if constexpr (D == 128)
        asm volatile("global_load_dword %0, %1, off" : "=v"(r) : "v"(p) : "memory");
    else
        asm volatile("global_load_ushort %0, %1, off" : "=v"(r) : "v"(p) : "memory");
    return r;
}
// 2^(e - 127) from an E8M0 byte e (e = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    return __uint_as_float(e ? (e << 23) : 0x00400000u);
}

// Scalar query path (query rows of more than 32 steps): the row's NL
// 64-byte lines are requested into the scalar cache all at once and waited
// for in the same statement (the loads share one scratch register set, dead
// afterwards), so the (chunk, head) steps find their values there instead of
// each waiting out a miss in turn.
#define QSA_QPF(LOADS) asm volatile(LOADS "s_waitcnt lgkmcnt(0)" : "=&s"(junk) : "s"(p) : "memory")
template <int NL>
__device__ __forceinline__ void query_prefetch(const uint32_t *p) {
    u32x16 junk;
    if constexpr (NL == 32)
        QSA_QPF("s_load_dwordx16 %0, %1, 0x0\n\t" "s_load_dwordx16 %0, %1, 0x40\n\t"
            "s_load_dwordx16 %0, %1, 0x80\n\t" "s_load_dwordx16 %0, %1, 0xc0\n\t"
            "s_load_dwordx16 %0, %1, 0x100\n\t" "s_load_dwordx16 %0, %1, 0x140\n\t"
            "s_load_dwordx16 %0, %1, 0x180\n\t" "s_load_dwordx16 %0, %1, 0x1c0\n\t"
            "s_load_dwordx16 %0, %1, 0x200\n\t" "s_load_dwordx16 %0, %1, 0x240\n\t"
            "s_load_dwordx16 %0, %1, 0x280\n\t" "s_load_dwordx16 %0, %1, 0x2c0\n\t"
            "s_load_dwordx16 %0, %1, 0x300\n\t" "s_load_dwordx16 %0, %1, 0x340\n\t"
            "s_load_dwordx16 %0, %1, 0x380\n\t" "s_load_dwordx16 %0, %1, 0x3c0\n\t"
            "s_load_dwordx16 %0, %1, 0x400\n\t" "s_load_dwordx16 %0, %1, 0x440\n\t"
            "s_load_dwordx16 %0, %1, 0x480\n\t" "s_load_dwordx16 %0, %1, 0x4c0\n\t"
            "s_load_dwordx16 %0, %1, 0x500\n\t" "s_load_dwordx16 %0, %1, 0x540\n\t"
            "s_load_dwordx16 %0, %1, 0x580\n\t" "s_load_dwordx16 %0, %1, 0x5c0\n\t"
            "s_load_dwordx16 %0, %1, 0x600\n\t" "s_load_dwordx16 %0, %1, 0x640\n\t"
            "s_load_dwordx16 %0, %1, 0x680\n\t" "s_load_dwordx16 %0, %1, 0x6c0\n\t"
            "s_load_dwordx16 %0, %1, 0x700\n\t" "s_load_dwordx16 %0, %1, 0x740\n\t"
            "s_load_dwordx16 %0, %1, 0x780\n\t" "s_load_dwordx16 %0, %1, 0x7c0\n\t");
    else if constexpr (NL == 64)
        QSA_QPF("s_load_dwordx16 %0, %1, 0x0\n\t" "s_load_dwordx16 %0, %1, 0x40\n\t"
            "s_load_dwordx16 %0, %1, 0x80\n\t" "s_load_dwordx16 %0, %1, 0xc0\n\t"
            "s_load_dwordx16 %0, %1, 0x100\n\t" "s_load_dwordx16 %0, %1, 0x140\n\t"
            "s_load_dwordx16 %0, %1, 0x180\n\t" "s_load_dwordx16 %0, %1, 0x1c0\n\t"
            "s_load_dwordx16 %0, %1, 0x200\n\t" "s_load_dwordx16 %0, %1, 0x240\n\t"
            "s_load_dwordx16 %0, %1, 0x280\n\t" "s_load_dwordx16 %0, %1, 0x2c0\n\t"
            "s_load_dwordx16 %0, %1, 0x300\n\t" "s_load_dwordx16 %0, %1, 0x340\n\t"
            "s_load_dwordx16 %0, %1, 0x380\n\t" "s_load_dwordx16 %0, %1, 0x3c0\n\t"
            "s_load_dwordx16 %0, %1, 0x400\n\t" "s_load_dwordx16 %0, %1, 0x440\n\t"
            "s_load_dwordx16 %0, %1, 0x480\n\t" "s_load_dwordx16 %0, %1, 0x4c0\n\t"
            "s_load_dwordx16 %0, %1, 0x500\n\t" "s_load_dwordx16 %0, %1, 0x540\n\t"
            "s_load_dwordx16 %0, %1, 0x580\n\t" "s_load_dwordx16 %0, %1, 0x5c0\n\t"
            "s_load_dwordx16 %0, %1, 0x600\n\t" "s_load_dwordx16 %0, %1, 0x640\n\t"
            "s_load_dwordx16 %0, %1, 0x680\n\t" "s_load_dwordx16 %0, %1, 0x6c0\n\t"
            "s_load_dwordx16 %0, %1, 0x700\n\t" "s_load_dwordx16 %0, %1, 0x740\n\t"
            "s_load_dwordx16 %0, %1, 0x780\n\t" "s_load_dwordx16 %0, %1, 0x7c0\n\t"
            "s_load_dwordx16 %0, %1, 0x800\n\t" "s_load_dwordx16 %0, %1, 0x840\n\t"
            "s_load_dwordx16 %0, %1, 0x880\n\t" "s_load_dwordx16 %0, %1, 0x8c0\n\t"
            "s_load_dwordx16 %0, %1, 0x900\n\t" "s_load_dwordx16 %0, %1, 0x940\n\t"
            "s_load_dwordx16 %0, %1, 0x980\n\t" "s_load_dwordx16 %0, %1, 0x9c0\n\t"
            "s_load_dwordx16 %0, %1, 0xa00\n\t" "s_load_dwordx16 %0, %1, 0xa40\n\t"
            "s_load_dwordx16 %0, %1, 0xa80\n\t" "s_load_dwordx16 %0, %1, 0xac0\n\t"
            "s_load_dwordx16 %0, %1, 0xb00\n\t" "s_load_dwordx16 %0, %1, 0xb40\n\t"
            "s_load_dwordx16 %0, %1, 0xb80\n\t" "s_load_dwordx16 %0, %1, 0xbc0\n\t"
            "s_load_dwordx16 %0, %1, 0xc00\n\t" "s_load_dwordx16 %0, %1, 0xc40\n\t"
            "s_load_dwordx16 %0, %1, 0xc80\n\t" "s_load_dwordx16 %0, %1, 0xcc0\n\t"
            "s_load_dwordx16 %0, %1, 0xd00\n\t" "s_load_dwordx16 %0, %1, 0xd40\n\t"
            "s_load_dwordx16 %0, %1, 0xd80\n\t" "s_load_dwordx16 %0, %1, 0xdc0\n\t"
            "s_load_dwordx16 %0, %1, 0xe00\n\t" "s_load_dwordx16 %0, %1, 0xe40\n\t"
            "s_load_dwordx16 %0, %1, 0xe80\n\t" "s_load_dwordx16 %0, %1, 0xec0\n\t"
            "s_load_dwordx16 %0, %1, 0xf00\n\t" "s_load_dwordx16 %0, %1, 0xf40\n\t"
            "s_load_dwordx16 %0, %1, 0xf80\n\t" "s_load_dwordx16 %0, %1, 0xfc0\n\t");
    else
        static_assert(NL == 32, "scalar query rows of 32 or 64 lines");
}
#undef QSA_QPF

// Vector query path.  Under a decode batch's key traffic a scalar-cache miss
// takes microseconds, and every (chunk, head) step of the scalar path waits
// for one; here the query row instead arrives with the wave's first vector
// loads (issued before the key row, so the wait for the first key chunk
// covers it) and reaches the fused multiply-adds through DPP row broadcasts.
//
// Step t = c * H + h uses the 16 query dwords of head h, dims 32c .. 32c+31
// (the step's block).  16-byte load g gives lane l dwords 4(l%4) .. +3 of
// block 4g + (l/4)%4, the same in each 16-lane row, so dword k of block t is
// in register k%4 of load t/4, at row lane 4(t%4) + k/4.  The registers of a
// load are widened to fp32 once (8 operations for 4 steps).
template <int H, int D>
struct QueryVec {
    static constexpr int NCH = D / kExactChunk;
    static constexpr int STEPS = NCH * H;
    static constexpr int NQ = (STEPS + 3) / 4;   // 16-byte loads per lane
    static constexpr bool kUse = STEPS <= 32;
};

// 8 fused multiply-adds acc += q * k, dims 8m .. 8m+7 of one step in
// ascending order: q from the widened registers (lo: even dims, hi: odd
// dims of dwords 4m .. 4m+3) broadcast from row lane LANE, k in registers.
// The leading s_nop gives the two wait states a DPP read needs after the
// VALU write of its source.
template <int LANE>
__device__ __forceinline__ void fma8_bcast(float &acc, const float (&lo)[4], const float (&hi)[4],
                                           const float *k) {
    static_assert(LANE >= 0 && LANE < 16, "row lane");
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %1, %9 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %5, %10 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %11 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %6, %12 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %3, %13 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %7, %14 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %15 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %8, %16 row_newbcast:%17 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(lo[0]), "v"(lo[1]), "v"(lo[2]), "v"(lo[3]), "v"(hi[0]), "v"(hi[1]), "v"(hi[2]), "v"(hi[3]),
          "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(k[4]), "v"(k[5]), "v"(k[6]), "v"(k[7]), "n"(LANE));
}

template <typename KT, int CH>
__device__ __forceinline__ void widen_chunk(const u32x4 (&u)[CH * KeyBits<KT>::value / 128], float (&f)[CH],
                                            float scl) {
    if constexpr (std::is_same<KT, Fp4x2>::value) {
        // byte j of the chunk holds dims 2j (low nibble) and 2j+1; the
        // conversion multiplies by the group's power of two exactly
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const u32x4 w4 = u[0];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f32x2 r0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w4[e], scl, 0);
            const f32x2 r1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w4[e], scl, 1);
            const f32x2 r2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w4[e], scl, 2);
            const f32x2 r3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w4[e], scl, 3);
            f[8 * e + 0] = r0.x; f[8 * e + 1] = r0.y; f[8 * e + 2] = r1.x; f[8 * e + 3] = r1.y;
            f[8 * e + 4] = r2.x; f[8 * e + 5] = r2.y; f[8 * e + 6] = r3.x; f[8 * e + 7] = r3.y;
        }
    } else if constexpr (std::is_same<KT, uint8_t>::value) {
#pragma unroll
        for (int v = 0; v < CH / 16; ++v) {
            const u32x4 w4 = u[v];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float2 a = e4m3x2_to_f32<false>(w4[e]);
                const float2 b = e4m3x2_to_f32<true>(w4[e]);
                f[16 * v + 4 * e] = a.x; f[16 * v + 4 * e + 1] = a.y;
                f[16 * v + 4 * e + 2] = b.x; f[16 * v + 4 * e + 3] = b.y;
            }
        }
    } else {
#pragma unroll
        for (int v = 0; v < CH / 8; ++v) {
            const u32x4 w4 = u[v];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[8 * v + 2 * e] = bf16lo(w4[e]);
                f[8 * v + 2 * e + 1] = bf16hi(w4[e]);
            }
        }
    }
}

// Decode batches (one query per sequence, at most kFlatMaxRows rows) number
// only the visible 256-block groups: workgroup g scores the g-th visible
// group in (row, group) order, and the workgroups past the last one exit.
// The grid is sized for every row at the longest length.  Numbered densely
// by (row, group), its empty workgroups sat among the visible ones, and the
// CUs that the launch's single round of workgroups gave to the longest rows
// scored four groups while others scored one.  Each wave finds its group by
// itself: 64 rows at a time (lane l: row r0 + l), one round of vector loads
// of the offsets, a lane scan of the rows' group counts and a ballot.
constexpr int kFlatMaxRows = 4 * kWave;
__device__ __forceinline__ int64_t readlane_i64(int64_t x, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(uint64_t)x, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), lane);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ bool flat_group(const int64_t *__restrict__ kv_off, const int64_t *__restrict__ blk_off,
                                           int num_seqs, int log2r, uint32_t g, int64_t &i, int64_t &by,
                                           QueryPos &qp) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t base = 0u;                              // groups of the rows before r0
    for (int r0 = 0; r0 < num_seqs; r0 += kWave) {
        const int row = r0 + lane;
        const bool in = row < num_seqs;
        const int64_t o0 = in ? kv_off[row] : 0;
        const int64_t o1 = in ? kv_off[row + 1] : 0;
        const int64_t b0 = in && blk_off ? blk_off[row] : 0;
        const uint32_t c = (uint32_t)((((o1 - o0) >> log2r) + kExactThreads - 1) / kExactThreads);
        const uint32_t incl = base + wave_incl_scan(c);
        const uint64_t m = __ballot(incl > g);
        if (m != 0u) {                               // uniform
            const int src = (int)__builtin_ctzll(m);
            i = r0 + src;
            by = g - (uint32_t)__builtin_amdgcn_readlane((int)(incl - c), src);
            qp.seq = (int)i;
            qp.kv_row0 = readlane_i64(o0, src);
            qp.L = readlane_i64(o1 - o0, src);
            qp.blk_row0 = readlane_i64(b0, src);
            return true;
        }
        base = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    }
    return false;                                    // past the last visible group
}

// SKIP_NEW: leave out the block the query's last token completes (L a
// multiple of the ratio), which the fused append scores itself.
template <typename KT, int D, int H, bool SKIP_NEW>
__device__ __forceinline__ void score_exact_body(
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w, const KT *__restrict__ kc,
    const void *__restrict__ kc_scale, int log2r, float *__restrict__ scores, int64_t ld, const PageMap &pm,
    const QueryPos &qp, int64_t i, int64_t by, const ListArgs &la) {
    constexpr bool kE4M3 = std::is_same<KT, uint8_t>::value;
    constexpr bool kFP4 = std::is_same<KT, Fp4x2>::value;
    constexpr int CH = kExactChunk;
    constexpr int NCH = D / CH;
    constexpr int LPC = CH * KeyBits<KT>::value / 128;   // 16-byte loads per chunk of one row
    constexpr int QW = CH / 2;                           // query dwords per (chunk, head)
    static_assert(D % CH == 0 && (LPC == 1 || LPC == 2 || LPC == 4) && QW == 16, "chunk layout");
    static_assert((NCH - 1) * LPC < 64, "loads in flight fit the wait counter");
    const int64_t nb = qp.L >> log2r;
    const int64_t b = by * kExactThreads + threadIdx.x;
    if (by * kExactThreads >= nb) return;   // whole workgroup invisible
    bool active = b < nb;
    if constexpr (SKIP_NEW) active = active && !(b == nb - 1 && (qp.L & ((1 << log2r) - 1)) == 0);
    const int64_t row = pm.table ? paged_row(pm, qp.seq, active ? b : 0, pm.log2_page - log2r)
                                 : qp.blk_row0 + (active ? b : 0);
    const float sc = kE4M3 ? static_cast<const float *>(kc_scale)[row] : 1.0f;
    const uint8_t *krow = reinterpret_cast<const uint8_t *>(kc) + row * (D * KeyBits<KT>::value / 8);
    const uint32_t *q32 = reinterpret_cast<const uint32_t *>(q_idx) + i * (int64_t)(H * D / 2);

    using QV = QueryVec<H, D>;
    u32x4 qv[QV::kUse ? QV::NQ : 1];
    if constexpr (QV::kUse) {
        const int lane = threadIdx.x & (kWave - 1);
        static_for<0, QV::NQ>([&](auto gg) {
            constexpr int g = decltype(gg)::value;
            int t = 4 * g + ((lane >> 2) & 3);
            if (t >= QV::STEPS) t = 0;                       // past the last step: any valid block
            const int c = t / H, h = t % H;
            qv[g] = key_load16<0>(q32 + h * (D / 2) + 16 * c + 4 * (lane & 3));
        });
    }
    uint32_t sbits = 0;
    if constexpr (kFP4) sbits = fp4_scale_load<D>(static_cast<const uint8_t *>(kc_scale) + row * (D / 32));
    u32x4 raw[NCH][LPC];
    static_for<0, NCH>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        raw[c][0] = key_load16<c * LPC * 16 + 0>(krow);
        if constexpr (LPC >= 2) raw[c][1] = key_load16<c * LPC * 16 + 16>(krow);
        if constexpr (LPC == 4) {
            raw[c][2] = key_load16<c * LPC * 16 + 32>(krow);
            raw[c][3] = key_load16<c * LPC * 16 + 48>(krow);
        }
    });
    u32x16 qbuf[2];
    if constexpr (!QV::kUse) {
        query_prefetch<H * D / 32>(q32);
        qbuf[0] = query_load16<0>(q32);
    }

    float acc[H];
#pragma unroll
    for (int h = 0; h < H; ++h) acc[h] = 0.0f;
    float qlo[4], qhi[4];
    // (chunk, head) steps in order; chunk c is waited for at its first step
    // (the loads of chunks c+1.. may still be in flight).
    static_for<0, NCH>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        key_wait<(NCH - 1 - c) * LPC>(raw[c]);
        if constexpr (kFP4 && c == 0) asm volatile("" : "+v"(sbits));   // landed before chunk 0
        if constexpr (QV::kUse && c == 0) {                              // issued before chunk 0
#pragma unroll
            for (int g = 0; g < QV::NQ; ++g) asm volatile("" : "+v"(qv[g]));
        }
        float kf[CH];
        widen_chunk<KT, CH>(raw[c], kf, kFP4 ? e8m0_to_f32((sbits >> (8 * c)) & 0xffu) : 1.0f);
        static_for<0, H>([&](auto hh) {
            constexpr int h = decltype(hh)::value;
            constexpr int t = c * H + h;
            if constexpr (QV::kUse) {
                if constexpr (t % 4 == 0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        qlo[r] = bf16lo(qv[t / 4][r]);
                        qhi[r] = bf16hi(qv[t / 4][r]);
                    }
                }
                fma8_bcast<4 * (t % 4) + 0>(acc[h], qlo, qhi, kf + 0);
                fma8_bcast<4 * (t % 4) + 1>(acc[h], qlo, qhi, kf + 8);
                fma8_bcast<4 * (t % 4) + 2>(acc[h], qlo, qhi, kf + 16);
                fma8_bcast<4 * (t % 4) + 3>(acc[h], qlo, qhi, kf + 24);
                return;
            }
            u32x16 &qu = qbuf[t & 1];
            constexpr int tn = t + 1;                // next step: its query offset in bytes
            constexpr int off = 4 * ((tn % H) * (D / 2) + (tn / H) * QW);
            if constexpr (tn < NCH * H) {
                if constexpr (t == 0)
                    qbuf[tn & 1] = query_wait_load16<off>(qu, q32);
                else
                    qbuf[tn & 1] = query_wait_load16<off>(qu, acc[(t - 1) % H], q32);
            } else {
                query_wait(qu, acc[(t - 1 + H) % H]);
            }
#pragma unroll
            for (int j = 0; j < QW; ++j) {
                acc[h] = __builtin_fmaf(bf16lo(qu[j]), kf[2 * j], acc[h]);
                acc[h] = __builtin_fmaf(bf16hi(qu[j]), kf[2 * j + 1], acc[h]);
            }
        });
    });
    const float *__restrict__ wi = w + i * (int64_t)H;
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < H; ++h) {
        float dot = acc[h];
        if constexpr (kE4M3) dot = dot * sc;
        const float r = dot > 0.0f ? dot : 0.0f;
        const float t = wi[h] * r;
        s = s + t;
    }
    if (active) scores[i * ld + b] = s;
    if (la.keys) {
        const int64_t chunk0 = b - (threadIdx.x & (kWave - 1));
        // the chunk of the block the append scores leaves its last slot
        const bool reserve = SKIP_NEW && (qp.L & ((1 << log2r) - 1)) == 0 && nb > 0 &&
                             chunk0 == ((nb - 1) & ~int64_t(kListChunk - 1));
        emit_chunk_list(la, i, nb, chunk0, active, s, threadIdx.x & (kWave - 1), reserve);
    }
}

template <typename KT, int D, int H>
__global__ __launch_bounds__(kExactThreads) void score_exact_kernel(
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w, const KT *__restrict__ kc,
    const void *__restrict__ kc_scale, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ blk_off, const int64_t *__restrict__ q_off, int num_seqs,
    int log2r, float *__restrict__ scores, int64_t ld, PageMap pm, ListArgs la, int flat) {
    if (la.mode && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *la.mode = 0u;   // plain lists
    int64_t i, by;
    QueryPos qp;
    if (flat) {
        if (!flat_group(kv_off, blk_off, num_seqs, log2r, blockIdx.x, i, by, qp)) return;
    } else {
        i = blockIdx.x;
        by = blockIdx.y;
        qp = query_pos(kv_off, blk_off, q_off, num_seqs, i);
    }
    score_exact_body<KT, D, H, false>(q_idx, w, kc, kc_scale, log2r, scores, ld, pm, qp, i, by, la);
}

// Canonical score of one block whose key a wave holds (lane l: dims
// l*DPL.., values as the scorer widens them; sc: the e4m3 row scale), with
// score_exact_body's arithmetic: per head an fp32 fused multiply-add chain
// over ascending d from +0, then the scale, ReLU and the weighted sum over
// ascending heads.  Lane h computes head h's chain; lane 0 writes.
template <int D, int H, bool E4M3>
__device__ __forceinline__ void score_one_block(const float (&dec)[D / kWave], float sc,
                                                const uint16_t *__restrict__ q_idx, const float *__restrict__ w,
                                                int64_t i, float *__restrict__ dst, int lane) {
    constexpr int DPL = D / kWave;
    const int h = lane < H ? lane : H - 1;
    const uint4 *q4 = reinterpret_cast<const uint4 *>(q_idx + (i * H + h) * D);
    uint32_t qd[D / 2];
#pragma unroll
    for (int j = 0; j < D / 8; ++j) {
        const uint4 v = q4[j];
        qd[4 * j] = v.x; qd[4 * j + 1] = v.y; qd[4 * j + 2] = v.z; qd[4 * j + 3] = v.w;
    }
    float dot = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const float k = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dec[d % DPL]), d / DPL));
        const float q = (d & 1) ? bf16hi(qd[d / 2]) : bf16lo(qd[d / 2]);
        dot = __builtin_fmaf(q, k, dot);
    }
    float s = 0.0f;
#pragma unroll
    for (int hh = 0; hh < H; ++hh) {
        float dd = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dot), hh));
        if constexpr (E4M3) dd = dd * sc;
        const float r = dd > 0.0f ? dd : 0.0f;
        const float t = w[i * H + hh] * r;
        s = s + t;
    }
    if (lane == 0) *dst = s;
}

// Append + canonical score in one launch, for a decode step (one new token
// and one query per sequence).  Scoring workgroups score a (query, 256-block
// group) as score_exact_kernel does, except the block the new token
// completes; append workgroups run one append wave per sequence
// (append_one), which writes that block's compressed key (or, when the
// append could not, takes the key already stored) and scores the block with
// the same arithmetic.  Nothing else the scorer reads is written here, so the
// result equals the append followed by the score, bit for bit.  Grid: with
// `flat`, one row, the append workgroups first and then the visible groups
// as flat_group numbers them; otherwise x < num_seqs scores query x (y: the
// group) and the x after them (y = 0) append.
template <typename KT, int D, int H, typename TIn>
__global__ __launch_bounds__(kExactThreads) void ingest_score_kernel(
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w, KT *__restrict__ kc,
    void *__restrict__ kc_scale, const int64_t *__restrict__ kv_off, const int64_t *__restrict__ blk_off,
    int num_seqs, int log2r, float *__restrict__ scores, int64_t ld, PageMap pm, const TIn *__restrict__ k_new,
    float inv_ratio, RingArgs ring, KvArgs kv, int32_t *__restrict__ status, ListArgs la, int flat) {
    constexpr int kWaves = kExactThreads / kWave;
    // the lists' form, for the selection that reads them
    if (la.mode && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *la.mode = kListNewBlockSlot;
    int ab;   // append workgroup
    if (flat) {
        // the append workgroups first, then the visible groups (flat_group)
        const int na = (num_seqs + kWaves - 1) / kWaves;
        if ((int)blockIdx.x >= na) {
            int64_t i, by;
            QueryPos qp;
            if (!flat_group(kv_off, blk_off, num_seqs, log2r, blockIdx.x - (uint32_t)na, i, by, qp)) return;
            score_exact_body<KT, D, H, true>(q_idx, w, kc, kc_scale, log2r, scores, ld, pm, qp, i, by, la);
            return;
        }
        ab = (int)blockIdx.x;
    } else {
        if ((int)blockIdx.x < num_seqs) {
            const QueryPos qp = query_pos(kv_off, blk_off, nullptr, num_seqs, blockIdx.x);
            score_exact_body<KT, D, H, true>(q_idx, w, kc, kc_scale, log2r, scores, ld, pm, qp, blockIdx.x,
                                             blockIdx.y, la);
            return;
        }
        if (blockIdx.y != 0) return;
        ab = (int)blockIdx.x - num_seqs;
    }
    constexpr int DPL = D / kWave;
    constexpr int KC = std::is_same<KT, Fp4x2>::value ? 3 : (std::is_same<KT, uint8_t>::value ? 2 : 1);
    const int lane = threadIdx.x & (kWave - 1);
    const int sq = ab * kWaves + (int)(threadIdx.x / kWave);
    if (sq >= num_seqs) return;
    AppendOut<DPL> a = append_one<TIn, DPL, KC>(k_new, kv_off, blk_off, sq, log2r, inv_ratio, ring, kc, kc_scale,
                                                kv, status, pm, lane);
    if (!a.complete) return;
    if (!a.stored) load_kc_values<KC, DPL>(kc, kc_scale, a.kc_row, lane, a.dec, a.sc);
    const int64_t g = ((kv_off[sq + 1] - kv_off[sq]) >> log2r) - 1;
    score_one_block<D, H, KC == 2>(a.dec, a.sc, q_idx, w, sq, scores + sq * ld + g, lane);
}

template <typename QT, typename KT, int D>
hipError_t dispatch_h(const qsa_indexer &ix, int log2r, const qsa_batch &b, float *scores,
                      int64_t ld, const PageMap &pm, dim3 grid, hipStream_t st, const ListArgs &la) {
    const QT *q = static_cast<const QT *>(ix.q_idx);
    const KT *kc = static_cast<const KT *>(ix.kc);
    constexpr bool kExact = std::is_same<QT, uint16_t>::value && !std::is_same<KT, float>::value;
    const int64_t max_nb = b.max_kv_len >> log2r;
    if constexpr (kExact) {
        grid.y = (unsigned)((max_nb + kExactThreads - 1) / kExactThreads);
        // decode batches: only the visible groups, numbered over one grid row
        const int flat = b.q_offsets == nullptr && b.total_q == b.num_seqs && b.num_seqs <= kFlatMaxRows;
        if (flat) {
            grid.x *= grid.y;
            grid.y = 1;
        }
        dim3 block(kExactThreads);
#define QSA_SCORE_LAUNCH(HH)                                                                       \
    hipLaunchKernelGGL((score_exact_kernel<KT, D, HH>), grid, block, 0, st, q, ix.w, kc,           \
                       ix.kc_scale, b.kv_offsets, b.blk_offsets, b.q_offsets, b.num_seqs, log2r,  \
                       scores, ld, pm, la, flat)
        switch (ix.h_idx) {
        case 1: QSA_SCORE_LAUNCH(1); break;
        case 2: QSA_SCORE_LAUNCH(2); break;
        case 4: QSA_SCORE_LAUNCH(4); break;
        case 8: QSA_SCORE_LAUNCH(8); break;
        default: QSA_SCORE_LAUNCH(16); break;
        }
#undef QSA_SCORE_LAUNCH
    } else {
        grid.y = (unsigned)((max_nb + kScoreThreads - 1) / kScoreThreads);
        dim3 block(kScoreThreads);
#define QSA_SCORE_LAUNCH(HH)                                                                       \
    hipLaunchKernelGGL((score_rounded_kernel<QT, KT, D, HH>), grid, block, 0, st, q, ix.w, kc,     \
                       static_cast<const float *>(ix.kc_scale), b.kv_offsets, b.blk_offsets,      \
                       b.q_offsets, b.num_seqs, log2r, scores, ld, pm, la)
        switch (ix.h_idx) {
        case 1: QSA_SCORE_LAUNCH(1); break;
        case 2: QSA_SCORE_LAUNCH(2); break;
        case 4: QSA_SCORE_LAUNCH(4); break;
        case 8: QSA_SCORE_LAUNCH(8); break;
        default: QSA_SCORE_LAUNCH(16); break;
        }
#undef QSA_SCORE_LAUNCH
    }
    return hipGetLastError();
}

template <typename QT, typename KT>
hipError_t dispatch_d(const qsa_indexer &ix, int log2r, const qsa_batch &b, float *scores,
                      int64_t ld, const PageMap &pm, dim3 grid, hipStream_t st, const ListArgs &la) {
    return ix.d_idx == 64 ? dispatch_h<QT, KT, 64>(ix, log2r, b, scores, ld, pm, grid, st, la)
                          : dispatch_h<QT, KT, 128>(ix, log2r, b, scores, ld, pm, grid, st, la);
}

struct FusedArgs {
    const uint16_t *q_idx;
    const float *w;
    void *kc, *kc_scale;
    const int64_t *kv_off, *blk_off;
    int num_seqs, log2r;
    float *scores;
    int64_t ld;
    PageMap pm;
    const void *k_new;
    float inv_ratio;
    RingArgs ring;
    KvArgs kv;
    int32_t *status;
    ListArgs la;
    int flat;   // the scoring workgroups number only the visible groups
};

template <typename KT, int D, int H, typename TIn>
hipError_t fused_launch(const FusedArgs &f, dim3 grid, hipStream_t st) {
    hipLaunchKernelGGL((ingest_score_kernel<KT, D, H, TIn>), grid, dim3(kExactThreads), 0, st, f.q_idx, f.w,
                       static_cast<KT *>(f.kc), f.kc_scale, f.kv_off, f.blk_off, f.num_seqs, f.log2r, f.scores,
                       f.ld, f.pm, static_cast<const TIn *>(f.k_new), f.inv_ratio, f.ring, f.kv, f.status, f.la,
                       f.flat);
    return hipGetLastError();
}

template <typename KT, int D, typename TIn>
hipError_t fused_h(const FusedArgs &f, int h, dim3 grid, hipStream_t st) {
    switch (h) {
    case 1: return fused_launch<KT, D, 1, TIn>(f, grid, st);
    case 2: return fused_launch<KT, D, 2, TIn>(f, grid, st);
    case 4: return fused_launch<KT, D, 4, TIn>(f, grid, st);
    case 8: return fused_launch<KT, D, 8, TIn>(f, grid, st);
    default: return fused_launch<KT, D, 16, TIn>(f, grid, st);
    }
}

template <typename KT>
hipError_t fused_d(const FusedArgs &f, int d, int h, bool k_bf16, dim3 grid, hipStream_t st) {
    if (d == 64)
        return k_bf16 ? fused_h<KT, 64, uint16_t>(f, h, grid, st) : fused_h<KT, 64, float>(f, h, grid, st);
    return k_bf16 ? fused_h<KT, 128, uint16_t>(f, h, grid, st) : fused_h<KT, 128, float>(f, h, grid, st);
}

}  // namespace

// Block pooling of token scores (max, or the fp32 mean in token order).
template <int MODE>
__global__ __launch_bounds__(kScoreThreads) void pool_scores_kernel(
    const float *__restrict__ tok, int64_t ld_tok, const int64_t *__restrict__ kv_off,
    const int64_t *__restrict__ q_off, int num_seqs, int log2r, float inv_ratio, float *__restrict__ blk,
    int64_t ld_blk) {
    const int64_t i = blockIdx.y;
    const QueryPos qp = query_pos(kv_off, nullptr, q_off, num_seqs, i);
    const int64_t nb = qp.L >> log2r;
    const int64_t b = (int64_t)blockIdx.x * kScoreThreads + threadIdx.x;
    if (b >= nb) return;
    const float *t = tok + i * ld_tok + (b << log2r);
    float acc = MODE == QSA_POOL_MAX ? t[0] : 0.0f + t[0];
    for (int j = 1; j < (1 << log2r); ++j) acc = MODE == QSA_POOL_MAX ? fmaxf(acc, t[j]) : acc + t[j];
    blk[i * ld_blk + b] = MODE == QSA_POOL_MAX ? acc : acc * inv_ratio;
}

hipError_t launch_pool_scores(const float *tok, int64_t ld_tok, int ratio, int mode, const qsa_batch &b,
                              float *blk, int64_t ld_blk, hipStream_t st) {
    const int log2r = __builtin_ctz((unsigned)ratio);
    const int64_t max_nb = b.max_kv_len >> log2r;
    if (b.total_q == 0 || max_nb == 0) return hipSuccess;
    dim3 grid((unsigned)((max_nb + kScoreThreads - 1) / kScoreThreads), (unsigned)b.total_q);
    const float inv = 1.0f / (float)ratio;
    trace("pool_scores grid=(%u,%u) ratio=%d mode=%d", grid.x, grid.y, ratio, mode);
    if (mode == QSA_POOL_MAX)
        hipLaunchKernelGGL(pool_scores_kernel<QSA_POOL_MAX>, grid, dim3(kScoreThreads), 0, st, tok, ld_tok,
                           b.kv_offsets, b.q_offsets, b.num_seqs, log2r, inv, blk, ld_blk);
    else
        hipLaunchKernelGGL(pool_scores_kernel<QSA_POOL_MEAN>, grid, dim3(kScoreThreads), 0, st, tok, ld_tok,
                           b.kv_offsets, b.q_offsets, b.num_seqs, log2r, inv, blk, ld_blk);
    return hipGetLastError();
}

hipError_t launch_score_canonical(const qsa_indexer &ix, int ratio, const qsa_batch &b,
                                  float *scores, int64_t ld, const qsa_paged_kv *pg, hipStream_t st,
                                  const ListArgs &la) {
    const PageMap pm = page_map(pg);
    const int log2r = __builtin_ctz((unsigned)ratio);
    const int64_t max_nb = b.max_kv_len >> log2r;
    if (b.total_q == 0 || max_nb == 0) return hipSuccess;
    dim3 grid((unsigned)b.total_q, 1);   // grid.y is set per kernel form
    trace("score_canonical grid=(%u,%u) h_idx=%d d_idx=%d q=%d kc=%d", grid.x, grid.y, ix.h_idx,
          ix.d_idx, ix.q_dtype, ix.kc_dtype);
    const bool qb = ix.q_dtype == QSA_BF16;
    switch (ix.kc_dtype) {
    case QSA_F32:
        return qb ? dispatch_d<uint16_t, float>(ix, log2r, b, scores, ld, pm, grid, st, la)
                  : dispatch_d<float, float>(ix, log2r, b, scores, ld, pm, grid, st, la);
    case QSA_BF16:
        return qb ? dispatch_d<uint16_t, uint16_t>(ix, log2r, b, scores, ld, pm, grid, st, la)
                  : dispatch_d<float, uint16_t>(ix, log2r, b, scores, ld, pm, grid, st, la);
    case QSA_FP8_E4M3:
        return qb ? dispatch_d<uint16_t, uint8_t>(ix, log2r, b, scores, ld, pm, grid, st, la)
                  : dispatch_d<float, uint8_t>(ix, log2r, b, scores, ld, pm, grid, st, la);
    default:   // fp4 keys take a bf16 query (checked by the caller)
        return dispatch_d<uint16_t, Fp4x2>(ix, log2r, b, scores, ld, pm, grid, st, la);
    }
}

hipError_t launch_ingest_score(const void *k_new, int k_dtype, int ratio, const qsa_batch &b,
                               const qsa_key_ring &ring, const qsa_kv_append *kv, int32_t *status,
                               const qsa_indexer &ix, float *scores, int64_t ld, const qsa_paged_kv *pg,
                               hipStream_t st, const ListArgs &la) {
    if (b.num_seqs == 0) return hipSuccess;
    FusedArgs f;
    f.la = la;
    f.q_idx = static_cast<const uint16_t *>(ix.q_idx);
    f.w = ix.w;
    f.kc = const_cast<void *>(ix.kc);
    f.kc_scale = const_cast<void *>(ix.kc_scale);
    f.kv_off = b.kv_offsets;
    f.blk_off = b.blk_offsets;
    f.num_seqs = b.num_seqs;
    f.log2r = __builtin_ctz((unsigned)ratio);
    f.scores = scores;
    f.ld = ld;
    f.pm = page_map(pg);
    f.k_new = k_new;
    f.inv_ratio = 1.0f / (float)(1 << f.log2r);
    f.ring = RingArgs{ring.keys, ring.window, ring.slots, ring.num_slots, (int64_t)ring.capacity};
    f.kv = KvArgs{nullptr, nullptr, nullptr, nullptr, 0};
    if (kv) {
        f.kv.k_new = static_cast<const uint8_t *>(kv->k_new);
        f.kv.v_new = static_cast<const uint8_t *>(kv->v_new);
        f.kv.k = static_cast<uint8_t *>(kv->k);
        f.kv.v = static_cast<uint8_t *>(kv->v);
        f.kv.row_bytes = kv->hkv * kv->d * (kv->dtype == QSA_BF16 ? 2 : 4);
    }
    f.status = status;
    // x: one scoring workgroup per query, then one append wave per sequence;
    // y: the scorer's 256-block groups (at least one, for the appends).  Up
    // to kFlatMaxRows sequences: x alone, the append workgroups and then
    // one scoring workgroup per (sequence, group) slot
    const int64_t max_nb = b.max_kv_len >> f.log2r;
    const int waves = kExactThreads / kWave;
    const unsigned ny = (unsigned)(max_nb > 0 ? (max_nb + kExactThreads - 1) / kExactThreads : 1);
    const unsigned na = (unsigned)((b.num_seqs + waves - 1) / waves);
    f.flat = b.num_seqs <= kFlatMaxRows;
    dim3 grid(f.flat ? na + (unsigned)b.num_seqs * ny : (unsigned)b.num_seqs + na, f.flat ? 1u : ny);
    trace("ingest_score grid=(%u,%u) h_idx=%d d_idx=%d kc=%d kv=%d", grid.x, grid.y, ix.h_idx, ix.d_idx,
          ix.kc_dtype, f.kv.row_bytes);
    const bool kb = k_dtype == QSA_BF16;
    switch (ix.kc_dtype) {
    case QSA_BF16: return fused_d<uint16_t>(f, ix.d_idx, ix.h_idx, kb, grid, st);
    case QSA_FP8_E4M3: return fused_d<uint8_t>(f, ix.d_idx, ix.h_idx, kb, grid, st);
    default: return fused_d<Fp4x2>(f, ix.d_idx, ix.h_idx, kb, grid, st);   // fp4 (checked by the caller)
    }
}

}  // namespace qsa
