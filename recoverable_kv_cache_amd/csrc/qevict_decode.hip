// Decode step, two launches per layer (one when each (sequence, KV head) has a single
// split).  k_decode_split appends the new token to its recent window and runs split-K
// attention over the accessible list (sinks, recent windows, Full bf16 windows, Quantized
// INT2 or INT4 windows); k_finish combines the splits of each query head with the global
// log-sum-exp, writes each entry's per-head share of this step's window mass, and advances
// the token count (with a single split the split kernel does all of that itself).  The shares are folded into the cumulative scores by the next
// k_decode_split of the unit (or by the router / an export, whichever comes
// first), which overlaps that read-modify-write with other work.
//
// Source: "QEvict: Recoverable Quantized KV Eviction for Attention-Drift-Robust
// Long-Context Decoding", §4.1 (accessible-set attention, scale 1/sqrt(d_kv);
// Quantized windows are dequantized in the execution datatype as
// off + scl * code, Eq. 5), §4.2 Eq. 1 (cumulative window score, averaged over
// the H_q query heads); Appendix G.3 (the 4-bit recoverable tier).
//
// Work split: one workgroup per (split, KV head, sequence); the G query heads of
// the GQA group share every K/V load.  All contractions run on 16x16 MFMA tiles
// with 16 columns: each query head owns two columns, a "high" and a "low" one,
// so that bf16 operands can carry fp32-accurate values as a sum of two bf16
// parts (query times K scale on the key side, probability times V scale on the
// value side).  With G <= 4 the 16 columns hold two independent column slots,
// so one wave job covers two Quantized windows at once and the softmax arithmetic
// of both runs in the same instructions.  The code width (2 or 4 bits) is a
// template parameter: it changes only how many code bytes a lane loads and how a
// byte expands into bf16 integers (4 codes of 2 bits or 2 of 4 bits per lookup).
#include <float.h>
#include <hip/hip_ext.h>

#include "qevict_common.h"
#include "qevict_internal.h"
#include "qevict_mass.h"

namespace qv {

constexpr int DW = 4;          // waves per workgroup
constexpr float M_INIT = -1e30f;   // running max before any token (finite: exp2(-inf - M_INIT) = 0)

typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// D[16x16] += A[16x32] B[32x16]: lane l holds A row l%16 / B column l%16 at k = 8(l/16)+i, D column l%16 rows 4(l/16)+i
__device__ __forceinline__ f4_t mfma32(u4_t a, u4_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), c, 0,
                                                   0, 0);
}
// D[16x16] += A[16x16] B[16x16]: k = 4(l/16)+i
__device__ __forceinline__ f4_t mfma16(u2_t a, u2_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, a), __builtin_bit_cast(s4_t, b), c, 0, 0,
                                                     0);
}
// both fp16 halves of a 32-bit word as fp32
__device__ __forceinline__ f2_t h2f(uint32_t w) { return __builtin_convertvector(__builtin_bit_cast(h2_t, w), f2_t); }
// x times the fp16 in the low / high half of w, one mixed-precision FMA with a zero
// addend (the same rounding as converting first and multiplying)
// (plain code, which the compiler selects as one v_fma_mix_f32 and sees in its hazard
// checks; an inline-asm version gave wrong outputs once v_dot2c_f32_bf16 was used beside it)
__device__ __forceinline__ float mul_h_lo(float x, uint32_t w) {
    return fmaf(x, (float)__builtin_bit_cast(h2_t, w).x, 0.0f);
}
__device__ __forceinline__ float mul_h_hi(float x, uint32_t w) {
    return fmaf(x, (float)__builtin_bit_cast(h2_t, w).y, 0.0f);
}
// maxima of operands that are never NaN (scores, -inf included), through compiler builtins
// (no inline assembly: the backend tracks the hazards with the lane permutes around them).
// max2 is the median of (a, b, +inf): one v_med3_f32, where fmaxf would first quiet
// operands that come from lane moves.
__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3(float a, float b, float c) { return max2(max2(a, b), c); }
// two fp32 -> packed bf16 pair, round to nearest even
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    const f2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2_t));
}
// top 16 bits of two fp32 (bf16 truncation)
__device__ __forceinline__ uint32_t bf16x2_trunc(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
// x0 - h.lo and x1 - h.hi for a packed bf16 pair h, as one bf16 pair (RNE).  Each difference
// is exact in fp32 whenever h holds x0, x1 rounded to bf16, and comes from a bf16 dot
// product of h with (-1, -0) or (0, -1) accumulated onto x.  (hipcc would encode the pair
// (-1, +0) as the inline constant -1.0, which the instruction reads as the fp32 word, i.e.
// as (0, -1); -0 keeps it a literal.)
__device__ __forceinline__ uint32_t bf16x2_rest(uint32_t h, float x0, float x1) {
    const bf2_t hb = __builtin_bit_cast(bf2_t, h);
    return bf16x2_rne(__builtin_amdgcn_fdot2_f32_bf16(hb, __builtin_bit_cast(bf2_t, 0x8000BF80u), x0, false),
                      __builtin_amdgcn_fdot2_f32_bf16(hb, __builtin_bit_cast(bf2_t, 0xBF800000u), x1, false));
}
// DPP lane moves.  Every pattern used here reads a lane of the same row of 16, so no
// lane is out of bounds and bound_ctrl changes no value; with it set the compiler can
// fold the move into the instruction that consumes it.
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// value of the lane at the mirrored position of this lane's SW-wide column group
// (row_half_mirror for SW = 8, row_mirror for SW = 16): pairs the high column of a
// head with its low column
template <int SW>
__device__ __forceinline__ float mirror(float x) {
    return dppf<SW == 8 ? 0x141 : 0x140>(x);
}
// value of lane (l ^ 8) within its row of 16 (row_ror:8): the other column slot
__device__ __forceinline__ float ror8(float x) { return dppf<0x128>(x); }
// Reductions over the 4 lane groups of a column (lanes l, l^16, l^32, l^48) with the
// gfx950 row-swap permutes: permlane16_swap(x, x) hands every lane the values of rows
// 2k and 2k+1 at its position, permlane32_swap(x, x) those of both 32-lane halves.  Both
// lanes of a pair add in the same order, so the result is identical across the group.
__device__ __forceinline__ float qg_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}
__device__ __forceinline__ float qg_max(float x) {   // (operands never NaN)
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max2(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
// sum over aligned groups of N consecutive lanes (N = 8, 16, 32 or 64) with DPP quad
// swaps, the half-row / row mirrors and the row swaps: no LDS traffic
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    x += dppf<0xB1>(x);                           // quad [1,0,3,2]
    x += dppf<0x4E>(x);                           // quad [2,3,0,1]
    if constexpr (N >= 8) x += dppf<0x141>(x);    // row_half_mirror
    if constexpr (N >= 16) x += dppf<0x140>(x);   // row_mirror
    if constexpr (N >= 32) {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    }
    if constexpr (N >= 64) {
        const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(c[0]) + __uint_as_float(c[1]);
    }
    return x;
}
// LDS traffic between lanes of one wave: the wave's LDS operations execute in
// order, so only the compiler has to be kept from reordering them
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }   // by value


template <int N>
__device__ __forceinline__ void ldw(uint32_t* d, const void* s) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int x = 0; x < N / 4; ++x) {
            const uint4 t = reinterpret_cast<const uint4*>(s)[x];
            d[4 * x] = t.x;
            d[4 * x + 1] = t.y;
            d[4 * x + 2] = t.z;
            d[4 * x + 3] = t.w;
        }
    } else if constexpr (N == 2) {
        const uint2 t = *reinterpret_cast<const uint2*>(s);
        d[0] = t.x;
        d[1] = t.y;
    } else {
        static_assert(N == 1, "word count");
        d[0] = *reinterpret_cast<const uint32_t*>(s);
    }
}
template <int N>
__device__ __forceinline__ void stw(void* p, const uint32_t* w) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int x = 0; x < N / 4; ++x)
            reinterpret_cast<uint4*>(p)[x] = make_uint4(w[4 * x], w[4 * x + 1], w[4 * x + 2], w[4 * x + 3]);
    } else if constexpr (N == 2) {
        *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    } else {
        static_assert(N == 1, "word count");
        *reinterpret_cast<uint32_t*>(p) = w[0];
    }
}

// Static shape of one instantiation: head dim D, query heads per KV head G,
// tiles per 32-token chunk TPC (1 for 16-token windows, else 2).
template <int D, int G, int TPC, int BITS, bool ROPE>
struct DecShape {
    static constexpr int CQ = D / 4;                 // channels per lane group (key side)
    static constexpr int KS = D / 32;                // 32-channel MFMA steps (key side)
    static constexpr int MB = D / 16;                // 16-channel blocks (value side)
    static constexpr int NSLOT = G <= 4 ? 2 : 1;     // column slots
    static constexpr int SW = 16 / NSLOT;            // columns per slot
    static constexpr int ROWS = NSLOT * G;           // (item, head) rows of the query-times-scale products
    static constexpr int LPR = 64 / ROWS;            // lanes per product row
    static constexpr int CPL = D / LPR;              // channels per lane in the products
    static constexpr int NV = 4 * TPC;               // scores per lane per quantized item
    // quantized job words per lane (BITS-bit codes): K codes and V codes of every item,
    // V offsets / scales of the lane's own item, K scales / offsets of the lane's product channels
    static constexpr int KCW = TPC * CQ * BITS / 32, VCW = MB * TPC * BITS / 8, VPW = 2 * TPC, KPW = CPL / 2;
    // (RoPE mode: plus the (cos, sin) of the lane's product channels at the chunk's first position)
    static constexpr int O_VC = NSLOT * KCW, O_VO = O_VC + NSLOT * VCW, O_VS = O_VO + VPW, O_KS = O_VS + VPW,
                         O_KO = O_KS + KPW, O_CS = O_KO + KPW, QW = O_CS + (ROPE ? 2 * CPL : 0);
    // bf16 tile job words per lane: K row (CQ bf16) then V (MB blocks x 4 tokens)
    static constexpr int FW = CQ / 2 + 2 * MB;
    static constexpr int RW = QW > FW ? QW : FW;
    static constexpr int QSTR = D + 8;               // bf16 per LDS operand row (padded)
    static_assert(KCW >= 1 && VCW >= 1 && KPW >= 1, "shape");
    static constexpr int KCB = 2 * TPC * D * BITS;   // K (or V) code bytes of one chunk of one item
};

// One unit of wave work.  Quantized job: chunk c of up to NSLOT Quantized windows
// (entries ia, ib), one per column slot.  bf16 job: tile t of one sink / page entry.
struct Job {
    int type;           // 0 none, 1 Quantized, 2 bf16
    int k;              // index in the batch's Quantized-pair / bf16-entry job table
    int ia, ib, c;      // Quantized: batch-local entry indices (ib = -1: slot 1 empty), chunk
    int sa, sb;         // Quantized: slot ids
    int pa, pb;         // Quantized: first positions of the two windows
    int i, t, kind, idx, ntok, Wn, start;   // bf16: entry, tile, kind, page id, valid tokens, block width, position 0
};

// FIN: one split per group, and the workgroup also finishes the step (no finish launch)
template <int D, int G, int TPC, int BITS, bool ROPE, bool FIN>
__global__ void __launch_bounds__(64 * DW) __attribute__((amdgpu_waves_per_eu(2)))
k_decode_split(Geo g, Bufs bf, int layer, const uint16_t* __restrict__ qin, const uint16_t* __restrict__ knew,
               const uint16_t* __restrict__ vnew, float* __restrict__ out, int score_now) {
    using S = DecShape<D, G, TPC, BITS, ROPE>;
    constexpr int CQ = S::CQ, KS = S::KS, MB = S::MB, NSLOT = S::NSLOT, SW = S::SW, LPR = S::LPR, CPL = S::CPL;
    constexpr int NV = S::NV, QSTR = S::QSTR;
    __shared__ uint2 lut[256];            // code byte -> its 4 (INT2) or 2 (INT4, in .x) codes as bf16 integers
    __shared__ uint2 lutk[ROPE ? 256 : 1];  // RoPE mode, key side: the same codes as fp16 integers
    // per wave: the Quantized query operand of the current job (16 rows); shared by the waves
    // (one KV head): rows 0-15 the bf16 query operand (every live column holds its head's
    // query, exact bf16), row 16 zeros
    __shared__ __attribute__((aligned(16))) uint16_t qs[DW][16][QSTR];
    __shared__ __attribute__((aligned(16))) uint16_t qsh[17][QSTR];
    __shared__ float kb[DW][16];                                         // per wave: key-offset bias per column
    __shared__ float s_m[DW][G], s_l[DW][G], s_vb[DW][G];
    __shared__ float s_acc[DW][G][D];
    __shared__ __attribute__((aligned(16))) uint16_t nkv[DW][2][D];     // per wave: the new token's K and V
    __shared__ int s_tok[2];             // one split per group: position and block the token was attended in
    // RoPE mode: (cos, sin) of positions 0..31 of a chunk (rows of the table), and per wave
    // the two windows' key parameters (fp16 offset | scale << 16, channel order)
    __shared__ __attribute__((aligned(16))) float2 ctab[ROPE ? 32 * (D / 2) : 1];
    __shared__ __attribute__((aligned(16))) uint32_t prm[ROPE ? DW : 1][2][D];

    const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int64_t u = unit_of(g, b, layer);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, qg = lane >> 4;            // MFMA column, lane group
    const int slot = n / SW, rn = n % SW;
    const bool hi = rn < G, lo = rn >= SW - G;           // high / low column of head `head`
    const int head = hi ? rn : (lo ? SW - 1 - rn : 0);
    const float lof = lo ? 1.f : 0.f;
    const int W = g.W, Ws = sink_width(g.n_sink), NCH = W / (16 * TPC), NT = W / 16;
    const float scale = 1.4426950408889634f / sqrtf((float)D);   // log2(e) / sqrt(d)

    // product assignment: row (item pitem, head phead), channels [CPL*pcb, CPL*pcb + CPL)
    const int prow = lane / LPR, pitem = prow / G, phead = prow % G, pcb = lane % LPR;

    // ---- prologue: one round trip brings the split block (header + first entries, one
    // per lane), the unit header and the queries; each wave stages its own operands.
    AccEntry me = bf.split_blk[(u * g.n_splits + split) * SPLIT_BLOCK + lane];
    const int n_old = bf.hdr[u].n;       // tokens before this step; the new one sits at position n_old
    const int pending = bf.hdr[u].mass_pending;
    const int n_tok = n_old + 1;
    const uint16_t* qhead = qin + ((int64_t)b * g.h_q + hk * G) * D;
    float qf[CPL];                  // q of the lane's product channels times log2(e)/sqrt(d), fp32
    {
        uint32_t w[CQ / 2];
        ldw<CQ / 2>(w, qhead + head * D + CQ * qg);
        uint32_t w2[CPL / 2];
        ldw<CPL / 2>(w2, qhead + phead * D + CPL * pcb);
        uint32_t kn = 0, vn = 0;
        if (lane < D / 2) {
            kn = reinterpret_cast<const uint32_t*>(knew + ((int64_t)b * g.h_kv + hk) * D)[lane];
            vn = reinterpret_cast<const uint32_t*>(vnew + ((int64_t)b * g.h_kv + hk) * D)[lane];
        }
        if constexpr (ROPE) {
            // the query (this lane's CQ channels of its head) and the step's key (two channels
            // per lane) turned by RoPE at the new position: exact fp64, one bf16 rounding
            constexpr int H2 = D / 2;
            const float2* crow = bf.rope + (int64_t)n_old * H2;
            uint32_t wp[CQ / 2];
            const int cq0 = CQ * qg, part = cq0 < H2 ? cq0 + H2 : cq0 - H2;
            ldw<CQ / 2>(wp, qhead + head * D + part);
            uint32_t knp = 0;
            if (lane < D / 2) {
                const int pl = lane < H2 / 2 ? lane + H2 / 2 : lane - H2 / 2;
                knp = reinterpret_cast<const uint32_t*>(knew + ((int64_t)b * g.h_kv + hk) * D)[pl];
            }
            auto turn = [&](float x, float xp, float2 cs, bool first) -> uint32_t {
                const double a = (double)x, c = (double)cs.x, sn = (double)cs.y, y = (double)xp;
                const double r = first ? __dsub_rn(__dmul_rn(a, c), __dmul_rn(y, sn))
                                       : __dadd_rn(__dmul_rn(a, c), __dmul_rn(y, sn));
                return (uint32_t)f64_to_bf16(r);
            };
#pragma unroll
            for (int x = 0; x < CQ / 2; ++x) {
                const int c0 = cq0 + 2 * x;
                const float2 cs0 = crow[c0 % H2], cs1 = crow[(c0 + 1) % H2];
                w[x] = turn(bf16lo(w[x]), bf16lo(wp[x]), cs0, c0 < H2) |
                       (turn(bf16hi(w[x]), bf16hi(wp[x]), cs1, c0 < H2) << 16);
            }
            if (lane < D / 2) {
                const int c0 = 2 * lane;
                const float2 cs0 = crow[c0 % H2], cs1 = crow[(c0 + 1) % H2];
                kn = turn(bf16lo(kn), bf16lo(knp), cs0, c0 < H2) | (turn(bf16hi(kn), bf16hi(knp), cs1, c0 < H2) << 16);
                if (split == 0)   // for the finish kernel, which stores the token
                    reinterpret_cast<uint32_t*>(bf.krot + (((int64_t)layer * g.B + b) * g.h_kv + hk) * D)[lane] = kn;
            }
            for (int x = threadIdx.x; x < 32 * H2; x += 64 * DW) ctab[x] = bf.rope[x];
        }
        // a code byte -> its codes as bf16 integers (4 of 2 bits, or 2 of 4 bits): one table
        // at a fixed LDS address, so a lookup is one shift of the code byte with the base in
        // the read's immediate offset
        if (threadIdx.x == 0) s_tok[0] = s_tok[1] = -1;
        for (int x = threadIdx.x; x < 256; x += 64 * DW) {
            auto bv = [](int c) -> uint32_t { return __float_as_uint((float)c) >> 16; };   // exact for c < 256
            if constexpr (BITS == 2)
                lut[x] = make_uint2(bv(x & 3) | (bv((x >> 2) & 3) << 16), bv((x >> 4) & 3) | (bv((x >> 6) & 3) << 16));
            else
                lut[x] = make_uint2(bv(x & 15) | (bv(x >> 4) << 16), 0u);
            if constexpr (ROPE) {
                auto hv = [](int c) -> uint32_t { return __builtin_bit_cast(uint16_t, (_Float16)c); };   // exact for c < 2048
                if constexpr (BITS == 2)
                    lutk[x] = make_uint2(hv(x & 3) | (hv((x >> 2) & 3) << 16), hv((x >> 4) & 3) | (hv((x >> 6) & 3) << 16));
                else
                    lutk[x] = make_uint2(hv(x & 15) | (hv(x >> 4) << 16), 0u);
            }
        }
        if (wave == 0) {
            stw<CQ / 2>(&qsh[n][CQ * qg], w);
            if (lane < D / 8) reinterpret_cast<uint4*>(&qsh[16][0])[lane] = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int x = 0; x < CPL / 2; ++x) {
            qf[2 * x] = bf16lo(w2[x]) * scale;
            qf[2 * x + 1] = bf16hi(w2[x]) * scale;
        }
        if constexpr (ROPE) (void)qf;
        if (lane < D / 2) {
            reinterpret_cast<uint32_t*>(nkv[wave][0])[lane] = kn;
            reinterpret_cast<uint32_t*>(nkv[wave][1])[lane] = vn;
        }
    }
    if (split == 0 && hk == 0 && threadIdx.x == 0) bf.hdr[u].pos = n_old;   // for the finish kernel
    const int e_total = __builtin_amdgcn_readlane(me.kind, 0);   // header: entries of the split, first entry
    const int e_begin = __builtin_amdgcn_readlane(me.idx, 0);

    float m_run = M_INIT, l_run = 0.f, lw = 0.f, vbias = 0.f;
    f4_t acc[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = f4_t{0.f, 0.f, 0.f, 0.f};

    const uint16_t* pages = bf.pages + u * (int64_t)g.n_pages * g.page_elems;
    const uint8_t* slots = bf.slots + u * (int64_t)g.n_slots * g.slot_bytes + (int64_t)hk * g.slot_head_bytes;
    const uint16_t* sinks = bf.sinks + u * g.sink_elems;
    float* lse_out = bf.lse_win + lse_win_off(g, u, n_old & 1) + hk * G;   // this step's half

    // ---- job sequence of this wave.  A batch is up to SPLIT_BLOCK - 1 entries, one per
    // lane 1..63.  INT2 entries are paired in order (one pair per job, chunk by chunk),
    // bf16 entries holding tokens follow (all tiles of an entry in one job); jobs go to
    // the waves round robin.  The r-th INT2 (bf16) entry is found by a ballot.
    int xb = 0;                      // split position of lane 1 in the current batch
    bool isq = false, isf = false;   // this lane's entry: INT2 / bf16 with tokens
    int rq = 0, rf = 0;              // rank among the batch's INT2 / bf16 entries
    int nq = 0, nf = 0, npair = 0;
    auto lane_of = [&](bool sel, int rank, int r) __attribute__((always_inline)) -> int {
        return (int)__builtin_ctzll(__ballot(sel && rank == r));
    };
    auto make_q = [&](int k) __attribute__((always_inline)) -> Job {   // INT2 job k: the batch's INT2 entries NSLOT k, NSLOT k + 1
        Job j;
        j.k = k;
        j.c = 0;
        if (k < npair) {
            const int la = lane_of(isq, rq, NSLOT * k);
            const int lb = (NSLOT == 2 && NSLOT * k + 1 < nq) ? lane_of(isq, rq, NSLOT * k + 1) : -1;
            j.type = 1;
            j.sa = __builtin_amdgcn_readlane(me.idx, la);
            j.sb = lb >= 0 ? __builtin_amdgcn_readlane(me.idx, lb) : j.sa;
            j.ia = e_begin + xb + la - 1;                       // accessible-list indices
            j.ib = lb >= 0 ? e_begin + xb + lb - 1 : -1;
            j.pa = __builtin_amdgcn_readlane(me.start, la);
            j.pb = lb >= 0 ? __builtin_amdgcn_readlane(me.start, lb) : j.pa;
        } else {
            j.type = 0;                          // no job left
            j.ia = j.ib = -1;
            j.sa = j.sb = 0;
            j.pa = j.pb = 0;
        }
        return j;
    };
    auto next_q = [&](Job j) __attribute__((always_inline)) -> Job {
        if (j.c + 1 < NCH) {
            j.c += 1;
            return j;
        }
        return make_q(j.k + DW);
    };
    auto make_f = [&](int k) __attribute__((always_inline)) -> Job {   // bf16 job k: all tiles of the k-th bf16 entry
        Job j;
        j.k = k;
        j.t = 0;
        if (k < nf) {
            const int L = lane_of(isf, rf, k);
            const int kind = __builtin_amdgcn_readlane(me.kind, L), start = __builtin_amdgcn_readlane(me.start, L);
            j.type = 2;
            j.i = e_begin + xb + L - 1;
            j.kind = kind;
            j.idx = __builtin_amdgcn_readlane(me.idx, L);
            // (geometry read from the kernel argument, not from captured locals: a select
            // between two captured locals would become a select between stack addresses)
            j.ntok = kind == EK_SINK ? imin(g.n_sink, n_tok) : imin(g.W, n_tok - start);
            j.Wn = kind == EK_SINK ? sink_width(g.n_sink) : g.W;
            j.start = kind == EK_SINK ? 0 : start;
        } else {
            j.type = 0;                          // no job left
            j.i = 0;
            j.kind = EK_SINK;
            j.idx = 0;
            j.ntok = 0;
            j.Wn = sink_width(g.n_sink);
            j.start = 0;
        }
        return j;
    };
    auto next_f = [&](Job j) __attribute__((always_inline)) -> Job {
        if (16 * (j.t + 1) < j.ntok) {
            j.t += 1;
            return j;
        }
        return make_f(j.k + DW);
    };

    struct Raw {
        uint32_t w[S::RW];
    };
    // Every load address is a wave-uniform base (SGPRs) plus an unsigned 32-bit lane
    // offset, which the hardware adds itself (global loads with an SGPR base).
    // (code bytes: a lane's K row of a tile is CQ*BITS/8 bytes, its V bytes per channel
    // block and tile BITS/2; one tensor's codes W*D*BITS/8)
    constexpr int KRB = CQ * BITS / 8, VTB = BITS / 2;
    const uint32_t cbytes = (uint32_t)(W * D * BITS / 8);
    const uint32_t kc_lane = (uint32_t)((n * 4 + qg) * TPC * KRB);                    // K codes: token row n, group qg
    const uint32_t vc_lane = cbytes + (uint32_t)((n * 4 + qg) * MB * TPC * VTB);       // V codes: channel row n
    const uint32_t vp_lane = 2 * cbytes + (uint32_t)(4 * D + qg * NT * 8);            // V offsets (V scales + 2W)
    // the lane's product channels: CPL of them from position CPL*pcb of the key-side channel
    // order (in RoPE mode all in one half, pairing as in lay_kc_pos)
    const int pch0 = [&]() {
        const int pos = CPL * pcb, pqg = pos / CQ, pcc = pos % CQ;
        if constexpr (!ROPE) return pos;
        return pcc < CQ / 2 ? pqg * (CQ / 2) + pcc : D / 2 + pqg * (CQ / 2) + pcc - CQ / 2;
    }();
    const uint32_t kp_lane = 2 * cbytes + (uint32_t)(pch0 * 2);                       // K offsets (K scales + 2D)
    auto load_q = [&](const Job& j, Raw& R) __attribute__((always_inline)) {
        const uint32_t oa = (uint32_t)j.sa * (uint32_t)g.slot_bytes, ob = (uint32_t)j.sb * (uint32_t)g.slot_bytes;
        const uint8_t* ca = slots + oa + (uint32_t)(j.c * 16 * 4 * TPC * KRB);   // chunk c of item a
        const uint8_t* cb = slots + ob + (uint32_t)(j.c * 16 * 4 * TPC * KRB);
        ldw<S::KCW>(R.w, ca + kc_lane);
        ldw<S::VCW>(R.w + S::O_VC, slots + oa + (uint32_t)(j.c * S::KCB) + vc_lane);
        if constexpr (NSLOT == 2) {
            ldw<S::KCW>(R.w + S::KCW, cb + kc_lane);
            ldw<S::VCW>(R.w + S::O_VC + S::VCW, slots + ob + (uint32_t)(j.c * S::KCB) + vc_lane);
        }
        // the lane's own item (V parameters) and the item of its products (K parameters)
        const uint32_t oo = (slot == 0 ? oa : ob) + vp_lane + (uint32_t)(TPC * j.c * 8);
        ldw<S::VPW>(R.w + S::O_VO, slots + oo);
        ldw<S::VPW>(R.w + S::O_VS, slots + oo + 2 * W);
        const uint32_t op = (pitem == 0 ? oa : ob) + kp_lane;
        ldw<S::KPW>(R.w + S::O_KS, slots + op + 2 * D);
        ldw<S::KPW>(R.w + S::O_KO, slots + op);
        if constexpr (ROPE) {   // (cos, sin) of the product channels' pairs at the chunk's first position
            const int A = (pitem == 0 ? j.pa : j.pb) + 32 * j.c;
            ldw<2 * CPL>(R.w + S::O_CS, bf.rope + (int64_t)A * (D / 2) + pch0 % (D / 2));
        }
    };
    // a bf16 job's K and V bytes of this lane (CQ * 2 bytes each)
    auto f_src = [&](const Job& j, const uint8_t*& kl, const uint8_t*& vl) __attribute__((always_inline)) {
        const int tpc = lay_tpc(j.Wn), nt16 = j.Wn / 16;
        const uint8_t* kbase = reinterpret_cast<const uint8_t*>(
            (j.kind == EK_SINK ? sinks : pages + (int64_t)j.idx * g.page_elems) + (int64_t)(2 * hk) * j.Wn * D);
        const uint8_t* vbase = kbase + (int64_t)j.Wn * D * 2;
        const int t0 = j.t / tpc, t1 = j.t % tpc;   // chunk, tile within it
        kl = kbase + (uint32_t)(t0 * 16 * 4 * tpc * CQ * 2 + t1 * CQ * 2) + (uint32_t)(((n * 4 + qg) * tpc) * CQ * 2);
        vl = vbase + (uint32_t)(j.t * MB * 8) + (uint32_t)((n * 4 + qg) * nt16 * MB * 8);
    };
    auto load_f = [&](const Job& j, Raw& R) __attribute__((always_inline)) {
        const uint8_t *kl, *vl;
        f_src(j, kl, vl);
        ldw<CQ / 2>(R.w, kl);
        ldw<2 * MB>(R.w + CQ / 2, vl);
    };

    // online softmax over the lane's NVV scores.  The reference max is shared by every
    // column of a head (max over the 4 lane groups and both column slots), so the slots
    // merge by plain addition at the end.  It moves lazily: only when a score exceeds it
    // by more than 8 (log2 units), so probabilities stay below 2^8 and the rescale of the
    // accumulators is rare after the wave's first job.
    auto softmax = [&](float* s, float* p, int nvv) __attribute__((always_inline)) {
        float mx = s[0];
        int v = 1;
        for (; v + 1 < nvv; v += 2) mx = max3(mx, s[v], s[v + 1]);
        if (v < nvv) mx = max2(mx, s[v]);
        mx = qg_max(mx);
        if constexpr (NSLOT == 2) mx = max2(mx, ror8(mx));
        if (__any(mx > m_run + 8.f)) {
            const float mnew = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
            l_run *= alpha;
            lw *= alpha;
            vbias *= alpha;
#pragma unroll
            for (int m = 0; m < MB; ++m) acc[m] *= alpha;
            m_run = mnew;
        }
        float ps = 0.f;
        for (int v = 0; v < nvv; ++v) {
            p[v] = __builtin_amdgcn_exp2f(s[v] - m_run);
            ps += p[v];
        }
        l_run += ps;
        lw += ps;
    };
    // bf16 pair of x: high lanes get bf16(x), low lanes bf16(x - bf16(x))
    auto hilo = [&](float x0, float x1) -> uint32_t {
        const uint32_t r = bf16x2_rne(x0, x1);
        return bf16x2_rne(fmaf(-lof, bf16lo(r), x0), fmaf(-lof, bf16hi(r), x1));
    };
    auto lut4 = [&](uint32_t w, int byte) -> u2_t {   // INT2: 4 codes of one byte
        const uint2 a = lut[(w >> (8 * byte)) & 0xffu];
        return u2_t{a.x, a.y};
    };
    auto lut2 = [&](uint32_t w, int byte) -> uint32_t {   // INT4: 2 codes of one byte
        return lut[(w >> (8 * byte)) & 0xffu].x;
    };
    // MFMA A operands from a lane's code words.  Key side, tile tc, 32-channel step ks:
    // channels CQ*qg + 8ks .. + 7 of the lane's token row.  Value side, channel block m:
    // tokens 4*qg .. + 3 of each tile of the chunk (zeros in the second half when TPC = 1).
    auto key_codes = [&](const uint32_t* w, int tc, int ks) __attribute__((always_inline)) -> u4_t {
        if constexpr (BITS == 2) {
            const int by = tc * (CQ / 4) + 2 * ks;
            const uint32_t x = w[by >> 2];
            const u2_t a0 = lut4(x, by & 3), a1 = lut4(x, (by & 3) + 1);
            return u4_t{a0.x, a0.y, a1.x, a1.y};
        } else {
            const uint32_t x = w[tc * (CQ / 8) + ks];
            return u4_t{lut2(x, 0), lut2(x, 1), lut2(x, 2), lut2(x, 3)};
        }
    };
    auto value_codes = [&](const uint32_t* w, int m) __attribute__((always_inline)) -> u4_t {
        if constexpr (BITS == 2) {
            if constexpr (TPC == 2) {
                const int by = 2 * m;
                const uint32_t x = w[by >> 2];
                const u2_t a0 = lut4(x, by & 3), a1 = lut4(x, (by & 3) + 1);
                return u4_t{a0.x, a0.y, a1.x, a1.y};
            } else {
                const u2_t a0 = lut4(w[m >> 2], m & 3);
                return u4_t{a0.x, a0.y, 0u, 0u};
            }
        } else {
            if constexpr (TPC == 2) {
                const uint32_t x = w[m];
                return u4_t{lut2(x, 0), lut2(x, 1), lut2(x, 2), lut2(x, 3)};
            } else {
                const uint32_t x = w[m >> 1];
                const int by = 2 * (m & 1);
                return u4_t{lut2(x, by), lut2(x, by + 1), 0u, 0u};
            }
        }
    };
    auto lse_store = [&](bool mine, int ie) {
        const float t = qg_sum(lw);
        if (mine) {
            if (qg == 0 && hi) lse_out[(int64_t)ie * g.h_q + head] = m_run + log2f(t);
            lw = 0.f;
        }
    };

    const uint16_t* qrow_a = (NSLOT == 2 && slot) ? &qsh[16][CQ * qg] : &qs[wave][n][CQ * qg];   // slot 0 columns only
    const uint16_t* qrow_b = (NSLOT == 2 && !slot) ? &qsh[16][CQ * qg] : &qs[wave][n][CQ * qg];  // slot 1 columns only
    // RoPE mode, key side of a Quantized job (see process_q): the 8 codes of positions
    // 8ks .. 8ks + 7 of the lane's row of tile tc, as 4 pairs of fp16 integers
    auto codes8 = [&](const uint32_t* w, int tc, int ks, uint32_t* c) __attribute__((always_inline)) {
        if constexpr (BITS == 2) {
            const int by = tc * (CQ / 4) + 2 * ks;
            const uint32_t x = w[by >> 2];
            const uint2 a0 = lutk[(x >> (8 * (by & 3))) & 0xffu], a1 = lutk[(x >> (8 * ((by & 3) + 1))) & 0xffu];
            c[0] = a0.x;
            c[1] = a0.y;
            c[2] = a1.x;
            c[3] = a1.y;
        } else {
            const uint32_t x = w[tc * (CQ / 8) + ks];
#pragma unroll
            for (int k = 0; k < 4; ++k) c[k] = lutk[(x >> (8 * k)) & 0xffu].x;
        }
    };
    // RoPE mode: the turned keys of one item for channel pairs (i, i + D/2), i = i0 .. i0 + 7,
    // at chunk position u, as bf16 high / low MFMA operands of the first-half and the
    // second-half channel blocks
    auto rope_keys = [&](const uint32_t* w, const uint32_t* pr, int tc, int ks, const float2* cs, u4_t& hf, u4_t& lf,
                         u4_t& hs, u4_t& ls) __attribute__((always_inline)) {
        uint32_t cf[4], cb[4];
        codes8(w, tc, ks, cf);
        codes8(w, tc, ks + KS / 2, cb);
        const int i0 = qg * (CQ / 2) + 8 * ks;
        uint4 pf0 = *reinterpret_cast<const uint4*>(pr + i0), pf1 = *reinterpret_cast<const uint4*>(pr + i0 + 4);
        uint4 pb0 = *reinterpret_cast<const uint4*>(pr + D / 2 + i0), pb1 = *reinterpret_cast<const uint4*>(pr + D / 2 + i0 + 4);
        const uint32_t pf[8] = {pf0.x, pf0.y, pf0.z, pf0.w, pf1.x, pf1.y, pf1.z, pf1.w};
        const uint32_t pb[8] = {pb0.x, pb0.y, pb0.z, pb0.w, pb1.x, pb1.y, pb1.z, pb1.w};
        float yf[8], yb[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            // (offset, scale) and the code, all fp16: one mixed-precision fma each, exact inputs
            const h2_t a = __builtin_bit_cast(h2_t, pf[k]), bb = __builtin_bit_cast(h2_t, pb[k]);
            const h2_t c2f = __builtin_bit_cast(h2_t, cf[k >> 1]), c2b = __builtin_bit_cast(h2_t, cb[k >> 1]);
            const _Float16 chf = (k & 1) ? c2f.y : c2f.x, chb = (k & 1) ? c2b.y : c2b.x;
            const float xf = fmaf((float)chf, (float)a.y, (float)a.x), xb = fmaf((float)chb, (float)bb.y, (float)bb.x);
            yf[k] = xf * cs[k].x - xb * cs[k].y;
            yb[k] = xb * cs[k].x + xf * cs[k].y;
        }
        // high parts RNE, low parts exact remainders (bf16x2_rest)
        uint32_t h1[4], l1[4], h2[4], l2[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            h1[k] = bf16x2_rne(yf[2 * k], yf[2 * k + 1]);
            l1[k] = bf16x2_rest(h1[k], yf[2 * k], yf[2 * k + 1]);
            h2[k] = bf16x2_rne(yb[2 * k], yb[2 * k + 1]);
            l2[k] = bf16x2_rest(h2[k], yb[2 * k], yb[2 * k + 1]);
        }
        hf = u4_t{h1[0], h1[1], h1[2], h1[3]};
        lf = u4_t{l1[0], l1[1], l1[2], l1[3]};
        hs = u4_t{h2[0], h2[1], h2[2], h2[3]};
        ls = u4_t{l2[0], l2[1], l2[2], l2[3]};
    };

    // A Quantized job in two parts: products_q writes the job's query operand to LDS and reads
    // the lane's columns back, scores_q does the rest.
    struct QOp {
        u4_t a[DecShape<D, G, TPC, BITS, ROPE>::KS], b[DecShape<D, G, TPC, BITS, ROPE>::KS];
        float c0;
    };
    auto products_q = [&](const Job& j, const Raw& R, QOp& op) __attribute__((always_inline)) {
        (void)j;
        // (1) q * sclK for every (item, head, channel) once, split into bf16 high + low
        //     rows of the wave's operand block; key-offset bias sum_c q_c offK_c per row.
        //     RoPE mode: instead the query turned back by the chunk's first position A,
        //     R(A)^T q, whose product with the keys turned by their offset u in the chunk
        //     equals q . R(A + u) k; the key parameters go to LDS for the dequantization.
        if constexpr (ROPE) {
            constexpr int H2 = D / 2;
            const bool first = pch0 < H2;
            const uint16_t* qrow = &qsh[phead][0];
            uint32_t hw[CPL / 2], lw2[CPL / 2];
#pragma unroll
            for (int x = 0; x < CPL / 2; ++x) {
                float qa[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int ch = pch0 + 2 * x + e, pc = first ? ch + H2 : ch - H2;
                    const float qv = bf16_to_f32(qrow[ch]), qp = bf16_to_f32(qrow[pc]);
                    const float c = __uint_as_float(R.w[S::O_CS + 4 * x + 2 * e]);
                    const float sn = __uint_as_float(R.w[S::O_CS + 4 * x + 2 * e + 1]);
                    qa[e] = (first ? fmaf(qp, sn, qv * c) : fmaf(-qp, sn, qv * c)) * scale;
                }
                hw[x] = bf16x2_trunc(qa[0], qa[1]);
                lw2[x] = bf16x2_rne(qa[0] - bf16lo(hw[x]), qa[1] - bf16hi(hw[x]));
            }
            wave_lds_fence();
            stw<CPL / 2>(&qs[wave][pitem * SW + phead][CPL * pcb], hw);
            stw<CPL / 2>(&qs[wave][pitem * SW + SW - 1 - phead][CPL * pcb], lw2);
            if (phead == 0) {
#pragma unroll
                for (int x = 0; x < CPL / 2; ++x) {
                    const uint32_t o = R.w[S::O_KO + x], sc = R.w[S::O_KS + x];
                    prm[wave][pitem][pch0 + 2 * x] = (o & 0xFFFFu) | (sc << 16);
                    prm[wave][pitem][pch0 + 2 * x + 1] = (o >> 16) | (sc & 0xFFFF0000u);
                }
            }
            wave_lds_fence();
        } else {
            float bias = 0.f;
            uint32_t hw[CPL / 2], lw2[CPL / 2];
#pragma unroll
            for (int x = 0; x < CPL / 2; ++x) {
                const f2_t o2 = h2f(R.w[S::O_KO + x]);
                const float x0 = mul_h_lo(qf[2 * x], R.w[S::O_KS + x]), x1 = mul_h_hi(qf[2 * x + 1], R.w[S::O_KS + x]);
                bias = fmaf(qf[2 * x], o2.x, bias);
                bias = fmaf(qf[2 * x + 1], o2.y, bias);
                hw[x] = bf16x2_trunc(x0, x1);
                lw2[x] = bf16x2_rne(x0 - bf16lo(hw[x]), x1 - bf16hi(hw[x]));
            }
            bias = group_sum<LPR>(bias);
            wave_lds_fence();
            stw<CPL / 2>(&qs[wave][pitem * SW + phead][CPL * pcb], hw);
            stw<CPL / 2>(&qs[wave][pitem * SW + SW - 1 - phead][CPL * pcb], lw2);
            if (pcb == 0) kb[wave][pitem * SW + phead] = bias;   // (read by the high column)
            wave_lds_fence();
        }
        // (2) the lane's column of the operand, once per window: each window's MFMAs see
        //     only the columns of its own slot (the other slot's lanes read the zero row), so
        //     both windows accumulate into one score tile
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            op.a[ks] = *reinterpret_cast<const u4_t*>(qrow_a + 8 * ks);
            if constexpr (NSLOT == 2) op.b[ks] = *reinterpret_cast<const u4_t*>(qrow_b + 8 * ks);
        }
        op.c0 = (hi && !ROPE) ? kb[wave][n] : 0.f;   // key-offset bias, once per head (high column)
    };
    auto scores_q = [&](const Job& j, const Raw& R, const QOp& op) __attribute__((always_inline)) {
        const u4_t* bqa = op.a;
        const u4_t* bqb = op.b;
        const float c0 = op.c0;
        // (3) scores S^T[token][column] = codes . (q * sclK) + bias, log2 units.  RoPE mode:
        //     dequantized keys turned by their offset u in the chunk, times R(A)^T q
        float s[NV];
        if constexpr (!ROPE) {
            // every code-table lookup of the key side goes out before the first MFMA, so that
            // their LDS latencies overlap (consumed one MFMA behind, they form a chain of 2*KS*TPC*NSLOT
            // round trips); the two tiles' chains then alternate
            u4_t kc[TPC][KS][NSLOT];
#pragma unroll
            for (int tc = 0; tc < TPC; ++tc)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    kc[tc][ks][0] = key_codes(R.w, tc, ks);
                    if constexpr (NSLOT == 2) kc[tc][ks][NSLOT - 1] = key_codes(R.w + S::KCW, tc, ks);
                }
            __builtin_amdgcn_sched_barrier(0);
            f4_t d[TPC];
#pragma unroll
            for (int tc = 0; tc < TPC; ++tc) d[tc] = f4_t{c0, c0, c0, c0};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int sl = 0; sl < NSLOT; ++sl)
#pragma unroll
                    for (int tc = 0; tc < TPC; ++tc) d[tc] = mfma32(kc[tc][ks][sl], sl ? bqb[ks] : bqa[ks], d[tc]);
#pragma unroll
            for (int tc = 0; tc < TPC; ++tc)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[4 * tc + i] = d[tc][i] + mirror<SW>(d[tc][i]);   // high + low query parts
        }
#pragma unroll
        for (int tc = 0; tc < (ROPE ? TPC : 0); ++tc) {
            f4_t d = {c0, c0, c0, c0};
            if constexpr (ROPE) {
                const int u = 16 * tc + n;
#pragma unroll
                for (int ks = 0; ks < KS / 2; ++ks) {
                    const float2* cs = &ctab[u * (D / 2) + qg * (CQ / 2) + 8 * ks];
                    u4_t hf, lf, hs, ls;
                    rope_keys(R.w, &prm[wave][0][0], tc, ks, cs, hf, lf, hs, ls);
                    d = mfma32(hf, bqa[ks], d);
                    d = mfma32(lf, bqa[ks], d);
                    d = mfma32(hs, bqa[ks + KS / 2], d);
                    d = mfma32(ls, bqa[ks + KS / 2], d);
                    if constexpr (NSLOT == 2) {
                        rope_keys(R.w + S::KCW, &prm[wave][1][0], tc, ks, cs, hf, lf, hs, ls);
                        d = mfma32(hf, bqb[ks], d);
                        d = mfma32(lf, bqb[ks], d);
                        d = mfma32(hs, bqb[ks + KS / 2], d);
                        d = mfma32(ls, bqb[ks + KS / 2], d);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) s[4 * tc + i] = d[i] + mirror<SW>(d[i]);   // high + low query parts
        }
        if (NSLOT == 2 && j.ib < 0) {
#pragma unroll
            for (int v = 0; v < NV; ++v) s[v] = slot ? -INFINITY : s[v];
        }
        float p[NV];
        softmax(s, p, NV);
        // (4) P' = p * sclV (high / low bf16 parts); value-offset bias sum_t p_t offV_t
        uint32_t P[NV / 2];
#pragma unroll
        for (int x = 0; x < NV / 2; ++x) {
            const f2_t o2 = h2f(R.w[S::O_VO + x]);
            vbias = fmaf(p[2 * x], o2.x, vbias);
            vbias = fmaf(p[2 * x + 1], o2.y, vbias);
            P[x] = hilo(mul_h_lo(p[2 * x], R.w[S::O_VS + x]), mul_h_hi(p[2 * x + 1], R.w[S::O_VS + x]));
        }
        u4_t pa, pb;
        if constexpr (TPC == 2) {
            pa = u4_t{P[0], P[1], P[2], P[3]};
        } else {
            pa = u4_t{P[0], P[1], 0u, 0u};
        }
        if constexpr (NSLOT == 2) {
            const u4_t z = {0u, 0u, 0u, 0u};
            pb = slot ? pa : z;
            pa = slot ? z : pa;
        }
        // (5) O^T[channel][column] += codes^T . P'
        //     (each slot's lookups all go out before its MFMAs, as on the key side)
        {
            u4_t vc[MB];
#pragma unroll
            for (int m = 0; m < MB; ++m) vc[m] = value_codes(R.w + S::O_VC, m);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < MB; ++m) acc[m] = mfma32(vc[m], pa, acc[m]);
        }
        if (NSLOT == 2 && j.ib >= 0) {
            u4_t vc[MB];
#pragma unroll
            for (int m = 0; m < MB; ++m) vc[m] = value_codes(R.w + S::O_VC + S::VCW, m);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < MB; ++m) acc[m] = mfma32(vc[m], pb, acc[m]);
        }
        // (6) both windows end on their last chunk: log-sum-exp of their mass per head
        if (j.c + 1 == NCH) lse_store(slot == 0 || j.ib >= 0, slot == 0 ? j.ia : j.ib);
    };

    auto process_f = [&](const Job& j, const Raw& R) __attribute__((always_inline)) {
        u4_t bq[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bq[ks] = *reinterpret_cast<const u4_t*>(&qsh[n][CQ * qg + 8 * ks]);
        uint32_t kw[CQ / 2], vw[2 * MB];
#pragma unroll
        for (int x = 0; x < CQ / 2; ++x) kw[x] = R.w[x];
#pragma unroll
        for (int x = 0; x < 2 * MB; ++x) vw[x] = R.w[CQ / 2 + x];
        const int pt = n_old - j.start - 16 * j.t;    // the new token's row in this tile, if any
        if (pt >= 0 && pt < 16 && n_old - j.start < j.ntok) {   // (a sink block's spare rows never hold it)
            // its block, for whoever stores the token: this workgroup at its end (one split per
            // group) or the finish kernel (one writer per unit)
            if (lane == 0) {
                const int tp = j.kind == EK_SINK ? -2 : j.idx;
                if constexpr (FIN) {
                    s_tok[0] = n_old;
                    s_tok[1] = tp;
                } else if (hk == 0) {
                    bf.hdr[u].tok_page = tp;
                    bf.hdr[u].tok_at = n_old;
                }
            }
            // its K row (lanes of token row pt) and its V column entries come from LDS
            if (n == pt) {
#pragma unroll
                for (int x = 0; x < CQ / 2; ++x) kw[x] = reinterpret_cast<const uint32_t*>(&nkv[wave][0][CQ * qg])[x];
            }
            if (qg == (pt >> 2)) {
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    const uint32_t v = nkv[wave][1][16 * m + n];
                    const int x = 2 * m + ((pt & 3) >> 1);
                    vw[x] = (pt & 1) ? ((vw[x] & 0xFFFFu) | (v << 16)) : ((vw[x] & 0xFFFF0000u) | v);
                }
            }
        }
        if (16 * (j.t + 1) > j.ntok) {
            // a tile past the block's last token: its rows beyond hold whatever the page held
            // before (a fresh page is not cleared), so their values are zeroed (their
            // probabilities are 0, and 0 * NaN would not be)
            const int r0 = 16 * j.t + 4 * qg;
            const uint32_t m0 = (r0 < j.ntok ? 0x0000FFFFu : 0u) | (r0 + 1 < j.ntok ? 0xFFFF0000u : 0u);
            const uint32_t m1 = (r0 + 2 < j.ntok ? 0x0000FFFFu : 0u) | (r0 + 3 < j.ntok ? 0xFFFF0000u : 0u);
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                vw[2 * m] &= m0;
                vw[2 * m + 1] &= m1;
            }
        }
        f4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) d = mfma32(u4_t{kw[4 * ks], kw[4 * ks + 1], kw[4 * ks + 2], kw[4 * ks + 3]}, bq[ks], d);
        float s[4], p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = slot == 0 && 16 * j.t + 4 * qg + i < j.ntok;
            s[i] = valid ? d[i] * scale : -INFINITY;
        }
        softmax(s, p, 4);
        const u2_t P = {hilo(p[0], p[1]), hilo(p[2], p[3])};
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[m] = mfma16(u2_t{vw[2 * m], vw[2 * m + 1]}, P, acc[m]);
        if (16 * (j.t + 1) >= j.ntok) lse_store(slot == 0, j.i);
    };

    // batches of up to SPLIT_BLOCK - 1 entries: the first from the split block, later
    // ones (splits longer than a block) straight from the accessible list
    int x = 0;                   // this lane's position in the split
    bool valid = false;          // this lane holds an entry of the batch
    auto classify = [&]() __attribute__((always_inline)) {
        x = xb + lane - 1;
        valid = lane >= 1 && x < e_total;
        if (xb > 0 && valid) me = bf.acc[u * g.n_acc_max + e_begin + x];
        isq = isf = false;
        if (valid) {
            if (me.kind == EK_SLOT) {
                isq = me.idx >= 0;
            } else {
                const int nt = me.kind == EK_SINK ? imin(g.n_sink, n_tok) : imin(W, n_tok - me.start);
                isf = nt > 0 && (me.kind == EK_SINK || me.idx >= 0);
                if (!isf && wave == 0)           // no tokens yet: window log-sum-exp -inf, no mass
                    for (int h = 0; h < G; ++h) lse_out[(int64_t)(e_begin + x) * g.h_q + h] = -INFINITY;
            }
        }
        const uint64_t mq = __ballot(isq), mf = __ballot(isf);
        rq = __builtin_amdgcn_mbcnt_hi((uint32_t)(mq >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mq, 0));
        rf = __builtin_amdgcn_mbcnt_hi((uint32_t)(mf >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mf, 0));
        nq = __popcll(mq);
        nf = __popcll(mf);
        npair = (nq + NSLOT - 1) / NSLOT;
    };
    // the wave's first bf16 job of a batch: its jobs continue the round robin after the
    // Quantized pairs
    auto first_f = [&]() __attribute__((always_inline)) { return make_f(((wave - npair) % DW + DW) % DW); };
    xb = 0;
    classify();
    __syncthreads();                 // the code table and the shared query rows
    for (xb = 0; xb == 0 || xb < e_total; xb += SPLIT_BLOCK - 1) {
        if (xb > 0) classify();
        {   // one job in flight per wave: the second wave on each SIMD hides its load latency
            Raw ra;
            Job j = make_q(wave);
            while (j.type != 0) {
                QOp op;
                load_q(j, ra);
                products_q(j, ra, op);
                scores_q(j, ra, op);
                j = next_q(j);
            }
        }
        {
            Raw ra;
            Job j = first_f();
            while (j.type != 0) {
                load_f(j, ra);
                process_f(j, ra);
                j = next_f(j);
            }
        }
        // the previous step's pending window-mass shares of this batch's entries (from its
        // window and row log-sum-exps, the other half of the window array): each entry
        // once, by the KV head whose index matches its position in the split
        if (pending && wave == DW - 1 && valid && x % g.h_kv == hk && me.win >= 0) {
            const float* row = bf.lse_win + lse_win_off(g, u, (n_old - 1) & 1) + (int64_t)(e_begin + x) * g.h_q;
            const float* lg = bf.lse_glob + lse_glob_off(g, u, (n_old - 1) & 1);
            double* sc = mass_target(g, bf) + u * g.n_windows + me.win;
            const double s0 = *sc;
            const double sm = entry_mass(row, lg, g.h_q);
            *sc = s0 + sm / g.h_q;
        }
    }

    // ---- wave state -> workgroup partial for this split.  All columns of a head share
    // the reference max, so the head's output is the plain sum of its high and low
    // columns and of both column slots; the value-offset bias joins once per head in the
    // block merge.
    float lt = qg_sum(l_run);
    float vb = qg_sum(vbias);
    float a[MB][4];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) a[m][i] = acc[m][i] + mirror<SW>(acc[m][i]);   // high + low columns
    if constexpr (NSLOT == 2) {   // row_mirror takes a slot's (high, low) pair to the other slot's
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) a[m][i] += dppf<0x140>(a[m][i]);
        lt += ror8(lt);
        vb += ror8(vb);
    }
    // (the sums stay ahead of the store branch below, where each folds with its lane move)
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(a[m][i]));
    if (slot == 0 && hi) {
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_acc[wave][rn][16 * m + 4 * qg + i] = a[m][i];
        if (qg == 0) {
            s_m[wave][rn] = m_run;
            s_l[wave][rn] = lt;
            s_vb[wave][rn] = vb;
        }
    }
    __syncthreads();
    // One split per group (FIN): the merge is the heads' output, and this workgroup also
    // does what the finish kernel does otherwise.  Else: the split's partial.
    float* pacc = bf.part_acc + ((u * g.n_splits + split) * (int64_t)g.h_q + hk * G) * D;
    float2* pml = bf.part_ml + (u * g.n_splits + split) * (int64_t)g.h_q + hk * G;
    float* og = out + ((int64_t)b * g.h_q + hk * G) * D;
    float* lseg = bf.lse_glob + lse_glob_off(g, u, n_old & 1) + hk * G;
    for (int x = threadIdx.x; x < G * D; x += 64 * DW) {
        const int gg = x / D, c = x % D;
        float M = s_m[0][gg];
#pragma unroll
        for (int w = 1; w < DW; ++w) M = fmaxf(M, s_m[w][gg]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < DW; ++w) {
            const float f = __builtin_amdgcn_exp2f(s_m[w][gg] - M);
            L += f * s_l[w][gg];
            A += f * (s_acc[w][gg][c] + s_vb[w][gg]);
        }
        if constexpr (FIN) {
            og[(int64_t)gg * D + c] = A / L;
            if (c == 0) lseg[gg] = M + log2f(L);
        } else {
            pacc[(int64_t)gg * D + c] = A;
            if (c == 0) pml[gg] = make_float2(M, L);
        }
    }
    if constexpr (!FIN) return;
    // ---- the step's token into the block this workgroup attended it in (a window the
    // router did not prepare is an error); then the last of the unit's h_kv workgroups to
    // get here advances the unit's token count (every workgroup of the unit has read it by
    // then: the count is an atomic, so the workgroups may run on any XCDs).
    const int tok_at = s_tok[0], page = s_tok[1];
    const bool ok = tok_at == n_old;
    if (ok && threadIdx.x < D) {
        uint16_t* blk;
        int Wp = g.W, i;
        if (page == -2) {
            blk = bf.sinks + u * g.sink_elems;
            Wp = sink_width(g.n_sink);
            i = n_old;
        } else {
            i = (n_old - g.n_sink) % g.W;
            blk = bf.pages + u * (int64_t)g.n_pages * g.page_elems + (int64_t)page * g.page_elems;
        }
        uint16_t* kh = blk + (int64_t)(2 * hk) * Wp * D;
        kh[lay_k(i, threadIdx.x, D, Wp)] = nkv[0][0][threadIdx.x];
        kh[(int64_t)Wp * D + lay_v(i, threadIdx.x, D, Wp)] = nkv[0][1][threadIdx.x];
    }
    if (threadIdx.x == 0) {
        if (!ok) atomicOr(&bf.hdr[u].status, QEVICT_DEV_E_WINDOW);
        const uint32_t done = __hip_atomic_fetch_add(bf.unit_arr + u, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
        if (done == (uint32_t)g.h_kv) {
            __hip_atomic_store(bf.unit_arr + u, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (ok) bf.hdr[u].n = n_old + 1;
            bf.hdr[u].mass_pending = score_now;
        }
    }
}

hipError_t launch_decode(const Geo& g, const Bufs& bf, int layer, const uint16_t* q, const uint16_t* k_new,
                         const uint16_t* v_new, float* out, int score_now, hipStream_t s, hipEvent_t ev0,
                         hipEvent_t ev1) {
    if (g.fuse && (g.n_splits != 1 || !out)) return hipErrorInvalidValue;
    const dim3 grid(g.n_splits, g.h_kv, g.B), block(64 * DW);
    const int G = g.h_q / g.h_kv, TPC = lay_tpc(g.W);
    const bool rope = (g.flags & QEVICT_F_ROPE) != 0, fin = g.fuse != 0;
#define QV_DEC3(D_, G_, T_, B_, R_, F_)                                                        \
    if (g.d == D_ && G == G_ && TPC == T_ && g.qbits == B_ && rope == R_ && fin == F_) {       \
        if (ev0)                                                                               \
            hipExtLaunchKernelGGL((k_decode_split<D_, G_, T_, B_, R_, F_>), grid, block, 0, s, ev0, ev1, 0, g, bf, \
                                  layer, q, k_new, v_new, out, score_now);                     \
        else                                                                                   \
            hipLaunchKernelGGL((k_decode_split<D_, G_, T_, B_, R_, F_>), grid, block, 0, s, g, bf, layer, q, k_new, \
                               v_new, out, score_now);                                         \
        return hipGetLastError();                                                              \
    }
#define QV_DEC2(D_, G_, T_, B_, R_) QV_DEC3(D_, G_, T_, B_, R_, false) QV_DEC3(D_, G_, T_, B_, R_, true)
#define QV_DEC1(D_, G_, T_, B_) QV_DEC2(D_, G_, T_, B_, false) QV_DEC2(D_, G_, T_, B_, true)
#define QV_DEC(D_, G_, T_) QV_DEC1(D_, G_, T_, 2) QV_DEC1(D_, G_, T_, 4)
    QV_DEC(128, 1, 2) QV_DEC(128, 2, 2) QV_DEC(128, 4, 2) QV_DEC(128, 8, 2)
    QV_DEC(64, 1, 2) QV_DEC(64, 2, 2) QV_DEC(64, 4, 2) QV_DEC(64, 8, 2)
    QV_DEC(128, 1, 1) QV_DEC(128, 2, 1) QV_DEC(128, 4, 1) QV_DEC(128, 8, 1)
    QV_DEC(64, 1, 1) QV_DEC(64, 2, 1) QV_DEC(64, 4, 1) QV_DEC(64, 8, 1)
#undef QV_DEC
#undef QV_DEC1
#undef QV_DEC2
#undef QV_DEC3
    return hipErrorInvalidValue;
}


// ------------------------------------------------------------------------------------ finish
// One workgroup per (query head, sequence): o_h = sum_s 2^(m_s - M) acc_s / L with
// L = sum_s 2^(m_s - M) l_s and LSE_h = M + log2 L (log2 domain), the step's token into
// its block, the token count.  The heads' shares of each window's mass follow from LSE_h
// and the window log-sum-exps; the next split kernel (or the router / an export) folds
// them into the scores.
constexpr int FN_THREADS = 256;
constexpr int FN_MAXS = 512;            // splits (the host caps n_splits below this)

// sum / max over all 64 lanes without LDS (DPP quad swaps, row mirrors, row swaps); every
// lane gets the same value
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }
__device__ __forceinline__ float wave_max(float x) {   // (operands never NaN)
    x = max2(x, dppf<0xB1>(x));
    x = max2(x, dppf<0x4E>(x));
    x = max2(x, dppf<0x141>(x));
    x = max2(x, dppf<0x140>(x));
    return qg_max(x);
}
// Loads in this kernel are unconditional, from clamped addresses (out-of-range positions
// repeat the last valid one), and the repeats are cancelled arithmetically: they cannot
// change a maximum, and their sum terms are multiplied by 0.  A load under a per-lane
// condition (or a select the compiler turns back into one) makes the compiler wait for
// it on the spot, and the loads would take one round trip each.
//
// M and L of head h over all splits, computed by one whole wave (lane = split mod 64,
// NB blocks of 64 splits): the loads, then the reduction, which also leaves in each lane
// the weights 2^(m_s - M) of its own splits (0 past NS)
template <int NB>
__device__ __forceinline__ void head_ml_load(const float2* ml, int NS, int h_q, int lane, float2* v) {
#pragma unroll
    for (int k = 0; k < NB; ++k) v[k] = ml[(int64_t)imin(lane + 64 * k, NS - 1) * h_q];
}
template <int NB>
__device__ __forceinline__ void head_ml(const float2* v, int NS, int lane, float& M, float& L, float* e) {
    float m = v[0].x;
#pragma unroll
    for (int k = 1; k < NB; ++k) m = max2(m, v[k].x);
    M = wave_max(m);
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        e[k] = __builtin_amdgcn_exp2f(v[k].x - M) * (lane + 64 * k < NS ? 1.f : 0.f);
        l += e[k] * v[k].y;
    }
    L = wave_sum(l);
}

template <int D, int NB>
__global__ void __launch_bounds__(FN_THREADS) k_finish(Geo g, Bufs bf, int layer, float* __restrict__ out,
                                                       const uint16_t* __restrict__ knew,
                                                       const uint16_t* __restrict__ vnew, int score_now) {
    const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t u = unit_of(g, b, layer);
    const int NS = g.n_splits;
    const float2* mlu = bf.part_ml + u * NS * (int64_t)g.h_q;
    // ---- output of head h: each wave owns D/16 float4 columns; its lanes split the splits
    // into 64/(D/16) phases, summed across lanes at the end.  No LDS, no barrier: every
    // wave reduces the split maxima / sums itself, and all loads are issued up front.
    static_assert(D <= FN_THREADS, "one thread per channel of the token");
    constexpr int CW = D / 16, PH = 64 / CW;
    const int h = blockIdx.x;
    const float2* ml = mlu + h;
    const int col = wv * CW + lane % CW, ph = lane / CW;
    const f4_t* pa = reinterpret_cast<const f4_t*>(bf.part_acc + (u * NS * (int64_t)g.h_q + h) * D) + col;
    const int64_t sstride = (int64_t)g.h_q * D / 4;   // float4 per split
    constexpr int NX = 8;            // splits of this lane's phase per batch of loads
    f4_t x[NX];
#pragma unroll
    for (int k = 0; k < NX; ++k) x[k] = pa[imin(ph + k * PH, NS - 1) * sstride];
    // the step's token goes into its sink / recent-window block (one workgroup per KV
    // head: the first query head of the group); its inputs and the block record are read
    // here, ahead of every store, so that all loads share one round trip
    const int G = g.h_q / g.h_kv, hk = h / G;
    const bool tok_wg = h % G == 0;
    UnitHdr* hdr = bf.hdr + u;
    // (read through a lane-varying zero index, so the values stay in vector registers and
    // nothing waits for them before the stores)
    const int z = (int)__builtin_amdgcn_mbcnt_lo(0u, 0u);
    const int* hw = reinterpret_cast<const int*>(hdr) + z;
    const int n_old = hw[offsetof(UnitHdr, pos) / 4];   // n is advanced below by head 0's workgroup
    const int tok_at = hw[offsetof(UnitHdr, tok_at) / 4], page = hw[offsetof(UnitHdr, tok_page) / 4];
    const uint16_t kn = knew[((int64_t)b * g.h_kv + hk) * D + imin(tid, D - 1)];
    const uint16_t vn = vnew[((int64_t)b * g.h_kv + hk) * D + imin(tid, D - 1)];
    float2 mlv[NB];
    head_ml_load<NB>(ml, NS, g.h_q, lane, mlv);
    // keep the scheduler from sinking the loads above to their uses (one round trip each)
    __builtin_amdgcn_sched_barrier(0);
    float M, L, e[NB];
    head_ml<NB>(mlv, NS, lane, M, L, e);
    // the first batch's split weights come from the lanes that own those splits: split
    // ph + k*PH sits in block (k*PH)/64 (PH divides 64), lane (ph + k*PH) mod 64
    float wk[NX];
#pragma unroll
    for (int k = 0; k < NX; ++k) {
        const int blk = (k * PH) / 64;
        wk[k] = blk < NB ? __shfl(e[blk < NB ? blk : 0], (ph + k * PH) & 63) : 0.f;
    }
    f4_t a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NX; ++k) a4 += wk[k] * x[k];
    float mx[NX];
    for (int sp0 = ph + NX * PH; sp0 < NS; sp0 += NX * PH) {      // more splits than one batch
#pragma unroll
        for (int k = 0; k < NX; ++k) {
            const int sp = sp0 + k * PH, sc = imin(sp, NS - 1);
            x[k] = pa[sc * sstride];
            mx[k] = ml[(int64_t)sc * g.h_q].x;
            wk[k] = sp < NS ? 1.f : 0.f;
        }
#pragma unroll
        for (int k = 0; k < NX; ++k) a4 += (__builtin_amdgcn_exp2f(mx[k] - M) * wk[k]) * x[k];
    }
    // sum over the phases: lanes l, l + CW, l + 2 CW, ... (row rotations, then row swaps)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = a4[i];
        if constexpr (CW == 4) v += dppf<0x124>(v);
        v += dppf<0x128>(v);
        a4[i] = qg_sum(v);
    }
    if (ph == 0) reinterpret_cast<f4_t*>(out + ((int64_t)b * g.h_q + h) * D)[col] = a4 / L;
    if (tid == 0) bf.lse_glob[lse_glob_off(g, u, n_old & 1) + h] = M + log2f(L);
    if (tok_wg) {
        // the block the split kernel attended the token in: found only when its sink /
        // recent window was accessible (a window the router did not prepare is an error)
        const bool ok = tok_at == n_old;
        uint16_t* blk = nullptr;
        int Wp = g.W, i = 0;
        if (ok && page == -2) {
            blk = bf.sinks + u * g.sink_elems;
            Wp = sink_width(g.n_sink);
            i = n_old;
        } else if (ok) {
            i = (n_old - g.n_sink) % g.W;
            blk = bf.pages + u * (int64_t)g.n_pages * g.page_elems + (int64_t)page * g.page_elems;
        }
        if (blk && tid < D) {
            uint16_t* kh = blk + (int64_t)(2 * hk) * Wp * D;
            kh[lay_k(i, tid, D, Wp)] = kn;
            kh[(int64_t)Wp * D + lay_v(i, tid, D, Wp)] = vn;
        }
        if (tid == 0) {
            if (!ok) atomicOr(&hdr->status, QEVICT_DEV_E_WINDOW);
            if (h == 0) {
                if (ok) hdr->n = n_old + 1;
                hdr->mass_pending = score_now;
            }
        }
    }
}

hipError_t launch_finish(const Geo& g, const Bufs& bf, int layer, float* out, const uint16_t* k_new,
                         const uint16_t* v_new, int score_now, hipStream_t s) {
    if (g.n_splits > FN_MAXS) return hipErrorInvalidValue;
    const dim3 grid(g.h_q, g.B), block(FN_THREADS);
    // RoPE mode: the key the split kernel turned (layer slice of [L][B][h_kv][d])
    const uint16_t* ks = (g.flags & QEVICT_F_ROPE) ? bf.krot + (int64_t)layer * g.B * g.h_kv * g.d : k_new;
    const int nb = g.n_splits <= 64 ? 1 : g.n_splits <= 128 ? 2 : g.n_splits <= 256 ? 4 : 8;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, s, g, bf, layer, out, ks, v_new, score_now); };
    if (g.d == 128) {
        if (nb == 1) go(k_finish<128, 1>);
        else if (nb == 2) go(k_finish<128, 2>);
        else if (nb == 4) go(k_finish<128, 4>);
        else go(k_finish<128, 8>);
    } else if (g.d == 64) {
        if (nb == 1) go(k_finish<64, 1>);
        else if (nb == 2) go(k_finish<64, 2>);
        else if (nb == 4) go(k_finish<64, 4>);
        else go(k_finish<64, 8>);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------ flush
// Folds a unit's pending window-mass shares into its scores (before an export).
__global__ void __launch_bounds__(256) k_flush_mass(Geo g, Bufs bf, int layer, int b) {
    const int64_t u = unit_of(g, b, layer);
    UnitHdr* hdr = bf.hdr + u;
    if (!hdr->mass_pending) return;
    apply_mass_range(g, bf, u, hdr->n - 1, threadIdx.x, hdr->n_acc, blockDim.x);   // the step at position n - 1
    __syncthreads();
    if (threadIdx.x == 0) hdr->mass_pending = 0;
}

hipError_t launch_flush_mass(const Geo& g, const Bufs& bf, int layer, int b, hipStream_t s) {
    hipLaunchKernelGGL(k_flush_mass, dim3(1), dim3(256), 0, s, g, bf, layer, b);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------ step mass
// Per-head attention mass of the last decode step on the sinks and on every window
// (the a_t(i) of one step summed over a window's tokens, [QEvict] Eq. 1 before the head
// average; Appendix I uses it per head): out[h][0] sinks, out[h][1 + w] window w, zero for
// windows the step did not attend.  From that step's window and row log-sum-exps.
__global__ void __launch_bounds__(256) k_step_mass_clear(Geo g, double* __restrict__ out) {
    const int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (x < (int64_t)g.h_q * (g.n_windows + 1)) out[x] = 0.0;
}

__global__ void __launch_bounds__(256) k_step_mass(Geo g, Bufs bf, int layer, int b, double* __restrict__ out) {
    const int64_t u = unit_of(g, b, layer);
    const UnitHdr* hdr = bf.hdr + u;
    const int cols = g.n_windows + 1;
    const float* lwin = bf.lse_win + lse_win_off(g, u, (hdr->n - 1) & 1);
    const float* lg = bf.lse_glob + lse_glob_off(g, u, (hdr->n - 1) & 1);
    const int x = blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= hdr->n_acc * g.h_q) return;
    const int e = x / g.h_q, h = x % g.h_q;
    const int w = bf.acc[u * g.n_acc_max + e].win;   // -1: the sinks
    out[(int64_t)h * cols + 1 + w] = (double)mass_share(lwin[(int64_t)e * g.h_q + h], lg[h]);
}

hipError_t launch_step_mass(const Geo& g, const Bufs& bf, int layer, int b, double* out, hipStream_t s) {
    const int64_t n_out = (int64_t)g.h_q * (g.n_windows + 1);
    hipLaunchKernelGGL(k_step_mass_clear, dim3((unsigned)((n_out + 255) / 256)), dim3(256), 0, s, g, out);
    const int64_t n_in = (int64_t)g.n_acc_max * g.h_q;
    hipLaunchKernelGGL(k_step_mass, dim3((unsigned)((n_in + 255) / 256)), dim3(256), 0, s, g, bf, layer, b, out);
    return hipGetLastError();
}

}  // namespace qv
