// Decode step: split-K attention over the accessible list (sinks, recent
// windows, Full bf16 windows, Quantized INT2 windows), then a combine pass that
// normalises the splits with the global log-sum-exp and turns per-window
// partial exp-sums into window masses.
//
// Source: "QEvict: Recoverable Quantized KV Eviction for Attention-Drift-Robust
// Long-Context Decoding", §4.1 (accessible-set attention, scale 1/sqrt(d_kv);
// Quantized windows are dequantized in the execution datatype as
// off + scl * code, Eq. 5), §4.2 Eq. 1 (cumulative window score, averaged over
// the H_q query heads).
//
// Work split: one workgroup per (split, KV head, sequence); the G query heads of
// the GQA group share every K/V load.  All contractions run on 16x16 MFMA tiles
// with 16 columns: each query head owns two columns, a "high" and a "low" one,
// so that bf16 operands can carry fp32-accurate values as a sum of two bf16
// parts (query times K scale on the key side, probability times V scale on the
// value side).  With G <= 4 the 16 columns hold two independent column slots,
// so one wave job covers two INT2 windows at once and the softmax arithmetic of
// both runs in the same instructions.
#include <float.h>

#include "qevict_common.h"
#include "qevict_internal.h"

namespace qv {

constexpr int DW = 4;          // waves per workgroup
constexpr int DMAXE = 256;     // accessible entries of one split, staged in LDS per batch
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
// two fp32 -> packed bf16 pair, round to nearest even
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    const f2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2_t));
}
// top 16 bits of two fp32 (bf16 truncation)
__device__ __forceinline__ uint32_t bf16x2_trunc(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
// value of the lane at the mirrored position of this lane's SW-wide column group
// (row_half_mirror for SW = 8, row_mirror for SW = 16): pairs the high column of a
// head with its low column
template <int SW>
__device__ __forceinline__ float mirror(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), SW == 8 ? 0x141 : 0x140, 0xF, 0xF, false));
}
// value of lane (l ^ 8) within its row of 16 (row_ror:8): the other column slot
__device__ __forceinline__ float ror8(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}
// LDS traffic between lanes of one wave: the wave's LDS operations execute in
// order, so only the compiler has to be kept from reordering them
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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
template <int D, int G, int TPC>
struct DecShape {
    static constexpr int CQ = D / 4;                 // channels per lane group (key side)
    static constexpr int KS = D / 32;                // 32-channel MFMA steps (key side)
    static constexpr int MB = D / 16;                // 16-channel blocks (value side)
    static constexpr int NSLOT = G <= 4 ? 2 : 1;     // column slots
    static constexpr int SW = 16 / NSLOT;            // columns per slot
    static constexpr int ROWS = NSLOT * G;           // (item, head) rows of the query-times-scale products
    static constexpr int LPR = 64 / ROWS;            // lanes per product row
    static constexpr int CPL = D / LPR;              // channels per lane in the products
    static constexpr int NV = 4 * TPC;               // scores per lane per INT2 item
    // INT2 job words per lane: K codes and V codes of every item, V offsets / scales of
    // the lane's own item, K scales / offsets of the lane's product channels
    static constexpr int KCW = TPC * CQ / 16, VCW = MB * TPC / 4, VPW = 2 * TPC, KPW = CPL / 2;
    static constexpr int O_VC = NSLOT * KCW, O_VO = O_VC + NSLOT * VCW, O_VS = O_VO + VPW, O_KS = O_VS + VPW,
                         O_KO = O_KS + KPW, QW = O_KO + KPW;
    // bf16 tile job words per lane: K row (CQ bf16) then V (MB blocks x 4 tokens)
    static constexpr int FW = CQ / 2 + 2 * MB;
    static constexpr int RW = QW > FW ? QW : FW;
    static constexpr int QSTR = D + 8;               // bf16 per LDS operand row (padded)
    static_assert(KCW >= 1 && VCW >= 1 && KPW >= 1, "shape");
};

// One unit of wave work.  INT2 job: chunk c of up to NSLOT Quantized windows
// (entries ia, ib), one per column slot.  bf16 job: tile t of one sink / page entry.
struct Job {
    int type;           // 0 none, 1 INT2, 2 bf16
    int ia, ib, c;      // INT2: batch-local entry indices (ib = -1: slot 1 empty), chunk
    int sa, sb;         // INT2: slot ids
    int i, t, kind, idx, ntok, Wn;   // bf16: entry, tile, kind, page id, valid tokens, block width
};

template <int D, int G, int TPC>
__global__ void __launch_bounds__(64 * DW) __attribute__((amdgpu_waves_per_eu(2)))
k_decode_split(Geo g, Bufs bf, int layer, const uint16_t* __restrict__ qin) {
    using S = DecShape<D, G, TPC>;
    constexpr int CQ = S::CQ, KS = S::KS, MB = S::MB, NSLOT = S::NSLOT, SW = S::SW, LPR = S::LPR, CPL = S::CPL;
    constexpr int NV = S::NV, QSTR = S::QSTR;
    __shared__ uint2 lut[256];
    __shared__ AccEntry ent[DMAXE];
    __shared__ __attribute__((aligned(16))) uint16_t qs[DW][16][QSTR];   // per wave: INT2 query operand rows
    __shared__ __attribute__((aligned(16))) uint16_t qb[16][QSTR];       // bf16 query operand rows
    __shared__ float kb[DW][16];                                         // per wave: key-offset bias per column
    __shared__ __attribute__((aligned(16))) float qfl[64][CPL];          // q of each lane's product channels
    __shared__ float s_m[DW][G], s_l[DW][G];
    __shared__ float s_acc[DW][G][D];

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

    const int32_t* splits = bf.splits + u * (g.n_splits + 1);
    const int e_begin = splits[split], e_total = splits[split + 1] - e_begin;
    const int n_tok = bf.hdr[u].n;
    const uint16_t* qhead = qin + ((int64_t)b * g.h_q + hk * G) * D;
    // 4 packed 2-bit codes -> 4 bf16 {0, 1, 2, 3}
    for (int x = threadIdx.x; x < 256; x += 64 * DW) {
        auto bv = [](int c) -> uint32_t { return c == 0 ? 0u : (c == 1 ? 0x3F80u : (c == 2 ? 0x4000u : 0x4040u)); };
        lut[x] = make_uint2(bv(x & 3) | (bv((x >> 2) & 3) << 16), bv((x >> 4) & 3) | (bv((x >> 6) & 3) << 16));
    }
    // bf16 windows: every live column holds its head's query (exact bf16);
    // INT2 windows: each lane's product channels of q, as fp32
    if (wave == 0) {
        uint32_t w[CQ / 2];
        ldw<CQ / 2>(w, qhead + head * D + CQ * qg);
        stw<CQ / 2>(&qb[n][CQ * qg], w);
        uint32_t w2[CPL / 2];
        ldw<CPL / 2>(w2, qhead + phead * D + CPL * pcb);
#pragma unroll
        for (int x = 0; x < CPL / 2; ++x) {
            qfl[lane][2 * x] = bf16lo(w2[x]);
            qfl[lane][2 * x + 1] = bf16hi(w2[x]);
        }
    }

    float m_run = M_INIT, l_run = 0.f, lw = 0.f, vbias = 0.f;
    f4_t acc[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = f4_t{0.f, 0.f, 0.f, 0.f};

    const uint16_t* pages = bf.pages + u * (int64_t)g.n_pages * g.page_elems;
    const uint8_t* slots = bf.slots + u * (int64_t)g.n_slots * g.slot_bytes + (int64_t)hk * g.slot_head_bytes;
    const uint16_t* sinks = bf.sinks + u * g.sink_elems;
    float* lse_out = bf.lse_win + u * (int64_t)g.n_acc_max * g.h_q + hk * G;
    int e0 = e_begin, ne = 0;

    // ---- job sequence of this wave: INT2 windows in pairs (chunk by chunk), then bf16 tiles
    auto rfl = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    auto ent_q = [&](int i) -> int {                 // first INT2 entry at or after i (stride DW)
        for (; i < ne; i += DW)
            if (rfl(ent[i].kind) == EK_SLOT && rfl(ent[i].idx) >= 0) return i;
        return -1;
    };
    auto ent_f = [&](int i) -> Job {                 // first bf16 tile job at or after entry i
        Job j;
        j.type = 0;
        for (; i < ne; i += DW) {
            const int kind = rfl(ent[i].kind), idx = rfl(ent[i].idx), start = rfl(ent[i].start);
            if (kind == EK_SLOT) continue;
            const int nt = kind == EK_SINK ? min(g.n_sink, n_tok) : min(W, n_tok - start);
            if (nt <= 0 || (kind != EK_SINK && idx < 0)) continue;
            j.type = 2;
            j.i = i;
            j.t = 0;
            j.kind = kind;
            j.idx = idx;
            j.ntok = nt;
            j.Wn = kind == EK_SINK ? Ws : W;
            return j;
        }
        return j;
    };
    auto make_q = [&](int i) -> Job {
        Job j;
        j.type = 1;
        j.ia = i;
        j.c = 0;
        j.sa = rfl(ent[i].idx);
        j.ib = NSLOT == 2 ? ent_q(i + DW) : -1;
        j.sb = j.ib >= 0 ? rfl(ent[j.ib].idx) : j.sa;
        return j;
    };
    auto first_q = [&]() -> Job {
        const int i = ent_q(wave);
        if (i >= 0) return make_q(i);
        Job j;
        j.type = 0;
        j.ia = j.ib = -1;
        j.c = 0;
        j.sa = j.sb = 0;
        return j;
    };
    auto next_q = [&](Job j) -> Job {
        if (j.c + 1 < NCH) {
            j.c += 1;
            return j;
        }
        const int i = (NSLOT == 2 && j.ib < 0) ? -1 : ent_q((NSLOT == 2 ? j.ib : j.ia) + DW);
        if (i >= 0) return make_q(i);
        j.type = 0;
        j.c = 0;
        return j;   // keeps valid slot ids: the tail prefetch reads them harmlessly
    };
    auto next_f = [&](Job j) -> Job {
        if (16 * (j.t + 1) < j.ntok) {
            j.t += 1;
            return j;
        }
        const Job k = ent_f(j.i + DW);
        if (k.type != 0) return k;
        j.type = 0;
        return j;   // keeps a valid block: the tail prefetch reads it harmlessly
    };

    struct Raw {
        uint32_t w[S::RW];
    };
    auto load_q = [&](const Job& j, Raw& R) __attribute__((always_inline)) {
        {
            const uint8_t* sa = slots + (int64_t)j.sa * g.slot_bytes;
            const uint8_t* sb = slots + (int64_t)j.sb * g.slot_bytes;
            const int kco = ((j.c * 16 + n) * 4 + qg) * TPC * (CQ / 4);        // K codes: token row n, channel group qg
            const int vco = W * D / 4 + (((n * 4 + qg) * NCH + j.c) * MB) * TPC;   // V codes: channel row n, tokens of qg
            ldw<S::KCW>(R.w, sa + kco);
            ldw<S::VCW>(R.w + S::O_VC, sa + vco);
            if constexpr (NSLOT == 2) {
                ldw<S::KCW>(R.w + S::KCW, sb + kco);
                ldw<S::VCW>(R.w + S::O_VC + S::VCW, sb + vco);
            }
            const uint8_t* so = slot == 0 ? sa : sb;                 // the lane's own item
            const uint16_t* offV = reinterpret_cast<const uint16_t*>(so + W * D / 2) + 2 * D;
            ldw<S::VPW>(R.w + S::O_VO, offV + (qg * NT + TPC * j.c) * 4);
            ldw<S::VPW>(R.w + S::O_VS, offV + W + (qg * NT + TPC * j.c) * 4);
            const uint8_t* sp = pitem == 0 ? sa : sb;                // the item of the lane's products
            const uint16_t* offK = reinterpret_cast<const uint16_t*>(sp + W * D / 2);
            ldw<S::KPW>(R.w + S::O_KS, offK + D + CPL * pcb);
            ldw<S::KPW>(R.w + S::O_KO, offK + CPL * pcb);
        }
    };
    auto load_f = [&](const Job& j, Raw& R) __attribute__((always_inline)) {
        {
            const int tpc = lay_tpc(j.Wn), nt16 = j.Wn / 16;
            const uint16_t* kbase = (j.kind == EK_SINK ? sinks : pages + (int64_t)j.idx * g.page_elems) +
                                    (int64_t)(2 * hk) * j.Wn * D;
            const uint16_t* vbase = kbase + (int64_t)j.Wn * D;
            ldw<CQ / 2>(R.w, kbase + ((((j.t / tpc) * 16 + n) * 4 + qg) * tpc + j.t % tpc) * CQ);
            ldw<2 * MB>(R.w + CQ / 2, vbase + (((n * 4 + qg) * nt16 + j.t) * MB) * 4);
        }
    };

    // online softmax over the lane's NVV scores (per column: max over the 4 lane groups)
    auto softmax = [&](float* s, float* p, int nvv) __attribute__((always_inline)) {
        float mx = s[0];
        for (int v = 1; v < nvv; ++v) mx = fmaxf(mx, s[v]);
        mx = fmaxf(mx, xor_lane<16>(mx));
        mx = fmaxf(mx, xor_lane<32>(mx));
        const float mnew = fmaxf(m_run, mx);
        if (__any(mnew > m_run)) {
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
    auto lut4 = [&](uint32_t w, int byte) -> u2_t {
        const uint2 a = lut[(w >> (8 * byte)) & 0xffu];
        return u2_t{a.x, a.y};
    };
    auto lse_store = [&](bool mine, int ie) {
        float t = lw;
        t += xor_lane<16>(t);
        t += xor_lane<32>(t);
        if (mine) {
            if (qg == 0 && hi) lse_out[(int64_t)(e0 + ie) * g.h_q + head] = m_run + log2f(t);
            lw = 0.f;
        }
    };

    auto process_q = [&](const Job& j, const Raw& R) __attribute__((always_inline)) {
        // (1) q * sclK for every (item, head, channel) once, split into bf16 high + low
        //     rows of the wave's operand block; key-offset bias sum_c q_c offK_c per row
        {
            float bias = 0.f;
            uint32_t hw[CPL / 2], lw2[CPL / 2];
            float qf[CPL];
#pragma unroll
            for (int x = 0; x < CPL; x += 4) *reinterpret_cast<f4_t*>(&qf[x]) = *reinterpret_cast<const f4_t*>(&qfl[lane][x]);
#pragma unroll
            for (int x = 0; x < CPL / 2; ++x) {
                const f2_t s2 = h2f(R.w[S::O_KS + x]), o2 = h2f(R.w[S::O_KO + x]);
                const float x0 = qf[2 * x] * s2.x, x1 = qf[2 * x + 1] * s2.y;
                bias = fmaf(qf[2 * x], o2.x, bias);
                bias = fmaf(qf[2 * x + 1], o2.y, bias);
                hw[x] = bf16x2_trunc(x0, x1);
                lw2[x] = bf16x2_rne(x0 - bf16lo(hw[x]), x1 - bf16hi(hw[x]));
            }
            bias = lanes_sum<1, LPR>(bias);
            wave_lds_fence();
            stw<CPL / 2>(&qs[wave][pitem * SW + phead][CPL * pcb], hw);
            stw<CPL / 2>(&qs[wave][pitem * SW + SW - 1 - phead][CPL * pcb], lw2);
            if (pcb == 0) {
                kb[wave][pitem * SW + phead] = bias;
                kb[wave][pitem * SW + SW - 1 - phead] = bias;
            }
            wave_lds_fence();
        }
        // (2) the lane's column of the operand
        u4_t bq[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bq[ks] = *reinterpret_cast<const u4_t*>(&qs[wave][n][CQ * qg + 8 * ks]);
        const float kbs = kb[wave][n] * scale;
        // (3) scores S^T[token][column] = codes . (q * sclK)
        float s[NV];
#pragma unroll
        for (int tc = 0; tc < TPC; ++tc) {
            f4_t da = {0.f, 0.f, 0.f, 0.f}, db = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int by = tc * (CQ / 4) + 2 * ks;
                const uint32_t wa = R.w[by >> 2];
                const u2_t a0 = lut4(wa, by & 3), a1 = lut4(wa, (by & 3) + 1);
                da = mfma32(u4_t{a0.x, a0.y, a1.x, a1.y}, bq[ks], da);
                if constexpr (NSLOT == 2) {
                    const uint32_t wb = R.w[S::KCW + (by >> 2)];
                    const u2_t b0 = lut4(wb, by & 3), b1 = lut4(wb, (by & 3) + 1);
                    db = mfma32(u4_t{b0.x, b0.y, b1.x, b1.y}, bq[ks], db);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = (NSLOT == 2 && slot) ? db[i] : da[i];
                v += mirror<SW>(v);                            // high + low query parts
                s[4 * tc + i] = fmaf(v, scale, kbs);
            }
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
            const f2_t o2 = h2f(R.w[S::O_VO + x]), c2 = h2f(R.w[S::O_VS + x]);
            vbias = fmaf(p[2 * x], o2.x, vbias);
            vbias = fmaf(p[2 * x + 1], o2.y, vbias);
            P[x] = hilo(p[2 * x] * c2.x, p[2 * x + 1] * c2.y);
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
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            u4_t a;
            if constexpr (TPC == 2) {
                const int by = 2 * m;
                const uint32_t w = R.w[S::O_VC + (by >> 2)];
                const u2_t a0 = lut4(w, by & 3), a1 = lut4(w, (by & 3) + 1);
                a = u4_t{a0.x, a0.y, a1.x, a1.y};
            } else {
                const u2_t a0 = lut4(R.w[S::O_VC + (m >> 2)], m & 3);
                a = u4_t{a0.x, a0.y, 0u, 0u};
            }
            acc[m] = mfma32(a, pa, acc[m]);
        }
        if (NSLOT == 2 && j.ib >= 0) {
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                u4_t a;
                if constexpr (TPC == 2) {
                    const int by = 2 * m;
                    const uint32_t w = R.w[S::O_VC + S::VCW + (by >> 2)];
                    const u2_t a0 = lut4(w, by & 3), a1 = lut4(w, (by & 3) + 1);
                    a = u4_t{a0.x, a0.y, a1.x, a1.y};
                } else {
                    const u2_t a0 = lut4(R.w[S::O_VC + S::VCW + (m >> 2)], m & 3);
                    a = u4_t{a0.x, a0.y, 0u, 0u};
                }
                acc[m] = mfma32(a, pb, acc[m]);
            }
        }
        // (6) both windows end on their last chunk: log-sum-exp of their mass per head
        if (j.c + 1 == NCH) lse_store(slot == 0 || j.ib >= 0, slot == 0 ? j.ia : j.ib);
    };

    auto process_f = [&](const Job& j, const Raw& R) __attribute__((always_inline)) {
        u4_t bq[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bq[ks] = *reinterpret_cast<const u4_t*>(&qb[n][CQ * qg + 8 * ks]);
        f4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            d = mfma32(u4_t{R.w[4 * ks], R.w[4 * ks + 1], R.w[4 * ks + 2], R.w[4 * ks + 3]}, bq[ks], d);
        float s[4], p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = slot == 0 && 16 * j.t + 4 * qg + i < j.ntok;
            s[i] = valid ? d[i] * scale : -INFINITY;
        }
        softmax(s, p, 4);
        const u2_t P = {hilo(p[0], p[1]), hilo(p[2], p[3])};
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[m] = mfma16(u2_t{R.w[CQ / 2 + 2 * m], R.w[CQ / 2 + 2 * m + 1]}, P, acc[m]);
        if (16 * (j.t + 1) >= j.ntok) lse_store(slot == 0, j.i);
    };

    // entries are staged in LDS in batches; each wave runs two passes (INT2 pairs,
    // then bf16 tiles), each a two-deep software pipeline in which the next job's
    // loads are in flight while a job is processed
    for (int bs = 0; bs < e_total; bs += DMAXE) {
        __syncthreads();
        e0 = e_begin + bs;
        ne = min(DMAXE, e_total - bs);
        for (int x = threadIdx.x; x < ne; x += 64 * DW) ent[x] = bf.acc[u * g.n_acc_max + e0 + x];
        __syncthreads();
        {   // unrolled by two so that the two buffers swap roles without copies
            Raw ra, rb;
            Job j = first_q();
            load_q(j, ra);
            while (j.type != 0) {
                Job jn = next_q(j);
                load_q(jn, rb);
                process_q(j, ra);
                j = jn;
                if (j.type == 0) break;
                jn = next_q(j);
                load_q(jn, ra);
                process_q(j, rb);
                j = jn;
            }
        }
        {
            Raw ra, rb;
            Job j = ent_f(wave);
            if (j.type == 0) {
                j.kind = EK_SINK;
                j.idx = 0;
                j.t = 0;
                j.Wn = Ws;
                j.ntok = 0;
                j.i = 0;
            }
            load_f(j, ra);
            while (j.type != 0) {
                Job jn = next_f(j);
                load_f(jn, rb);
                process_f(j, ra);
                j = jn;
                if (j.type == 0) break;
                jn = next_f(j);
                load_f(jn, ra);
                process_f(j, rb);
                j = jn;
            }
        }
    }

    // ---- wave state -> workgroup partial for this split
    float lt = l_run;
    lt += xor_lane<16>(lt);
    lt += xor_lane<32>(lt);
    float vb = vbias;
    vb += xor_lane<16>(vb);
    vb += xor_lane<32>(vb);
    float a[MB][4];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) a[m][i] = acc[m][i] + mirror<SW>(acc[m][i]) + vb;   // high + low columns
    float mw = m_run;
    if constexpr (NSLOT == 2) {
        const float m1 = ror8(m_run), l1 = ror8(lt);
        const float M = fmaxf(m_run, m1);
        const float f0 = exp2f(m_run - M), f1 = exp2f(m1 - M);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) a[m][i] = f0 * a[m][i] + f1 * ror8(a[m][i]);
        lt = f0 * lt + f1 * l1;
        mw = M;
    }
    if (slot == 0 && hi) {
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_acc[wave][rn][16 * m + 4 * qg + i] = a[m][i];
        if (qg == 0) {
            s_m[wave][rn] = mw;
            s_l[wave][rn] = lt;
        }
    }
    __syncthreads();
    float* pacc = bf.part_acc + ((u * g.n_splits + split) * (int64_t)g.h_q + hk * G) * D;
    float2* pml = bf.part_ml + (u * g.n_splits + split) * (int64_t)g.h_q + hk * G;
    for (int x = threadIdx.x; x < G * D; x += 64 * DW) {
        const int gg = x / D, c = x % D;
        float M = s_m[0][gg];
#pragma unroll
        for (int w = 1; w < DW; ++w) M = fmaxf(M, s_m[w][gg]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < DW; ++w) {
            const float f = exp2f(s_m[w][gg] - M);
            L += f * s_l[w][gg];
            A += f * s_acc[w][gg][c];
        }
        pacc[(int64_t)gg * D + c] = A;
        if (c == 0) pml[gg] = make_float2(M, L);
    }
}

hipError_t launch_decode(const Geo& g, const Bufs& bf, int layer, const uint16_t* q, hipStream_t s) {
    const dim3 grid(g.n_splits, g.h_kv, g.B), block(64 * DW);
    const int G = g.h_q / g.h_kv, TPC = lay_tpc(g.W);
#define QV_DEC(D_, G_, T_)                                                                     \
    if (g.d == D_ && G == G_ && TPC == T_) {                                                   \
        hipLaunchKernelGGL((k_decode_split<D_, G_, T_>), grid, block, 0, s, g, bf, layer, q); \
        return hipGetLastError();                                                              \
    }
    QV_DEC(128, 1, 2) QV_DEC(128, 2, 2) QV_DEC(128, 4, 2) QV_DEC(128, 8, 2)
    QV_DEC(64, 1, 2) QV_DEC(64, 2, 2) QV_DEC(64, 4, 2) QV_DEC(64, 8, 2)
    QV_DEC(128, 1, 1) QV_DEC(128, 2, 1) QV_DEC(128, 4, 1) QV_DEC(128, 8, 1)
    QV_DEC(64, 1, 1) QV_DEC(64, 2, 1) QV_DEC(64, 4, 1) QV_DEC(64, 8, 1)
#undef QV_DEC
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------ combine
// o_h = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s ; LSE_h = M + log2 L (log2 domain)
constexpr int CB_THREADS = 256;
constexpr int CB_MAXS = 1024;

__global__ void __launch_bounds__(CB_THREADS) k_combine(Geo g, Bufs bf, int layer, float* __restrict__ out) {
    __shared__ float wsp[CB_MAXS];
    __shared__ float red[CB_THREADS];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int64_t u = unit_of(g, b, layer);
    const int NS = g.n_splits;
    const float2* pml = bf.part_ml + u * NS * (int64_t)g.h_q + h;
    const float* pacc = bf.part_acc + (u * NS * (int64_t)g.h_q + h) * g.d;   // + channel below
    float M = -INFINITY;
    for (int s = tid; s < NS; s += CB_THREADS) M = fmaxf(M, pml[(int64_t)s * g.h_q].x);
    red[tid] = M;
    __syncthreads();
    for (int o = CB_THREADS / 2; o > 0; o >>= 1) {
        if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
        __syncthreads();
    }
    M = red[0];
    __syncthreads();
    float L = 0.f;
    for (int s = tid; s < NS; s += CB_THREADS) {
        const float2 ml = pml[(int64_t)s * g.h_q];
        const float f = ml.x > -INFINITY ? exp2f(ml.x - M) : 0.f;
        wsp[s] = f;
        L += f * ml.y;
    }
    red[tid] = L;
    __syncthreads();
    for (int o = CB_THREADS / 2; o > 0; o >>= 1) {
        if (tid < o) red[tid] += red[tid + o];
        __syncthreads();
    }
    L = red[0];
    __syncthreads();
    const int parts = CB_THREADS / g.d, c = tid % g.d, part = tid / g.d;
    pacc += c;
    float A = 0.f;
    if (part < parts) {
        int s = part;
        for (; s + 3 * parts < NS; s += 4 * parts) {
            const float a0 = pacc[(int64_t)s * g.h_q * g.d], a1 = pacc[(int64_t)(s + parts) * g.h_q * g.d];
            const float a2 = pacc[(int64_t)(s + 2 * parts) * g.h_q * g.d];
            const float a3 = pacc[(int64_t)(s + 3 * parts) * g.h_q * g.d];
            A += wsp[s] * a0 + wsp[s + parts] * a1 + wsp[s + 2 * parts] * a2 + wsp[s + 3 * parts] * a3;
        }
        for (; s < NS; s += parts) A += wsp[s] * pacc[(int64_t)s * g.h_q * g.d];
    }
    red[tid] = A;
    __syncthreads();
    if (tid < g.d) {
        float t = 0.f;
        for (int pp = 0; pp < parts; ++pp) t += red[pp * g.d + tid];
        out[((int64_t)b * g.h_q + h) * g.d + tid] = t / L;
    }
    if (tid == 0) bf.lse_glob[u * g.h_q + h] = M + log2f(L);
}

hipError_t launch_combine(const Geo& g, const Bufs& bf, int layer, float* out, hipStream_t s) {
    hipLaunchKernelGGL(k_combine, dim3(g.h_q, g.B), dim3(CB_THREADS), 0, s, g, bf, layer, out);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------ window mass
// u(w) = (1/H_q) sum_h 2^(lse_w,h - LSE_h) = (1/H_q) sum_h sum_{i in w} a_h(i);  S_bar(w) += u(w)
// One wave per accessible entry, lanes over query heads.
__global__ void __launch_bounds__(256) k_mass(Geo g, Bufs bf, int layer) {
    const int b = blockIdx.y;
    const int64_t u = unit_of(g, b, layer);
    const UnitHdr* hdr = bf.hdr + u;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (e == 0 || e >= hdr->n_acc) return;
    if (g.flags & QEVICT_F_SCORE_ROUTE_ONLY) {
        const int j = hdr->n - hdr->prompt_len - 1;   // index of the decode step just taken
        if ((j + 1) % g.omega != 0) return;
    }
    const AccEntry en = bf.acc[u * g.n_acc_max + e];
    if (en.start >= hdr->n) return;
    double s = 0.0;
    if (lane < g.h_q) s = (double)exp2f(bf.lse_win[(u * g.n_acc_max + e) * (int64_t)g.h_q + lane] -
                                        bf.lse_glob[u * g.h_q + lane]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0) bf.score[u * g.n_windows + en.win] += s / g.h_q;
}

hipError_t launch_mass(const Geo& g, const Bufs& bf, int layer, hipStream_t s) {
    const int nb = (g.n_acc_max + 3) / 4;
    hipLaunchKernelGGL(k_mass, dim3(nb, g.B), dim3(256), 0, s, g, bf, layer);
    return hipGetLastError();
}

}  // namespace qv
