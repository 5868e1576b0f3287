// Decode step: split-K attention over the chronological accessible list
// (sinks, recent windows, Full bf16 windows, Quantized INT2 windows dequantized
// in registers), then a combine pass that normalises the splits with the global
// log-sum-exp and turns per-window partial exp-sums into window masses.
//
// Source: "QEvict: Recoverable Quantized KV Eviction for Attention-Drift-Robust
// Long-Context Decoding", §4.1 (accessible-set attention, scale 1/sqrt(d_kv)),
// §4.2 Eq. 1 (cumulative window score, averaged over the H_q query heads).
//
// Work split: one workgroup per (split, KV head, sequence); the G query heads of
// the GQA group share every K/V load.  Inside a wave, a token is handled by LPT
// lanes that each own CPL contiguous channels; TPI = 64 / LPT tokens are in
// flight per wave iteration.  Each wave walks whole windows of the split, so it
// can emit the window's log-sum-exp (log2 domain) without extra passes.
#include <float.h>

#include <type_traits>

#include "qevict_common.h"
#include "qevict_internal.h"

namespace qv {

constexpr int DW = 4;          // waves per workgroup
constexpr int DMAXE = 512;     // accessible entries of one split, staged in LDS

typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f4_t mfma16(s4_t a, s4_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
// both fp16 halves of a 32-bit word as fp32 (the word stays a 32-bit value in the IR)
__device__ __forceinline__ f2_t h2f(uint32_t w) { return __builtin_convertvector(__builtin_bit_cast(h2_t, w), f2_t); }
__device__ __forceinline__ s4_t s4_of(uint32_t lo, uint32_t hi) {
    const u2_t v = {lo, hi};
    return __builtin_bit_cast(s4_t, v);
}
// two fp32 -> packed bf16 pair, round to nearest even
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    const f2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2_t));
}
// top 16 bits of two fp32 (bf16 truncation, exact when the values are bf16)
__device__ __forceinline__ uint32_t bf16x2_trunc(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// One unit of work for a wave: up to 32 tokens (one or two 16-token tiles) of one
// accessible-list entry.  All fields are wave-uniform.
struct Job {
    int i;      // entry index within the split (-1: none)
    int ch;     // chunk of the entry
    int nch;    // chunks of the entry
    int kind;   // EK_SINK / EK_PAGE / EK_SLOT
    int ntok;   // valid tokens of the entry
    int Wn;     // tokens per page of the entry (W, or the sink width)
    int idx;    // page / slot id
};

template <int D>
struct Raw {                       // per-lane operands of one job, as loaded from HBM (pairs of 32-bit words)
    // bf16 job (one tile): k = the lane's K row slice (CQ channels), v = its V^T slice (4 tokens x MB blocks).
    // INT2 job (up to two tiles): words k[0..3] K codes, k[4..7] V codes, k[8..11] V offsets,
    //           k[12..15] V scales; v[0..CQ/2) K scales, v[CQ/2..3CQ/4) K offsets (first chunk only).
    u2_t k[8];
    u2_t v[3 * D / 32];
};

template <int N>
__device__ __forceinline__ void ld4(u2_t* dst, const void* src) {
    const uint4* p = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int x = 0; x < N; ++x) {
        const uint4 t = p[x];
        dst[2 * x] = u2_t{t.x, t.y};
        dst[2 * x + 1] = u2_t{t.z, t.w};
    }
}
__device__ __forceinline__ void ld2(u2_t* dst, const void* src) {
    const uint2 t = *reinterpret_cast<const uint2*>(src);
    dst[0] = u2_t{t.x, t.y};
}
__device__ __forceinline__ uint32_t word(const u2_t* a, int w) { return a[w >> 1][w & 1]; }
__device__ __forceinline__ s4_t pair_s4(u2_t v) { return __builtin_bit_cast(s4_t, v); }

template <int D, int G>
__global__ void __launch_bounds__(64 * DW) __attribute__((amdgpu_waves_per_eu(2))) k_decode_split(Geo g, Bufs bf, int layer, const uint16_t* __restrict__ qin) {
    constexpr int CQ = D / 4;      // channels of one lane group on the K side
    constexpr int KK = D / 16;     // MFMA k-steps over channels
    constexpr int MB = D / 16;     // 16-channel blocks on the V side
    constexpr int NKR = D / 16;    // uint4 of K per lane per 2-tile chunk (bf16)
    static_assert(2 * G <= 16, "hi/lo query columns must fit one 16-wide tile");
    __shared__ uint2 lut[256];
    __shared__ AccEntry ent[DMAXE];
    __shared__ float s_m[DW][16], s_l[DW][16];
    __shared__ float s_acc[DW][G][D];

    const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int64_t u = unit_of(g, b, layer);
    const int n = bf.hdr[u].n;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int r = lane & 15, qg = lane >> 4;
    const int W = g.W, Ws = sink_width(g.n_sink);

    // 4 packed 2-bit codes -> 4 bf16 {0, 1, 2, 3}
    for (int x = threadIdx.x; x < 256; x += 64 * DW) {
        const uint32_t v0 = 0, v1 = 0x3F80, v2 = 0x4000, v3 = 0x4040;
        auto bv = [&](int c) { return c == 0 ? v0 : (c == 1 ? v1 : (c == 2 ? v2 : v3)); };
        lut[x] = make_uint2(bv(x & 3) | (bv((x >> 2) & 3) << 16), bv((x >> 4) & 3) | (bv((x >> 6) & 3) << 16));
    }
    const int32_t* splits = bf.splits + u * (g.n_splits + 1);
    const int e_begin = splits[split], e_total = splits[split + 1] - e_begin;
    int e0 = e_begin, ne = 0;   // current batch of entries staged in LDS
    __syncthreads();

    // B operand for bf16 windows: columns r and r + G (r < G) both hold query head r
    // (exact bf16), others zero; the two copies later carry the high and low bf16
    // parts of the probabilities on the value side
    u2_t qB[KK];                  // 4 bf16 per k-step
    ld4<KK / 2>(qB, qin + ((int64_t)b * g.h_q + hk * G + r % G) * D + qg * CQ);
    if (r >= 2 * G) {
#pragma unroll
        for (int x = 0; x < KK; ++x) qB[x] = u2_t{0u, 0u};
    }
    const float scale = 1.4426950408889634f / sqrtf((float)D);   // log2(e) / sqrt(d)
    // columns of the INT2 query operand: r < G: high part of q*scl for head r;
    // G <= r < 2G: low part for head r - G; others zero
    const uint32_t lo_mask = (r >= G && r < 2 * G) ? 0xFFFF0000u : 0u;
    const bool live = r < 2 * G;       // lanes holding a query column (two copies per head)
    const bool prim = r < G;           // the copy that owns the head's softmax statistics

    float m_run = -INFINITY, l_run = 0.f, lw = 0.f, vbias = 0.f;
    f4_t acc[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = f4_t{0.f, 0.f, 0.f, 0.f};
    u2_t qpB[KK];
    float kbias = 0.f;

    const uint16_t* pages = bf.pages + u * (int64_t)g.n_pages * g.page_elems;
    const uint8_t* slots = bf.slots + u * (int64_t)g.n_slots * g.slot_bytes;
    const uint16_t* sinks = bf.sinks + u * g.sink_elems;
    float* lse_out = bf.lse_win + u * (int64_t)g.n_acc_max * g.h_q;

    auto resolve = [&](int i) __attribute__((always_inline)) -> Job {
        Job j;
        j.ch = 0;
        for (; i < ne; i += DW) {
            AccEntry en = ent[i];
            en.kind = __builtin_amdgcn_readfirstlane(en.kind);
            en.idx = __builtin_amdgcn_readfirstlane(en.idx);
            en.start = __builtin_amdgcn_readfirstlane(en.start);
            int nt;
            if (en.kind == EK_SINK) nt = min(g.n_sink, n);
            else nt = min(W, n - en.start);
            if (nt <= 0 || (en.kind != EK_SINK && en.idx < 0)) continue;
            j.i = i;
            j.kind = en.kind;
            j.ntok = nt;
            j.Wn = en.kind == EK_SINK ? Ws : W;
            j.idx = en.idx;
            j.nch = en.kind == EK_SLOT ? (nt + 31) / 32 : (nt + 15) / 16;   // INT2: 32-token jobs, bf16: 16
            return j;
        }
        j.i = -1;
        j.kind = EK_PAGE;
        j.ntok = 0;
        j.Wn = W;
        j.idx = 0;
        j.nch = 0;
        return j;
    };
    auto next = [&](Job j) __attribute__((always_inline)) -> Job {
        if (j.i < 0) return j;
        if (j.ch + 1 < j.nch) {
            j.ch += 1;
            return j;
        }
        return resolve(j.i + DW);
    };

    auto load = [&](const Job& j, Raw<D>& R) __attribute__((always_inline)) {
        if (j.i < 0) return;
        const int tpc = lay_tpc(j.Wn), NT = j.Wn / 16;
        if (j.kind != EK_SLOT) {
            const uint16_t* kb = (j.kind == EK_SINK ? sinks : pages + (int64_t)j.idx * g.page_elems) +
                                 (int64_t)(2 * hk) * j.Wn * D;
            const uint16_t* vb = kb + (int64_t)j.Wn * D;
            const int tile = j.ch;                                  // one 16-token tile per bf16 job
            const uint16_t* pk = kb + ((((tile / tpc) * 16 + r) * 4 + qg) * tpc + tile % tpc) * CQ;
            const uint16_t* pv = vb + (((r * 4 + qg) * NT + tile) * MB) * 4;
            ld4<CQ / 8>(R.k, pk);
            ld4<MB / 2>(R.v, pv);
        } else {
            const uint8_t* sl = slots + (int64_t)j.idx * g.slot_bytes + (int64_t)hk * g.slot_head_bytes;
            const uint8_t* kc = sl + (((j.ch * 16 + r) * 4 + qg) * tpc) * (CQ / 4);
            const uint8_t* vc = sl + W * D / 4 + ((r * 4 + qg) * NT + 2 * j.ch) * MB;
            const uint16_t* oK = reinterpret_cast<const uint16_t*>(sl + W * D / 2);
            const uint16_t* oV = oK + 2 * D;
            const int vpo = (qg * NT + 2 * j.ch) * 4;
            // K codes: tpc*CQ/4 bytes, V codes: tpc*MB bytes, V offsets / scales: tpc*4 halves each
            if (tpc == 2) {
                if constexpr (D == 128) {
                    ld4<1>(R.k, kc);
                    ld4<1>(R.k + 2, vc);
                } else {
                    ld2(R.k, kc);
                    ld2(R.k + 2, vc);
                }
                ld4<1>(R.k + 4, oV + vpo);
                ld4<1>(R.k + 6, oV + W + vpo);
            } else {
                if constexpr (D == 128) {
                    ld2(R.k, kc);
                    ld2(R.k + 2, vc);
                } else {
                    R.k[0] = u2_t{*reinterpret_cast<const uint32_t*>(kc), 0u};
                    R.k[2] = u2_t{*reinterpret_cast<const uint32_t*>(vc), 0u};
                }
                ld2(R.k + 4, oV + vpo);
                ld2(R.k + 6, oV + W + vpo);
            }
            if (j.ch == 0) {
                // K scales of the lane's CQ channels (q * scl for its query column) and
                // K offsets of half of them (bias)
                const int half = (r >= G && r < 2 * G) ? 1 : 0;
                ld4<CQ / 8>(R.v, oK + D + qg * CQ);
                ld4<CQ / 16>(R.v + CQ / 4, oK + qg * CQ + half * (CQ / 2));
            }
        }
    };

    auto process = [&](const Job& j, const Raw<D>& R) __attribute__((always_inline)) {
        const bool quant = j.kind == EK_SLOT;
        const int tiles = quant ? lay_tpc(j.Wn) : 1;
        const int base_t = (quant ? 32 : 16) * j.ch;
        const int nt_here = min(j.ntok - base_t, 16 * tiles);   // valid tokens in this job
        const int ntiles = (nt_here + 15) / 16;
        if (quant && j.ch == 0) {
            // query operand q * scl split into bf16 high + low parts (exact high, truncated low),
            // and the window's key-offset bias sum_c q_c * off_c (per head, log2 domain later)
            const u2_t* scl = R.v;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                uint32_t w2[2];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int cc = 4 * kk + 2 * h2;             // channel pair within the lane group
                    const f2_t sp = h2f(word(scl, cc / 2));
                    const uint32_t qw = word(qB, cc / 2);         // query channels cc, cc + 1 (bf16)
                    const float x0 = bf16lo(qw) * sp.x;
                    const float x1 = bf16hi(qw) * sp.y;
                    const float y0 = x0 - __uint_as_float(__float_as_uint(x0) & lo_mask);
                    const float y1 = x1 - __uint_as_float(__float_as_uint(x1) & lo_mask);
                    w2[h2] = bf16x2_trunc(y0, y1);
                }
                qpB[kk] = u2_t{w2[0], w2[1]};
            }
            const u2_t* off = R.v + CQ / 4;
            const int half = (r >= G && r < 2 * G) ? 1 : 0;
            float sb = 0.f;
#pragma unroll
            for (int x = 0; x < CQ / 4; ++x) {
                const f2_t op = h2f(word(off, x));
                const uint32_t qw = word(qB, half * (CQ / 4) + x);
                sb = fmaf(bf16lo(qw), op.x, sb);
                sb = fmaf(bf16hi(qw), op.y, sb);
            }
            sb += xor_lane<G>(sb);                 // high-part lane + low-part lane
            sb += xor_lane<16>(sb);
            sb += xor_lane<32>(sb);
            kbias = sb;
        }
        // ---- scores of the chunk: S^T[token][column] = K_tile . Q^T
        float s[2][4];
        auto score_tile = [&](auto TCc) __attribute__((always_inline)) {
            constexpr int tc = decltype(TCc)::value;
            f4_t c = {0.f, 0.f, 0.f, 0.f};
            if (!quant) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    c = mfma16(pair_s4(R.k[tc * (CQ / 4) + kk]), pair_s4(qB[kk]), c);
            } else {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    constexpr int dummy = 0;
                    (void)dummy;
                    const int byte = tc * (CQ / 4) + kk;
                    const uint32_t code = (word(R.k, byte >> 2) >> (8 * (byte & 3))) & 0xffu;
                    const uint2 a = lut[code];
                    c = mfma16(s4_of(a.x, a.y), pair_s4(qpB[kk]), c);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = c[i];
                if (quant) v = v + xor_lane<G>(v) + kbias;
                const bool valid = tc * 16 + 4 * qg + i < nt_here;
                s[tc][i] = valid ? v * scale : -INFINITY;
            }
        };
        score_tile(std::integral_constant<int, 0>{});
        if (ntiles > 1) {
            score_tile(std::integral_constant<int, 1>{});
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) s[1][i] = -INFINITY;
        }
        // ---- online softmax per query column (lanes r < G)
        float mx = -INFINITY;
#pragma unroll
        for (int tc = 0; tc < 2; ++tc)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[tc][i]);
        mx = fmaxf(mx, xor_lane<16>(mx));
        mx = fmaxf(mx, xor_lane<32>(mx));
        if (!live) mx = 0.f;
        const float mnew = fmaxf(m_run, mx);
        if (__any(mnew > m_run)) {
            const float alpha = exp2f(m_run - mnew);
            l_run *= alpha;
            lw *= alpha;
            vbias *= alpha;
#pragma unroll
            for (int m = 0; m < MB; ++m) acc[m] *= alpha;
            m_run = mnew;
        }
        float p[2][4];
        float ps = 0.f;
#pragma unroll
        for (int tc = 0; tc < 2; ++tc)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[tc][i] = live ? exp2f(s[tc][i] - m_run) : 0.f;
                ps += p[tc][i];
            }
        l_run += ps;
        lw += ps;
        // ---- O^T[channel][column] += V^T_tile . P
        auto value_tile = [&](auto TCc) __attribute__((always_inline)) {
            constexpr int tc = decltype(TCc)::value;
            float pv[4];
            if (!quant) {
#pragma unroll
                for (int i = 0; i < 4; ++i) pv[i] = p[tc][i];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f2_t o2 = h2f(word(R.k, 8 + 2 * tc + (i >> 1))), s2 = h2f(word(R.k, 12 + 2 * tc + (i >> 1)));
                    const float o = (i & 1) ? o2.y : o2.x;
                    const float sc = (i & 1) ? s2.y : s2.x;
                    vbias = fmaf(p[tc][i], o, vbias);
                    pv[i] = p[tc][i] * sc;
                }
            }
            // column r < G: bf16(pv); column r + G: bf16(pv - bf16(pv))
            const uint32_t h01 = bf16x2_rne(pv[0], pv[1]), h23 = bf16x2_rne(pv[2], pv[3]);
            uint32_t w01 = h01, w23 = h23;
            if (!prim) {
                w01 = bf16x2_rne(pv[0] - bf16lo(h01), pv[1] - bf16hi(h01));
                w23 = bf16x2_rne(pv[2] - bf16lo(h23), pv[3] - bf16hi(h23));
            }
            const s4_t bP = s4_of(w01, w23);
            if (!quant) {
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    acc[m] = mfma16(pair_s4(R.v[tc * MB + m]), bP, acc[m]);
            } else {
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    const int byte = tc * MB + m;
                    const uint32_t code = (word(R.k, 4 + (byte >> 2)) >> (8 * (byte & 3))) & 0xffu;
                    const uint2 a = lut[code];
                    acc[m] = mfma16(s4_of(a.x, a.y), bP, acc[m]);
                }
            }
        };
        value_tile(std::integral_constant<int, 0>{});
        if (ntiles > 1) value_tile(std::integral_constant<int, 1>{});
        if (j.ch + 1 == j.nch) {
            // window done: log-sum-exp of its attention mass per query head (log2 domain)
            float t = lw;
            t += xor_lane<16>(t);
            t += xor_lane<32>(t);
            if (qg == 0 && r < G) lse_out[(int64_t)(e0 + j.i) * g.h_q + hk * G + r] = m_run + log2f(t);
            lw = 0.f;
        }
    };

    // entries are staged in LDS in batches; inside a batch each wave runs a software
    // pipeline in which the next job's loads are in flight while a job is processed
    for (int bs = 0; bs < e_total; bs += DMAXE) {
        __syncthreads();
        e0 = e_begin + bs;
        ne = min(DMAXE, e_total - bs);
        for (int x = threadIdx.x; x < ne; x += 64 * DW) ent[x] = bf.acc[u * g.n_acc_max + e0 + x];
        __syncthreads();
        Raw<D> cur, nxt;
        Job j = resolve(wave);
        load(j, cur);
        while (j.i >= 0) {
            const Job jn = next(j);
            load(jn, nxt);          // in flight while the current job is processed
            process(j, cur);
            cur = nxt;
            j = jn;
        }
    }

    // ---- wave state -> workgroup partial for this split
    float lt = l_run;
    lt += xor_lane<16>(lt);
    lt += xor_lane<32>(lt);
    float vb = vbias;
    vb += xor_lane<16>(vb);
    vb += xor_lane<32>(vb);
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = acc[m][i] + xor_lane<G>(acc[m][i]);     // high + low probability columns
            if (prim) s_acc[wave][r][16 * m + 4 * qg + i] = a + vb;
        }
    if (qg == 0) {
        s_m[wave][r] = m_run;
        s_l[wave][r] = lt;
    }
    __syncthreads();
    float* pacc = bf.part_acc + ((u * g.n_splits + split) * (int64_t)g.h_q + hk * G) * D;
    float2* pml = bf.part_ml + (u * g.n_splits + split) * (int64_t)g.h_q + hk * G;
    for (int x = threadIdx.x; x < G * D; x += 64 * DW) {
        const int gg = x / D, c = x % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < DW; ++w) M = fmaxf(M, s_m[w][gg]);
        float L = 0.f, A = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int w = 0; w < DW; ++w) {
                const float f = s_m[w][gg] > -INFINITY ? exp2f(s_m[w][gg] - M) : 0.f;
                L += f * s_l[w][gg];
                A += f * s_acc[w][gg][c];
            }
        }
        pacc[(int64_t)gg * D + c] = A;
        if (c == 0) pml[gg] = make_float2(M, L);
    }
}

hipError_t launch_decode(const Geo& g, const Bufs& bf, int layer, const uint16_t* q, hipStream_t s) {
    const dim3 grid(g.n_splits, g.h_kv, g.B), block(64 * DW);
    const int G = g.h_q / g.h_kv;
#define QV_DEC(D_, G_)                                                                          \
    if (g.d == D_ && G == G_) {                                                                 \
        hipLaunchKernelGGL((k_decode_split<D_, G_>), grid, block, 0, s, g, bf, layer, q);      \
        return hipGetLastError();                                                               \
    }
    QV_DEC(128, 1) QV_DEC(128, 2) QV_DEC(128, 4) QV_DEC(128, 8)
    QV_DEC(64, 1) QV_DEC(64, 2) QV_DEC(64, 4) QV_DEC(64, 8)
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
