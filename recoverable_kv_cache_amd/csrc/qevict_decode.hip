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

#include "qevict_common.h"
#include "qevict_internal.h"

namespace qv {

constexpr int DEC_WAVES = 4;

template <int CPL>
struct Row {
    float v[CPL];
};

// CPL bf16 values at p (16-byte aligned)
template <int CPL>
__device__ __forceinline__ void load_bf16_row(const uint16_t* __restrict__ p, float* x) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int k = 0; k < CPL / 8; ++k) {
        const uint4 w = q[k];
        x[8 * k + 0] = bf16lo(w.x); x[8 * k + 1] = bf16hi(w.x);
        x[8 * k + 2] = bf16lo(w.y); x[8 * k + 3] = bf16hi(w.y);
        x[8 * k + 4] = bf16lo(w.z); x[8 * k + 5] = bf16hi(w.z);
        x[8 * k + 6] = bf16lo(w.w); x[8 * k + 7] = bf16hi(w.w);
    }
}

// CPL 2-bit codes at p (channel c of the row: byte c/4, bits 2(c%4)) -> floats
template <int CPL>
__device__ __forceinline__ void load_codes(const uint8_t* __restrict__ p, float* x) {
    if constexpr (CPL == 16) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t m = (w >> (2 * s)) & 0x03030303u;
            x[0 + s] = (float)(m & 0xffu);
            x[4 + s] = (float)((m >> 8) & 0xffu);
            x[8 + s] = (float)((m >> 16) & 0xffu);
            x[12 + s] = (float)(m >> 24);
        }
    } else {
        const uint32_t w = *reinterpret_cast<const uint16_t*>(p);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t m = (w >> (2 * s)) & 0x0303u;
            x[0 + s] = (float)(m & 0xffu);
            x[4 + s] = (float)(m >> 8);
        }
    }
}

template <int CPL>
__device__ __forceinline__ void load_f16_row(const uint16_t* __restrict__ p, float* x) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) x[k] = fp16_bits_to_f32(p[k]);
}

template <int D, int G>
__global__ void __launch_bounds__(64 * DEC_WAVES) k_decode_split(Geo g, Bufs bf, int layer,
                                                                  const uint16_t* __restrict__ qin) {
    constexpr int CPL = G <= 4 ? 16 : 8;     // channels per lane
    constexpr int LPT = D / CPL;             // lanes per token
    constexpr int TPI = 64 / LPT;            // tokens per wave iteration
    const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int64_t u = unit_of(g, b, layer);
    const int n = bf.hdr[u].n;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tg = lane / LPT, j = lane % LPT, c0 = j * CPL;
    const int W = g.W;

    // queries of the group, pre-scaled to the log2 domain: log2(e) / sqrt(d)
    const float qscale = 1.4426950408889634f / sqrtf((float)D);
    float qf[G][CPL];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
        float t[CPL];
        load_bf16_row<CPL>(qin + ((int64_t)b * g.h_q + hk * G + gg) * D + c0, t);
#pragma unroll
        for (int c = 0; c < CPL; ++c) qf[gg][c] = t[c] * qscale;
    }
    float m_run[G], l_run[G], acc[G][CPL];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
        m_run[gg] = -INFINITY;
        l_run[gg] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[gg][c] = 0.f;
    }

    const int32_t* splits = bf.splits + u * (g.n_splits + 1);
    const int e0 = splits[split], e1 = splits[split + 1];
    const AccEntry* list = bf.acc + u * g.n_acc_max;
    const uint16_t* pages = bf.pages + u * (int64_t)g.n_pages * g.page_elems;
    const uint8_t* slots = bf.slots + u * (int64_t)g.n_slots * g.slot_bytes;
    float* lse_out = bf.lse_win + u * (int64_t)g.n_acc_max * g.h_q;

    for (int e = e0 + wave; e < e1; e += DEC_WAVES) {
        const AccEntry en = list[e];
        int ntok;
        if (en.kind == EK_SINK) ntok = g.n_sink < n ? g.n_sink : n;
        else ntok = n - en.start < W ? n - en.start : W;
        if (ntok <= 0 || (en.kind != EK_SINK && en.idx < 0)) continue;
        const bool quant = en.kind == EK_SLOT;
        const uint16_t *kb = nullptr, *vb = nullptr;
        const uint8_t *kc = nullptr, *vc = nullptr;
        const uint16_t *offV = nullptr, *sclV = nullptr;
        float offK[CPL], sclK[CPL];
        if (en.kind == EK_SINK) {
            const int ns = g.n_sink;
            kb = bf.sinks + u * g.sink_elems + (int64_t)(2 * hk) * ns * D;
            vb = kb + (int64_t)ns * D;
        } else if (!quant) {
            kb = pages + (int64_t)en.idx * g.page_elems + (int64_t)(2 * hk) * W * D;
            vb = kb + (int64_t)W * D;
        } else {
            const uint8_t* sl = slots + (int64_t)en.idx * g.slot_bytes + (int64_t)hk * g.slot_head_bytes;
            kc = sl;
            vc = sl + W * D / 4;
            const uint16_t* oK = (const uint16_t*)(sl + W * D / 2);
            const uint16_t* sK = oK + D;
            offV = sK + D;
            sclV = offV + W;
            load_f16_row<CPL>(oK + c0, offK);
            load_f16_row<CPL>(sK + c0, sclK);
        }
        float lw[G];
#pragma unroll
        for (int gg = 0; gg < G; ++gg) lw[gg] = 0.f;

        for (int t0 = 0; t0 < ntok; t0 += TPI) {
            const int t = t0 + tg;
            const bool valid = t < ntok;
            const int tt = valid ? t : 0;
            float x[CPL];
            if (!quant) {
                load_bf16_row<CPL>(kb + (int64_t)tt * D + c0, x);
            } else {
                load_codes<CPL>(kc + tt * (D / 4) + c0 / 4, x);
#pragma unroll
                for (int c = 0; c < CPL; ++c) x[c] = fmaf(x[c], sclK[c], offK[c]);
            }
            float sl[G];
#pragma unroll
            for (int gg = 0; gg < G; ++gg) {
                float dot = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) dot = fmaf(qf[gg][c], x[c], dot);
#pragma unroll
                for (int o = 1; o < LPT; o <<= 1) dot += wave_xor(dot, o);
                sl[gg] = valid ? dot : -INFINITY;
            }
            float p[G];
#pragma unroll
            for (int gg = 0; gg < G; ++gg) {
                float mx = sl[gg];
#pragma unroll
                for (int o = LPT; o < 64; o <<= 1) mx = fmaxf(mx, wave_xor(mx, o));
                const float mnew = fmaxf(m_run[gg], mx);
                if (mnew > m_run[gg]) {
                    const float alpha = exp2f(m_run[gg] - mnew);
                    l_run[gg] *= alpha;
                    lw[gg] *= alpha;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) acc[gg][c] *= alpha;
                    m_run[gg] = mnew;
                }
                p[gg] = valid ? exp2f(sl[gg] - m_run[gg]) : 0.f;
                l_run[gg] += p[gg];
                lw[gg] += p[gg];
            }
            float y[CPL];
            if (!quant) {
                load_bf16_row<CPL>(vb + (int64_t)tt * D + c0, y);
            } else {
                load_codes<CPL>(vc + tt * (D / 4) + c0 / 4, y);
                const float ov = fp16_bits_to_f32(offV[tt]), sv = fp16_bits_to_f32(sclV[tt]);
#pragma unroll
                for (int c = 0; c < CPL; ++c) y[c] = fmaf(y[c], sv, ov);
            }
#pragma unroll
            for (int gg = 0; gg < G; ++gg)
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[gg][c] = fmaf(p[gg], y[c], acc[gg][c]);
        }
        // per-window log-sum-exp of every query head of the group (log2 domain)
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
            float s = lw[gg];
#pragma unroll
            for (int o = LPT; o < 64; o <<= 1) s += wave_xor(s, o);
            if (lane == 0) lse_out[(int64_t)e * g.h_q + hk * G + gg] = m_run[gg] + log2f(s);
        }
    }

    // reduce the wave's state over its token groups, then across the waves
    __shared__ float s_m[DEC_WAVES][G], s_l[DEC_WAVES][G];
    __shared__ float s_acc[DEC_WAVES][G][D];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
        float l = l_run[gg];
#pragma unroll
        for (int o = LPT; o < 64; o <<= 1) l += wave_xor(l, o);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float a = acc[gg][c];
#pragma unroll
            for (int o = LPT; o < 64; o <<= 1) a += wave_xor(a, o);
            if (tg == 0) s_acc[wave][gg][c0 + c] = a;
        }
        if (lane == 0) {
            s_m[wave][gg] = m_run[gg];
            s_l[wave][gg] = l;
        }
    }
    __syncthreads();
    float* pacc = bf.part_acc + ((u * g.n_splits + split) * (int64_t)g.h_q + hk * G) * D;
    float2* pml = bf.part_ml + (u * g.n_splits + split) * (int64_t)g.h_q + hk * G;
    for (int i = threadIdx.x; i < G * D; i += 64 * DEC_WAVES) {
        const int gg = i / D, c = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, s_m[w][gg]);
        float L = 0.f, A = 0.f;
        if (M > -INFINITY) {
#pragma unroll
            for (int w = 0; w < DEC_WAVES; ++w) {
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
    const dim3 grid(g.n_splits, g.h_kv, g.B), block(64 * DEC_WAVES);
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
__global__ void k_combine(Geo g, Bufs bf, int layer, float* __restrict__ out) {
    const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
    const int64_t u = unit_of(g, b, layer);
    const float2* pml = bf.part_ml + u * g.n_splits * (int64_t)g.h_q + h;
    const float* pacc = bf.part_acc + (u * g.n_splits * (int64_t)g.h_q + h) * g.d + c;
    float M = -INFINITY;
    for (int s = 0; s < g.n_splits; ++s) M = fmaxf(M, pml[(int64_t)s * g.h_q].x);
    float L = 0.f, A = 0.f;
    for (int s = 0; s < g.n_splits; ++s) {
        const float2 ml = pml[(int64_t)s * g.h_q];
        const float f = ml.x > -INFINITY ? exp2f(ml.x - M) : 0.f;
        L += f * ml.y;
        A += f * pacc[(int64_t)s * g.h_q * g.d];
    }
    out[((int64_t)b * g.h_q + h) * g.d + c] = A / L;
    if (c == 0) bf.lse_glob[u * g.h_q + h] = M + log2f(L);
}

hipError_t launch_combine(const Geo& g, const Bufs& bf, int layer, float* out, hipStream_t s) {
    hipLaunchKernelGGL(k_combine, dim3(g.h_q, g.B), dim3(g.d), 0, s, g, bf, layer, out);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------ window mass
// u(w) = (1/H_q) sum_h 2^(lse_w,h - LSE_h) = (1/H_q) sum_h sum_{i in w} a_h(i);  S_bar(w) += u(w)
__global__ void k_mass(Geo g, Bufs bf, int layer) {
    const int b = blockIdx.y;
    const int64_t u = unit_of(g, b, layer);
    const UnitHdr* hdr = bf.hdr + u;
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e == 0 || e >= hdr->n_acc) return;
    if (g.flags & QEVICT_F_SCORE_ROUTE_ONLY) {
        const int j = hdr->n - hdr->prompt_len - 1;   // index of the decode step just taken
        if ((j + 1) % g.omega != 0) return;
    }
    const AccEntry en = bf.acc[u * g.n_acc_max + e];
    if (en.start >= hdr->n) return;
    const float* lw = bf.lse_win + (u * g.n_acc_max + e) * (int64_t)g.h_q;
    const float* lg = bf.lse_glob + u * g.h_q;
    double s = 0.0;
    for (int h = 0; h < g.h_q; ++h) s += (double)exp2f(lw[h] - lg[h]);
    bf.score[u * g.n_windows + en.win] += s / g.h_q;
}

hipError_t launch_mass(const Geo& g, const Bufs& bf, int layer, hipStream_t s) {
    const int nb = (g.n_acc_max + 255) / 256;
    hipLaunchKernelGGL(k_mass, dim3(nb, g.B), dim3(256), 0, s, g, bf, layer);
    return hipGetLastError();
}

}  // namespace qv
