// Prefill score initialisation: causal prompt-attention column sums on MFMA.
//
// Source: "QEvict: Recoverable Quantized KV Eviction for Attention-Drift-Robust
// Long-Context Decoding", §4.2 (prompt attention initialises the window scores):
//   S_bar_0(w) = (1/H_q) sum_h sum_{u < S} sum_{t in w} P_h[u, t],
//   P_h = softmax_causal(Q_h K_g^T / sqrt(d)).
// Column sums of P are formed without materialising it, as the notes
// "Learned KV-cache eviction" describe for their target (log-sum-exp per row,
// then a second pass with query and key roles swapped):
//   pass 1: LSE_u = log sum_{t <= u} exp(l(u, t))               (per query row)
//   pass 2: c_t   = sum_{u >= t} exp(l(u, t) - LSE_u)            (per key column)
// Both passes run bf16 MFMA 16x16x32 tiles with fp32 accumulation; column sums
// accumulate in fp32 within a 64-row tile and in fp64 across tiles.
#include "qevict_common.h"
#include "qevict_internal.h"
#include "qevict_mass.h"

namespace qv {

typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int PF_TILE = 64;
constexpr int PF_PAD = 8;   // LDS row padding (bf16 elements; rows stay 16-byte aligned)
constexpr int PF_GQ = 2;    // query heads per workgroup of the LSE pass (when it divides the GQA group)
constexpr int PF_KB = 2;    // 16-key blocks per wave of the column-sum pass

__device__ __forceinline__ float4_t mfma32x(short8_t a, short8_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(__bf16 __attribute__((ext_vector_type(8))), a),
                                                   __builtin_bit_cast(__bf16 __attribute__((ext_vector_type(8))), b), c, 0,
                                                   0, 0);
}

// Row tile [64][D] of a [.., S_max, D] bf16 buffer, staged through registers so that its
// loads can be issued a tile ahead: D/32 16-byte chunks per thread of a 256-thread
// workgroup, zero past S; then stored to LDS.
template <int D>
__device__ __forceinline__ void tile_regs(uint4* v, const uint16_t* __restrict__ src, int row0, int S) {
    constexpr int CH = D / 8;
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
        const int i = threadIdx.x + 256 * k, r = i / CH, c = (i % CH) * 8;
        v[k] = make_uint4(0, 0, 0, 0);
        if (row0 + r < S) v[k] = *reinterpret_cast<const uint4*>(src + (int64_t)(row0 + r) * D + c);
    }
}
template <int D>
__device__ __forceinline__ void tile_store(uint16_t (*dst)[D + PF_PAD], const uint4* v) {
    constexpr int CH = D / 8;
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
        const int i = threadIdx.x + 256 * k, r = i / CH, c = (i % CH) * 8;
        uint2* d2 = reinterpret_cast<uint2*>(&dst[r][c]);
        d2[0] = make_uint2(v[k].x, v[k].y);
        d2[1] = make_uint2(v[k].z, v[k].w);
    }
}

// ---------------------------------------------------------------- pass 1: row log-sum-exp (log2 domain)
// One workgroup: a 64-row query tile (16 rows per wave) of GQ query heads that share one
// KV head; every key-tile operand read from LDS serves the GQ heads.  Key tiles are
// double-buffered: the next tile's loads go out before this tile's products, and one
// barrier per tile separates the last reads of a buffer from its next fill.
template <int D, int GQ>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) k_prefill_lse(Geo g, Bufs bf, int layer, const uint16_t* __restrict__ qp,
                                                    const uint16_t* __restrict__ kp, float* __restrict__ lse2) {
    __shared__ uint16_t ks[2][PF_TILE][D + PF_PAD];
    const int tile = blockIdx.x, h0 = blockIdx.y * GQ, b = blockIdx.z;
    const int S = bf.hdr[unit_of(g, b, layer)].prompt_len;
    if (tile * PF_TILE >= S) return;
    const int G = g.h_q / g.h_kv, hk = h0 / G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const float scale = 1.4426950408889634f / sqrtf((float)D);
    const uint16_t* K = kp + ((int64_t)b * g.h_kv + hk) * g.S_max * D;
    const int r0 = tile * PF_TILE + wave * 16;
    short8_t qa[GQ][D / 32];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
        const uint16_t* Q = qp + ((int64_t)b * g.h_q + h0 + hh) * g.S_max * D;
        const int row = r0 + lr;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row < S) v = *reinterpret_cast<const uint4*>(Q + (int64_t)row * D + kk * 32 + 8 * lq);
            qa[hh][kk] = __builtin_bit_cast(short8_t, v);
        }
    }
    float m[GQ][4], l[GQ][4];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m[hh][i] = -INFINITY;
            l[hh][i] = 0.f;
        }
    const int last_row = min(tile * PF_TILE + PF_TILE, S) - 1;
    const int n_kt = last_row / PF_TILE + 1;
    uint4 pre[D / 32];
    tile_regs<D>(pre, K, 0, S);
    tile_store<D>(ks[0], pre);
    __syncthreads();
    for (int kt = 0; kt < n_kt; ++kt) {
        if (kt + 1 < n_kt) tile_regs<D>(pre, K, (kt + 1) * PF_TILE, S);
        const uint16_t(*kb)[D + PF_PAD] = ks[kt & 1];
        float4_t sacc[GQ][4];
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
#pragma unroll
            for (int hh = 0; hh < GQ; ++hh) sacc[hh][sub] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                const short8_t bb = *reinterpret_cast<const short8_t*>(&kb[sub * 16 + lr][kk * 32 + 8 * lq]);
#pragma unroll
                for (int hh = 0; hh < GQ; ++hh) sacc[hh][sub] = mfma32x(qa[hh][kk], bb, sacc[hh][sub]);
            }
        }
        // key tiles wholly below the row tile need neither the causal nor the length mask.
        // The reference m of a row moves lazily: only when a score exceeds it by more than 8
        // (log2 units), so terms stay below 2^8 and the rescale is rare after the first tile;
        // the scale folds into one fma per score (it is positive, so the raw maximum orders
        // the scaled ones)
        const bool full = (kt + 1) * PF_TILE <= tile * PF_TILE && (kt + 1) * PF_TILE <= S;
#pragma unroll
        for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = r0 + 4 * lq + i;
                if (full) {
                    const float mx =
                        fmaxf(fmaxf(sacc[hh][0][i], sacc[hh][1][i]), fmaxf(sacc[hh][2][i], sacc[hh][3][i])) * scale;
                    if (mx > m[hh][i] + 8.f) {
                        l[hh][i] *= m[hh][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[hh][i] - mx);
                        m[hh][i] = mx;
                    }
                    float s = l[hh][i];
#pragma unroll
                    for (int sub = 0; sub < 4; ++sub) s += __builtin_amdgcn_exp2f(fmaf(sacc[hh][sub][i], scale, -m[hh][i]));
                    l[hh][i] = s;
                } else {
                    float x[4], mx = -INFINITY;
#pragma unroll
                    for (int sub = 0; sub < 4; ++sub) {
                        const int key = kt * PF_TILE + sub * 16 + lr;
                        x[sub] = (key <= row && key < S) ? sacc[hh][sub][i] * scale : -INFINITY;
                        mx = fmaxf(mx, x[sub]);
                    }
                    if (mx == -INFINITY) continue;
                    if (mx > m[hh][i] + 8.f) {
                        l[hh][i] *= m[hh][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[hh][i] - mx);
                        m[hh][i] = mx;
                    }
                    float s = l[hh][i];
#pragma unroll
                    for (int sub = 0; sub < 4; ++sub)
                        s += x[sub] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[sub] - m[hh][i]);
                    l[hh][i] = s;
                }
            }
        if (kt + 1 < n_kt) tile_store<D>(ks[(kt + 1) & 1], pre);
        __syncthreads();
    }
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float mi = m[hh][i], li = l[hh][i];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const float m2 = wave_xor(mi, o), l2 = wave_xor(li, o);
                const float M = fmaxf(mi, m2);
                float s = 0.f;
                if (M > -INFINITY) {
                    s = (mi > -INFINITY ? li * exp2f(mi - M) : 0.f) + (m2 > -INFINITY ? l2 * exp2f(m2 - M) : 0.f);
                }
                mi = M;
                li = s;
            }
            const int row = r0 + 4 * lq + i;
            if (lr == 0 && row < S) lse2[((int64_t)b * g.h_q + h0 + hh) * g.S_max + row] = mi + log2f(li);
        }
}

// ---------------------------------------------------------------- pass 2: column sums (roles swapped)
// One workgroup: 64*KB keys of one query head; wave w holds the 16-key blocks w, w + 4, ...
// (interleaved, so the causal triangle spreads evenly over the waves), and every query-tile
// operand read from LDS serves its KB blocks.  Query tiles and their row LSEs are
// double-buffered as in pass 1.  Per key the column sum runs over the query tiles in order.
template <int D, int KB>
__global__ void __launch_bounds__(256) k_prefill_colsum(Geo g, Bufs bf, int layer, const uint16_t* __restrict__ qp,
                                                       const uint16_t* __restrict__ kp,
                                                       const float* __restrict__ lse2, double* __restrict__ col) {
    __shared__ uint16_t qs[2][PF_TILE][D + PF_PAD];
    __shared__ float ls[2][PF_TILE];
    const int kgrp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int S = bf.hdr[unit_of(g, b, layer)].prompt_len;
    const int kg0 = kgrp * PF_TILE * KB;   // first key of the workgroup
    if (kg0 >= S) return;
    const int G = g.h_q / g.h_kv, hk = h / G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const float scale = 1.4426950408889634f / sqrtf((float)D);
    const uint16_t* Q = qp + ((int64_t)b * g.h_q + h) * g.S_max * D;
    const uint16_t* K = kp + ((int64_t)b * g.h_kv + hk) * g.S_max * D;
    const float* LS = lse2 + ((int64_t)b * g.h_q + h) * g.S_max;
    short8_t ka[KB][D / 32];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int key = kg0 + (kb * 4 + wave) * 16 + lr;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (key < S) v = *reinterpret_cast<const uint4*>(K + (int64_t)key * D + kk * 32 + 8 * lq);
            ka[kb][kk] = __builtin_bit_cast(short8_t, v);
        }
    }
    double cs[KB][4];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) cs[kb][i] = 0.0;
    const int n_qt = (S - 1) / PF_TILE + 1, qt0 = kg0 / PF_TILE;
    uint4 pre[D / 32];
    float lpre = INFINITY;
    tile_regs<D>(pre, Q, qt0 * PF_TILE, S);
    if (threadIdx.x < PF_TILE && qt0 * PF_TILE + (int)threadIdx.x < S) lpre = LS[qt0 * PF_TILE + threadIdx.x];
    tile_store<D>(qs[0], pre);
    if (threadIdx.x < PF_TILE) ls[0][threadIdx.x] = lpre;
    __syncthreads();
    for (int qt = qt0; qt < n_qt; ++qt) {
        const int nb = (qt - qt0) & 1;
        if (qt + 1 < n_qt) {
            tile_regs<D>(pre, Q, (qt + 1) * PF_TILE, S);
            lpre = INFINITY;
            if (threadIdx.x < PF_TILE && (qt + 1) * PF_TILE + (int)threadIdx.x < S)
                lpre = LS[(qt + 1) * PF_TILE + threadIdx.x];
        }
        const uint16_t(*qb)[D + PF_PAD] = qs[nb];
        const float* lb = ls[nb];
        float part[KB][4];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) part[kb][i] = 0.f;
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
            float4_t c[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) c[kb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                const short8_t bb = *reinterpret_cast<const short8_t*>(&qb[sub * 16 + lr][kk * 32 + 8 * lq]);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) c[kb] = mfma32x(ka[kb][kk], bb, c[kb]);
            }
            const int query = qt * PF_TILE + sub * 16 + lr;
            const float lq_ = lb[sub * 16 + lr];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int kbs = kg0 + (kb * 4 + wave) * 16;   // first key of the block
                // (a block whose keys all follow the tile's queries adds exact zeros: skipped)
                if (qt * PF_TILE + PF_TILE - 1 < kbs) continue;
                // query tile wholly after the key block and inside the prompt: no masks
                const bool full = qt * PF_TILE >= kbs + 16 && (qt + 1) * PF_TILE <= S;
                if (full) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) part[kb][i] += __builtin_amdgcn_exp2f(fmaf(c[kb][i], scale, -lq_));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = kbs + 4 * lq + i;
                        if (query >= key && query < S) part[kb][i] += __builtin_amdgcn_exp2f(fmaf(c[kb][i], scale, -lq_));
                    }
                }
            }
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) cs[kb][i] += (double)part[kb][i];
        if (qt + 1 < n_qt) {
            tile_store<D>(qs[nb ^ 1], pre);
            if (threadIdx.x < PF_TILE) ls[nb ^ 1][threadIdx.x] = lpre;
        }
        __syncthreads();
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            double v = cs[kb][i];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
            const int key = kg0 + (kb * 4 + wave) * 16 + 4 * lq + i;
            if (lr == 0 && key < S) col[((int64_t)b * g.h_q + h) * g.S_max + key] = v;
        }
}

// ---------------------------------------------------------------- per-window reduction
// Window scores from the column sums: a workgroup takes 64 windows, its four waves a
// quarter of the query heads each (partial sums over their heads and the window's tokens,
// then summed in LDS); the first workgroup also sums the sink columns.
__global__ void __launch_bounds__(256) k_prefill_windows(Geo g, Bufs bf, int layer, const double* __restrict__ col) {
    __shared__ double part[4][64];
    const int b = blockIdx.x;
    const int64_t u = unit_of(g, b, layer);
    UnitHdr* hdr = bf.hdr + u;
    const int S = hdr->prompt_len;
    const int n_win = S > g.n_sink ? (S - g.n_sink + g.W - 1) / g.W : 0;
    const int w = blockIdx.y * 64 + (threadIdx.x & 63), hg = threadIdx.x >> 6;
    double s = 0.0;
    if (col && w < n_win) {
        const int a = g.n_sink + w * g.W, e = min(a + g.W, S);
        for (int h = hg; h < g.h_q; h += 4) {
            const double* c = col + ((int64_t)b * g.h_q + h) * g.S_max;
#pragma unroll 8
            for (int t = a; t < e; ++t) s += c[t];
        }
    }
    part[hg][threadIdx.x & 63] = s;
    __syncthreads();
    if (threadIdx.x < 64 && w < g.n_windows) {
        double t = 0.0;
        if (w < n_win) t = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x] + part[3][threadIdx.x]) / g.h_q;
        // (p-norm ranker: P_0 = S_0^3, the initialisation as the first event-level score)
        bf.score[u * g.n_windows + w] = (g.flags & QEVICT_F_RANK_PNORM) ? t * t * t : t;
        bf.uacc[u * g.n_windows + w] = 0.0;
    }
    if (blockIdx.y == 0 && threadIdx.x == 0) {
        double sm = 0.0;
        const int ns = min(g.n_sink, S);
        if (col)
            for (int h = 0; h < g.h_q; ++h)
                for (int t = 0; t < ns; ++t) sm += col[((int64_t)b * g.h_q + h) * g.S_max + t];
        hdr->sink_mass = sm / g.h_q;
    }
}

__global__ void k_score_copy(Geo g, Bufs bf, int layer, const double* __restrict__ init) {
    const int b = blockIdx.x;
    const int64_t u = unit_of(g, b, layer);
    const int S = bf.hdr[u].prompt_len;
    const int n_win = S > g.n_sink ? (S - g.n_sink + g.W - 1) / g.W : 0;
    for (int w = threadIdx.x; w < g.n_windows; w += blockDim.x) {
        const double s = w < n_win ? init[(int64_t)b * g.n_windows + w] : 0.0;
        bf.score[u * g.n_windows + w] = (g.flags & QEVICT_F_RANK_PNORM) ? s * s * s : s;
        bf.uacc[u * g.n_windows + w] = 0.0;
    }
    if (threadIdx.x == 0) bf.hdr[u].sink_mass = 0.0;
}

// Key-norm ranker at prefill (Appendix J, Eq. 24): the rank keys of the prompt windows that
// age at the prefill routing, from the prompt's bf16 keys; the others start at 0 and get
// theirs from their pages when they age.  One workgroup per (window, sequence).
__global__ void __launch_bounds__(256) k_prefill_keynorm(Geo g, Bufs bf, int layer, const uint16_t* __restrict__ kp) {
    __shared__ double tokn[64];
    const int w = blockIdx.x, b = blockIdx.y;
    const int64_t u = unit_of(g, b, layer);
    const int S = bf.hdr[u].prompt_len;
    const int a = g.n_sink + w * g.W;
    double r = 0.0;
    if (a + g.W <= S - g.n_local) {
        r = key_norm_block(g, g.W, [&](int i, int hk, int c) {
            return __uint_as_float((uint32_t)kp[(((int64_t)b * g.h_kv + hk) * g.S_max + a + i) * g.d + c] << 16);
        }, tokn);
    }
    if (threadIdx.x == 0) {
        bf.score[u * g.n_windows + w] = r;
        bf.uacc[u * g.n_windows + w] = 0.0;
        if (w == 0) bf.hdr[u].sink_mass = 0.0;
    }
}

// RoPE of a prompt tensor [B][H][S_max][d] (bf16 in, bf16 out): each thread turns one
// channel pair (i, i + d/2) of one position, exactly in fp64, rounded once to bf16.
__global__ void __launch_bounds__(256) k_rope_prompt(Geo g, Bufs bf, const uint16_t* __restrict__ x,
                                                      uint16_t* __restrict__ y, int H) {
    const int h = g.d / 2;
    const int64_t n_pairs = (int64_t)g.B * H * g.S_max * h;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n_pairs; e += (int64_t)gridDim.x * blockDim.x) {
        const int i = (int)(e % h);
        const int64_t row = e / h;                      // (b, head, p)
        const int p = (int)(row % g.S_max);
        const float2 cs = bf.rope[(int64_t)p * h + i];
        const double a = (double)bf16_to_f32(x[row * g.d + i]), b = (double)bf16_to_f32(x[row * g.d + i + h]);
        y[row * g.d + i] = f64_to_bf16(__dsub_rn(__dmul_rn(a, (double)cs.x), __dmul_rn(b, (double)cs.y)));
        y[row * g.d + i + h] = f64_to_bf16(__dadd_rn(__dmul_rn(b, (double)cs.x), __dmul_rn(a, (double)cs.y)));
    }
}

hipError_t launch_rope_prompt(const Geo& g, const Bufs& bf, const uint16_t* qp, const uint16_t* kp, void* ws,
                              const uint16_t** qr, const uint16_t** kr, hipStream_t s) {
    uint16_t* q_out = (uint16_t*)((char*)ws + rope_ws_offset(g));
    const size_t nq = (size_t)g.B * g.h_q * g.S_max * g.d * 2;
    uint16_t* k_out = (uint16_t*)((char*)q_out + ((nq + 255) & ~size_t(255)));
    *qr = qp ? q_out : nullptr;
    *kr = k_out;
    if (g.S_max == 0) return hipSuccess;
    if (qp) hipLaunchKernelGGL(k_rope_prompt, dim3(2048), dim3(256), 0, s, g, bf, qp, q_out, g.h_q);
    hipLaunchKernelGGL(k_rope_prompt, dim3(2048), dim3(256), 0, s, g, bf, kp, k_out, g.h_kv);
    return hipGetLastError();
}

hipError_t launch_prefill_scores(const Geo& g, const Bufs& bf, int layer, const uint16_t* qp, const uint16_t* kp,
                                 const double* score_init, void* ws, hipStream_t s) {
    if (g.flags & QEVICT_F_RANK_KEYNORM) {   // no attention mass: scores from the prompt keys
        hipLaunchKernelGGL(k_prefill_keynorm, dim3(g.n_windows, g.B), dim3(256), 0, s, g, bf, layer, kp);
        return hipGetLastError();
    }
    if (score_init) {
        hipLaunchKernelGGL(k_score_copy, dim3(g.B), dim3(256), 0, s, g, bf, layer, score_init);
        return hipGetLastError();
    }
    const dim3 grid_w(g.B, std::max(1, (g.n_windows + 63) / 64));
    if (g.S_max == 0) {
        hipLaunchKernelGGL(k_prefill_windows, grid_w, dim3(256), 0, s, g, bf, layer, (const double*)nullptr);
        return hipGetLastError();
    }
    const size_t n = (size_t)g.B * g.h_q * g.S_max;
    float* lse2 = (float*)ws;
    double* col = (double*)((char*)ws + ((n * 4 + 255) & ~size_t(255)));
    // query heads per LSE workgroup (PF_GQ when it divides the GQA group) and 16-key blocks per
    // wave in the column-sum pass
    const int G = g.h_q / g.h_kv, gq = G % PF_GQ == 0 ? PF_GQ : 1;
    const dim3 grid_l((g.S_max + PF_TILE - 1) / PF_TILE, g.h_q / gq, g.B);
    const dim3 grid_c((g.S_max + PF_TILE * PF_KB - 1) / (PF_TILE * PF_KB), g.h_q, g.B);
    if (g.d == 128) {
        if (gq == PF_GQ) hipLaunchKernelGGL((k_prefill_lse<128, PF_GQ>), grid_l, dim3(256), 0, s, g, bf, layer, qp, kp, lse2);
        else hipLaunchKernelGGL((k_prefill_lse<128, 1>), grid_l, dim3(256), 0, s, g, bf, layer, qp, kp, lse2);
        hipLaunchKernelGGL((k_prefill_colsum<128, PF_KB>), grid_c, dim3(256), 0, s, g, bf, layer, qp, kp, lse2, col);
    } else {
        if (gq == PF_GQ) hipLaunchKernelGGL((k_prefill_lse<64, PF_GQ>), grid_l, dim3(256), 0, s, g, bf, layer, qp, kp, lse2);
        else hipLaunchKernelGGL((k_prefill_lse<64, 1>), grid_l, dim3(256), 0, s, g, bf, layer, qp, kp, lse2);
        hipLaunchKernelGGL((k_prefill_colsum<64, PF_KB>), grid_c, dim3(256), 0, s, g, bf, layer, qp, kp, lse2, col);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_prefill_windows, grid_w, dim3(256), 0, s, g, bf, layer, col);
    return hipGetLastError();
}

}  // namespace qv
