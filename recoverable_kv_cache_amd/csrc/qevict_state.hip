// State kernels: arena initialisation, prefill setup, the
// window router (candidate pool + two-stage TopK + migration bookkeeping +
// chronological compaction) and the INT2 pack / dequantize-promote kernels.
//
// Source: "QEvict: Recoverable Quantized KV Eviction for Attention-Drift-Robust
// Long-Context Decoding", §4.3 (Eq. 3 capacities, "Migration-Stable
// Quantization", Eqs. 4-6), Appendix A Algorithm 1.
#include "qevict_common.h"
#include "qevict_internal.h"

#include <type_traits>
#include <hip/hip_ext.h>

#include "qevict_mass.h"

namespace qv {

// ------------------------------------------------------------------------------------ init
__global__ void k_init(Geo g, Bufs bf, const int32_t* plens, const int32_t* kf, const int32_t* kq) {
    const int64_t u = blockIdx.x;
    const int b = (int)(u / g.L);
    if (threadIdx.x == 0) {
        UnitHdr h = {};
        h.prompt_len = plens[b];
        h.n_free_pages = g.n_pages;
        h.n_free_slots = g.n_slots;
        h.K_f = kf[b];
        h.K_q = kq[b];
        bf.hdr[u] = h;
    }
    for (int i = threadIdx.x; i < g.n_pages; i += blockDim.x) bf.free_pages[u * g.n_pages + i] = g.n_pages - 1 - i;
    for (int i = threadIdx.x; i < g.n_slots; i += blockDim.x) bf.free_slots[u * g.n_slots + i] = g.n_slots - 1 - i;
    for (int w = threadIdx.x; w < g.n_windows; w += blockDim.x) {
        bf.win[u * g.n_windows + w] = WinRec{ST_NONE, -1, -1, 0};
        bf.score[u * g.n_windows + w] = 0.0;
        bf.uacc[u * g.n_windows + w] = 0.0;
        bf.target[u * g.n_windows + w] = 0;
    }
    for (int s = threadIdx.x; s <= g.n_splits; s += blockDim.x) bf.splits[u * (g.n_splits + 1) + s] = 0;
    if (threadIdx.x == 0) bf.unit_arr[u] = 0u;
}

hipError_t launch_init(const Geo& g, const Bufs& bf, const int32_t* plens, const int32_t* kf, const int32_t* kq,
                       hipStream_t s) {
    hipLaunchKernelGGL(k_init, dim3(g.B * g.L), dim3(256), 0, s, g, bf, plens, kf, kq);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------ prefill setup
// n = prompt_len; every window holding prompt tokens is marked PROMPT (its
// data still lives in the caller's buffer); sink tokens are copied.
__global__ void k_prefill_setup(Geo g, Bufs bf, int layer, const uint16_t* __restrict__ kp,
                                const uint16_t* __restrict__ vp) {
    const int b = blockIdx.x;
    const int64_t u = unit_of(g, b, layer);
    UnitHdr* hdr = bf.hdr + u;
    const int S = hdr->prompt_len;
    const int n_win = S > g.n_sink ? (S - g.n_sink + g.W - 1) / g.W : 0;
    for (int w = threadIdx.x; w < n_win; w += blockDim.x) bf.win[u * g.n_windows + w].state = ST_PROMPT;
    const int Ws = sink_width(g.n_sink);
    const int nsk = S < g.n_sink ? S : g.n_sink;
    uint16_t* sb = bf.sinks + u * g.sink_elems;
    for (int e = threadIdx.x; e < g.sink_elems; e += blockDim.x) sb[e] = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < g.h_kv * nsk * g.d; e += blockDim.x) {
        const int h = e / (nsk * g.d), t = (e / g.d) % nsk, c = e % g.d;
        const int64_t src = (((int64_t)b * g.h_kv + h) * g.S_max + t) * g.d + c;
        uint16_t* kh = sb + (int64_t)(2 * h) * Ws * g.d;
        kh[lay_k(t, c, g.d, Ws)] = kp[src];
        kh[(int64_t)Ws * g.d + lay_v(t, c, g.d, Ws)] = vp[src];
    }
    if (threadIdx.x == 0) {
        hdr->n = S;
        hdr->n_win = n_win;
        hdr->mass_pending = 0;
        hdr->tok_at = -1;
    }
}

hipError_t launch_prefill_setup(const Geo& g, const Bufs& bf, int layer, const uint16_t* kp, const uint16_t* vp,
                                hipStream_t s) {
    hipLaunchKernelGGL(k_prefill_setup, dim3(g.B), dim3(256), 0, s, g, bf, layer, kp, vp);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------ forced targets
__global__ void k_force_targets(Geo g, Bufs bf, int layer, const int32_t* __restrict__ ids, int n, int tgt) {
    const int b = blockIdx.x;
    const int64_t u = unit_of(g, b, layer);
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int w = ids[(int64_t)b * n + i];
        if (w >= 0 && w < g.n_windows) bf.target[u * g.n_windows + w] = (int8_t)tgt;
    }
}

hipError_t launch_force_targets(const Geo& g, const Bufs& bf, int layer, const int32_t* ids, int n, int tgt,
                                hipStream_t s) {
    hipLaunchKernelGGL(k_force_targets, dim3(g.B), dim3(256), 0, s, g, bf, layer, ids, n, tgt);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------ router
// Reduction over the 64 lanes of a wave (every lane gets the result) with DPP moves and
// the gfx950 row swaps: no LDS traffic.  Every DPP pattern reads a lane of the same row,
// so bound_ctrl changes no value.  op: associative and commutative.
template <typename Op>
__device__ __forceinline__ unsigned wave_reduce_u32(unsigned x, Op op) {
    x = op(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true));    // quad [1,0,3,2]
    x = op(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true));    // quad [2,3,0,1]
    x = op(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, true));   // row_half_mirror
    x = op(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, true));   // row_mirror
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = op(a[0], a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return op(c[0], c[1]);
}
// min and max over aligned groups of G consecutive lanes (G a power of two, at most 64);
// every lane of a group gets its group's results.  Quad permutes, then the mirrors within
// 8 and within 16 lanes, then the row swaps: each step stays inside the group.
template <int G>
__device__ __forceinline__ void group_minmax(float& mn, float& mx) {
    auto dpp = [](float v, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, true));
    };
    if constexpr (G >= 2) {
        mn = fminf(mn, dpp(mn, std::integral_constant<int, 0xB1>{}));
        mx = fmaxf(mx, dpp(mx, std::integral_constant<int, 0xB1>{}));
    }
    if constexpr (G >= 4) {
        mn = fminf(mn, dpp(mn, std::integral_constant<int, 0x4E>{}));
        mx = fmaxf(mx, dpp(mx, std::integral_constant<int, 0x4E>{}));
    }
    if constexpr (G >= 8) {
        mn = fminf(mn, dpp(mn, std::integral_constant<int, 0x141>{}));
        mx = fmaxf(mx, dpp(mx, std::integral_constant<int, 0x141>{}));
    }
    if constexpr (G >= 16) {
        mn = fminf(mn, dpp(mn, std::integral_constant<int, 0x140>{}));
        mx = fmaxf(mx, dpp(mx, std::integral_constant<int, 0x140>{}));
    }
    if constexpr (G >= 32) {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
        const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mn = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
        mx = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
    }
    if constexpr (G >= 64) {
        const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
        const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mn = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
        mx = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
    }
}

__device__ __forceinline__ int wave_sum_i32(int x) {
    return (int)wave_reduce_u32((unsigned)x, [](unsigned p, unsigned q) { return p + q; });
}
__device__ __forceinline__ unsigned wave_and_u32(unsigned x) {
    return wave_reduce_u32(x, [](unsigned p, unsigned q) { return p & q; });
}
__device__ __forceinline__ unsigned wave_or_u32(unsigned x) {
    return wave_reduce_u32(x, [](unsigned p, unsigned q) { return p | q; });
}

// Inclusive prefix sum over the 64 lanes of a wave: row shifts within the rows of 16, then
// the row broadcasts carry the totals of rows 0 and 0-1 upward.  Lanes a DPP move does
// not write (no source lane, or a row outside row_mask) take 0.
__device__ __forceinline__ unsigned wave_scan_incl(unsigned x) {
    x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}
// Cost of one accessible entry for a decode wave, in halves of a job: a Quantized
// window is half of a pair job, a bf16 page of W tokens takes about as long as a pair
// job of W-token windows, the sink block its share of a page.  Splits are balanced on
// these, so that each workgroup's four waves get a like number of jobs (a workgroup
// ends with its slowest wave).
__device__ __forceinline__ int per_head_cost(const Geo& g, int kind) {
    if (kind == EK_SINK) return max(1, 4 * sink_width(g.n_sink) / g.W);
    if (kind == EK_PAGE) return 4;
    return 2;
}

// Total order of doubles as unsigned integers, ascending; -0 counts as +0 (so equal
// scores tie and fall to the window index).  Rank keys of every ranker, negative ones
// (key-norm) included.
__device__ inline unsigned long long ord_key(double s) {
    const unsigned long long bits = (unsigned long long)__double_as_longlong(s + 0.0);
    return (bits >> 63) ? ~bits : (bits | (1ull << 63));
}
// the router, per workgroup size (qevict_route_impl.h)
namespace rt1024 {
#define QV_RT_THREADS 1024
#include "qevict_route_impl.h"
#undef QV_RT_THREADS
}  // namespace rt1024
namespace rt256 {
#define QV_RT_THREADS 256
#include "qevict_route_impl.h"
#undef QV_RT_THREADS
}  // namespace rt256

// ------------------------------------------------------------------------------------ migration work lists
// A routing launch covers units ub = 0..n_units-1 (layer >= 0: (ub, layer); else (ub / L,
// ub % L)).  The pack / fill items of all its units form one list, unit by unit, which the
// workgroups of a migration kernel share (few items per routing event: a grid sized by
// unit would be almost all empty workgroups).  Every workgroup reads the per-unit counts
// and keeps their running sums in LDS; a list index finds its unit by binary search.
// (512 threads: with 1024 a thread has 128 registers, and the pack and fill items of one
// kernel then spill)
constexpr int PK_THREADS = 512;   // threads of the migration kernel (one item per workgroup: latency)

__device__ __forceinline__ int64_t mig_unit(const Geo& g, int layer, int ub, int& b) {
    b = layer >= 0 ? ub : ub / g.L;
    const int l = layer >= 0 ? layer : ub % g.L;
    return unit_of(g, b, l);
}
// the unit of list index i: the last ub with pre[ub] <= i
__device__ __forceinline__ int mig_find(const int* pre, int n_units, int i) {
    int lo = 0, hi = n_units - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= i) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// ------------------------------------------------------------------------------------ pack (INT2 / INT4, once)
// Keys: per (head, channel) over the window's tokens; values: per (head, token)
// over channels.  With L = 2^b - 1 levels (b = 2, or 4 for the INT4 tier):
// off = RD_fp16(min), scl = RU_fp16((max - off)/L), code =
// #{k in 1..L : 2(x - off) >= (2k-1) scl}, 0 when scl == 0.  All comparisons in
// fp64, where they are exact for bf16 x and fp16 off/scl.
//
// One workgroup per (window, KV head) item: the bf16 keys and values come into LDS in
// [token][channel] order by 16-byte loads; the parameters are min / max reductions with
// every thread taking a slice (a key channel's tokens, a value token's channels), combined
// across lanes; then each thread produces code bytes of the slot, computing the codes of
// each byte where it is written.  A workgroup of 512 threads takes one item at a time:
// a routing event moves few windows, and their latency is what counts.
constexpr int PK_MAXE = 64 * 128;   // W * d

// position (token t, channel c) of the element at offset o of a page's key block (lay_k)
__device__ __forceinline__ void page_k_pos(int o, int D, int W, int& t, int& c) {
    const int CQ = D / 4, TPC = lay_tpc(W);
    const int cq = o % CQ;
    int x = o / CQ;
    const int tc = x % TPC;
    x /= TPC;
    const int qg = x % 4;
    x /= 4;
    const int r = x % 16, ch = x / 16;
    t = (ch * TPC + tc) * 16 + r;
    c = qg * CQ + cq;
}
// the same for a page's value block (lay_v)
__device__ __forceinline__ void page_v_pos(int o, int D, int W, int& t, int& c) {
    const int NT = W / 16, MB = D / 16;
    const int t3 = o & 3;
    int x = o >> 2;
    const int cb = x % MB;
    x /= MB;
    const int tt = x % NT;
    x /= NT;
    const int tq = x % 4, c15 = x / 4;
    t = tt * 16 + tq * 4 + t3;
    c = cb * 16 + c15;
}
// key code byte B (lay_kc_byte): its token and the channel of its first code; the code at
// bits b*j (j < 8/b) is that of channel kc_chan(.., j)
__device__ __forceinline__ void kc_byte_pos(int B, int D, int W, int b, int& t, int& qg, int& cc0) {
    const int CQ = D / 4, TPC = lay_tpc(W), P = 8 / b, CQP = CQ / P;
    cc0 = (B % CQP) * P;
    int x = B / CQP;
    const int tc = x % TPC;
    x /= TPC;
    qg = x % 4;
    x /= 4;
    const int r = x % 16, ch = x / 16;
    t = (ch * TPC + tc) * 16 + r;
}
__device__ __forceinline__ int kc_chan(int qg, int cc, int D, bool rope) {   // inverse of lay_kc_pos
    const int CQ = D / 4;
    if (!rope) return qg * CQ + cc;
    return cc < CQ / 2 ? qg * (CQ / 2) + cc : D / 2 + qg * (CQ / 2) + (cc - CQ / 2);
}
// value code byte B (lay_vc_byte): its channel and the token of its first code; the code at
// bits b*j is that of token t0 + j
__device__ __forceinline__ void vc_byte_pos(int B2, int D, int W, int b, int& t0, int& c) {
    const int TPC = lay_tpc(W), MB = D / 16, P = 8 / b, Q = 4 / P;
    const int sub = B2 % Q;
    int x = B2 / Q;
    const int tt = x % TPC;
    x /= TPC;
    const int cb = x % MB;
    x /= MB;
    const int tq = x % 4;
    x /= 4;
    const int c15 = x % 16, tch = x / 16;
    t0 = (tch * TPC + tt) * 16 + tq * 4 + sub * P;
    c = cb * 16 + c15;
}

// the level of t2 = 2(x - off) >= 0 among 0..L (nearest, ties up): an estimate from the
// reciprocal of the scale (inv = 0 when scl = 0), settled by exact fp64 comparisons with the
// thresholds on either side (the estimate is off by at most one: the product carries two
// roundings).  Branch-free.
__device__ __forceinline__ int nearest_level(double t2, double scl, double inv, int L) {
    int k = (int)((t2 * inv + 1.0) * 0.5);
    k = k > L ? L : k;
    k += (k < L && t2 >= (double)(2 * k + 1) * scl) ? 1 : 0;
    k -= (k > 0 && t2 < (double)(2 * k - 1) * scl) ? 1 : 0;
    return scl == 0.0 ? 0 : k;
}

// LDS of the migration kernel: a pack item's bf16 staging and parameters, or a fill item's
// slot words (the two never hold data at the same time), and the work-list sums.  (The
// staging takes 16-byte LDS stores: 16-byte alignment.)
struct alignas(16) MigSmem {
    union alignas(16) {
        struct {
            uint16_t sk[PK_MAXE];
            uint16_t sv[PK_MAXE];
        } p;
        uint32_t sw[(2 * PK_MAXE / 2 + 4 * (128 + 64)) / 4];   // slot head words at W*d = 8192, INT4
    } st;
    double p_off[128 + 64], p_scl[128 + 64], p_inv[128 + 64];   // key channels, then value tokens
    uint16_t p_bits[2 * (128 + 64)];
    int pre[MIG_MAX_UNITS + 1];     // pack items of the units before each unit
    int pre_f[MIG_MAX_UNITS + 1];   // fill items of the units before each unit
    int wtot[PK_THREADS / 64], wtot2[PK_THREADS / 64];
};

// One pack item: head h of window pi.win of unit u into slot pi.dst_slot.  All threads call.
// W, d, QB: the window, head dimension and code bits (one instance per supported shape, so
// that the layout arithmetic is shifts and masks)
template <int W, int d, int QB>
__device__ void pack_item(const Geo& g, const Bufs& bf, int64_t u, int b, const PackItem& pi, int h,
                          const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp, MigSmem& sm) {
    uint16_t* sk = sm.st.p.sk;
    uint16_t* sv = sm.st.p.sv;
    double* p_off = sm.p_off;
    double* p_scl = sm.p_scl;
    double* p_inv = sm.p_inv;
    uint16_t* p_bits = sm.p_bits;
    constexpr int WD = W * d;
    const int tid = threadIdx.x;
    const bool rope = (g.flags & QEVICT_F_ROPE) != 0;
    constexpr int hd = d / 2;
    UnitHdr* hdr = bf.hdr + u;
    {
        const int start = g.n_sink + pi.win * W;
        if (pi.dst_slot < 0 || (!pi.src_prompt && pi.src_page < 0)) {
            if (tid == 0) atomicOr(&hdr->status, QEVICT_DEV_E_POOL);
            return;
        }
        // ---- stage keys and values, [token][channel]
        if (pi.src_prompt) {
            const uint16_t* srck = kp + (((int64_t)b * g.h_kv + h) * g.S_max + start) * d;
            const uint16_t* srcv = vp + (((int64_t)b * g.h_kv + h) * g.S_max + start) * d;
            if ((((uintptr_t)srck | (uintptr_t)srcv) & 15) == 0) {
                for (int o = 8 * tid; o < WD; o += 8 * PK_THREADS) {
                    const uint4 xk = *reinterpret_cast<const uint4*>(srck + o);
                    const uint4 xv = *reinterpret_cast<const uint4*>(srcv + o);
                    *reinterpret_cast<uint4*>(sk + o) = xk;
                    *reinterpret_cast<uint4*>(sv + o) = xv;
                }
            } else {   // (a caller buffer that is not 16-byte aligned)
                for (int e = tid; e < WD; e += PK_THREADS) {
                    sk[e] = srck[e];
                    sv[e] = srcv[e];
                }
            }
        } else {
            const uint16_t* pg = bf.pages + u * (int64_t)g.n_pages * g.page_elems + (int64_t)pi.src_page * g.page_elems;
            const uint16_t* srck = pg + (int64_t)(2 * h) * WD;
            const uint16_t* srcv = pg + (int64_t)(2 * h + 1) * WD;
            for (int o = 8 * tid; o < WD; o += 8 * PK_THREADS) {
                const uint4 xk = *reinterpret_cast<const uint4*>(srck + o);
                const uint4 xv = *reinterpret_cast<const uint4*>(srcv + o);
                int t, c;
                page_k_pos(o, d, W, t, c);          // 8 consecutive channels of token t
                *reinterpret_cast<uint4*>(sk + t * d + c) = xk;
                page_v_pos(o, d, W, t, c);          // tokens t..t+3 of channels c and c + 16
                const uint32_t w4[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int tj = t + (j & 3), cj = c + 16 * (j >> 2);
                    sv[tj * d + cj] = (uint16_t)(w4[j >> 1] >> (16 * (j & 1)));
                }
            }
        }
        __syncthreads();
        uint8_t* slot = bf.slots + u * (int64_t)g.n_slots * g.slot_bytes + (int64_t)pi.dst_slot * g.slot_bytes +
                        (int64_t)h * g.slot_head_bytes;
        constexpr int qb = QB, P = 8 / qb, L = (1 << qb) - 1, cbytes = W * d * qb / 8;
        // the fp16 parameters, in slot order (offK[d], sclK[d], offV[W], sclV[W]), go to LDS
        // first and to the slot with the codes
        uint16_t* params16 = (uint16_t*)(slot + 2 * cbytes);
        uint16_t* offK = p_bits;
        uint16_t* sclK = offK + d;
        uint16_t* offV = sclK + d;
        uint16_t* sclV = offV + W;
        // keys as quantized: the stored (bf16) values, or in RoPE mode those values turned
        // back to the pre-RoPE domain at their positions (exact products, one rounding)
        auto key_at = [&](int t, int c) -> double {
            if (!rope) return (double)bf16_to_f32(sk[t * d + c]);
            const int i = c < hd ? c : c - hd;
            const float2 cs = bf.rope[(int64_t)(start + t) * hd + i];
            const double a = (double)bf16_to_f32(sk[t * d + i]), bb = (double)bf16_to_f32(sk[t * d + i + hd]);
            return c < hd ? __dadd_rn(__dmul_rn(a, (double)cs.x), __dmul_rn(bb, (double)cs.y))
                          : __dsub_rn(__dmul_rn(bb, (double)cs.x), __dmul_rn(a, (double)cs.y));
        };
        bool bad = false;
        auto set_params = [&](bool key, int gi, double mn, double mx) {
            if (fabs(mn) > 65504.0 || fabs(mx) > 65504.0) bad = true;
            const double off = fp16_round_down(mn);
            const double scl = fp16_round_up((mx - off) / (double)L);
            if (fabs(off) > 65504.0 || scl > 65504.0) bad = true;
            if (key) {
                offK[gi] = fp16_bits_exact(off);
                sclK[gi] = fp16_bits_exact(scl);
            } else {
                offV[lay_vp(gi, W)] = fp16_bits_exact(off);
                sclV[lay_vp(gi, W)] = fp16_bits_exact(scl);
            }
            const int pi_ = key ? gi : d + gi;
            p_off[pi_] = off;
            p_scl[pi_] = scl;
            p_inv[pi_] = scl == 0.0 ? 0.0 : 1.0 / scl;
        };
        // ---- key parameters: KT threads per channel, each over W / KT tokens.  bf16 keys: min
        //      and max in fp32 (exact); RoPE-mode keys are fp64 values
        {
            constexpr int KT = PK_THREADS / d, nt = W / KT;
            const int c = tid / KT, part = tid % KT;
            double mn, mx;
            if (!rope) {
                float fmn = bf16_to_f32(sk[part * nt * d + c]), fmx = fmn;
                for (int i = 1; i < nt; ++i) {
                    const float x = bf16_to_f32(sk[(part * nt + i) * d + c]);
                    fmn = fminf(fmn, x);
                    fmx = fmaxf(fmx, x);
                }
                group_minmax<KT>(fmn, fmx);
                mn = fmn;
                mx = fmx;
            } else {
                mn = key_at(part * nt, c);
                mx = mn;
                for (int i = 1; i < nt; ++i) {
                    const double x = key_at(part * nt + i, c);
                    mn = fmin(mn, x);
                    mx = fmax(mx, x);
                }
                for (int m = 1; m < KT; m <<= 1) {
                    mn = fmin(mn, __shfl_xor(mn, m, 64));
                    mx = fmax(mx, __shfl_xor(mx, m, 64));
                }
            }
            if (part == 0) set_params(true, c, mn, mx);
        }
        // ---- value parameters: VT threads per token, each over d / VT channels (fp32, exact)
        {
            constexpr int VT = PK_THREADS / W, nc = d / VT;
            const int t = tid / VT, part = tid % VT;
            const uint16_t* row = sv + t * d + part * nc;
            float mn = bf16_to_f32(row[0]), mx = mn;
            for (int i = 1; i < nc; ++i) {
                const float x = bf16_to_f32(row[i]);
                mn = fminf(mn, x);
                mx = fmaxf(mx, x);
            }
            group_minmax<VT>(mn, mx);
            if (part == 0) set_params(false, t, mn, mx);
        }
        if (bad) atomicOr(&hdr->status, QEVICT_DEV_E_RANGE);
        __syncthreads();
        // ---- codes, a key byte (P channels of one token) and a value byte (P tokens of one
        //      channel) per thread and round
        for (int B = tid; B < cbytes; B += PK_THREADS) {
            int t, qg, cc0;
            kc_byte_pos(B, d, W, qb, t, qg, cc0);
            uint32_t bk = 0, bv = 0;
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const int c = kc_chan(qg, cc0 + j, d, rope);
                bk |= (uint32_t)nearest_level(2.0 * (key_at(t, c) - p_off[c]), p_scl[c], p_inv[c], L) << (qb * j);
            }
            int t0, c;
            vc_byte_pos(B, d, W, qb, t0, c);
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const int tt = t0 + j;
                const double x = (double)bf16_to_f32(sv[tt * d + c]);
                bv |= (uint32_t)nearest_level(2.0 * (x - p_off[d + tt]), p_scl[d + tt], p_inv[d + tt], L) << (qb * j);
            }
            slot[B] = (uint8_t)bk;
            slot[cbytes + B] = (uint8_t)bv;
        }
        for (int i = tid; i < 2 * (d + W); i += PK_THREADS) params16[i] = p_bits[i];
    }
}

// ------------------------------------------------------------------------------------ fill (promote / copy)
// Promotion writes bf16(off + code*scl), rounded once from the exact fp64 value
// (§4.3: promotion reconstructs the same low-bit approximation in the execution
// datatype).  Prefill copies prompt tokens into pages.  One workgroup per (window, KV
// head) item; the slot comes into LDS by 32-bit loads, and every thread writes whole
// 16-byte runs of the page (8 consecutive elements of its key / value block).
// One fill item: head h of window fi.win of unit u into page fi.dst_page.  All threads call.
template <int W, int d, int QB>
__device__ void fill_item(const Geo& g, const Bufs& bf, int64_t u, int b, const FillItem& fi, int h,
                          const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp, MigSmem& smem) {
    uint32_t* sw = smem.st.sw;
    constexpr int WD = W * d;
    const int tid = threadIdx.x;
    UnitHdr* hdr = bf.hdr + u;
    {
        const int S = hdr->prompt_len;
        if (fi.dst_page < 0) {
            if (tid == 0) atomicOr(&hdr->status, QEVICT_DEV_E_POOL);
            return;
        }
        uint16_t* pg = bf.pages + u * (int64_t)g.n_pages * g.page_elems + (int64_t)fi.dst_page * g.page_elems;
        uint16_t* dk = pg + (int64_t)(2 * h) * WD;
        uint16_t* dv = pg + (int64_t)(2 * h + 1) * WD;
        const int start = g.n_sink + fi.win * W;
        if (fi.src_slot >= 0) {
            const uint8_t* slot = bf.slots + u * (int64_t)g.n_slots * g.slot_bytes +
                                  (int64_t)fi.src_slot * g.slot_bytes + (int64_t)h * g.slot_head_bytes;
            constexpr int qb = QB, mask = (1 << qb) - 1, cbytes = W * d * qb / 8;
            const int nw = (2 * cbytes + 4 * (d + W)) / 4;
            for (int q = tid; q < nw; q += PK_THREADS) sw[q] = reinterpret_cast<const uint32_t*>(slot)[q];
            __syncthreads();
            const uint8_t* sb = reinterpret_cast<const uint8_t*>(sw);
            const uint16_t* offK = reinterpret_cast<const uint16_t*>(sb + 2 * cbytes);
            const uint16_t* sclK = offK + d;
            const uint16_t* offV = sclK + d;
            const uint16_t* sclV = offV + W;
            const bool rope = (g.flags & QEVICT_F_ROPE) != 0;
            constexpr int hd = d / 2;
            auto khat = [&](int i, int c) -> double {   // dequantized key (exact in fp64)
                const int kc = (sb[lay_kc_byte(i, c, d, W, qb, rope)] >> lay_kc_shift(c, qb)) & mask;
                return (double)fp16_bits_to_f32(offK[c]) + kc * (double)fp16_bits_to_f32(sclK[c]);
            };
            for (int vi = tid; vi < 2 * WD / 8; vi += PK_THREADS) {   // key runs, then value runs
                const bool is_v = vi >= WD / 8;
                const int o = 8 * (is_v ? vi - WD / 8 : vi);
                int t, c;
                uint16_t r[8];
                if (!is_v) {
                    page_k_pos(o, d, W, t, c);          // 8 consecutive channels of token t
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int cj = c + j;
                        double kx = khat(t, cj);
                        if (rope) {   // RoPE re-applied at the window's positions, then one bf16 rounding
                            const int pi = cj < hd ? cj : cj - hd;
                            const float2 cs = bf.rope[(int64_t)(start + t) * hd + pi];
                            const double xp = khat(t, cj < hd ? cj + hd : cj - hd);
                            kx = cj < hd ? __dsub_rn(__dmul_rn(kx, (double)cs.x), __dmul_rn(xp, (double)cs.y))
                                         : __dadd_rn(__dmul_rn(kx, (double)cs.x), __dmul_rn(xp, (double)cs.y));
                        }
                        r[j] = f64_to_bf16(kx);
                    }
                } else {
                    page_v_pos(o, d, W, t, c);          // tokens t..t+3 of channels c and c + 16
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int tj = t + (j & 3), cj = c + 16 * (j >> 2);
                        const int vc = (sb[cbytes + lay_vc_byte(tj, cj, d, W, qb)] >> lay_vc_shift(tj, qb)) & mask;
                        const int vpp = lay_vp(tj, W);
                        r[j] = f64_to_bf16((double)fp16_bits_to_f32(offV[vpp]) + vc * (double)fp16_bits_to_f32(sclV[vpp]));
                    }
                }
                *reinterpret_cast<uint4*>((is_v ? dv : dk) + o) =
                    make_uint4((uint32_t)r[0] | ((uint32_t)r[1] << 16), (uint32_t)r[2] | ((uint32_t)r[3] << 16),
                               (uint32_t)r[4] | ((uint32_t)r[5] << 16), (uint32_t)r[6] | ((uint32_t)r[7] << 16));
            }
        } else {   // src_slot -1: the prompt tokens of the window
            const uint16_t* sk = kp + (((int64_t)b * g.h_kv + h) * g.S_max + start) * d;
            const uint16_t* sv = vp + (((int64_t)b * g.h_kv + h) * g.S_max + start) * d;
            int ntok = S - start;
            if (ntok > W) ntok = W;
            for (int o = 8 * tid; o < WD; o += 8 * PK_THREADS) {
                int t, c;
                page_k_pos(o, d, W, t, c);
                uint16_t xk[8], xv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) xk[j] = t < ntok ? sk[t * d + c + j] : (uint16_t)0;
                page_v_pos(o, d, W, t, c);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int tj = t + (j & 3), cj = c + 16 * (j >> 2);
                    xv[j] = tj < ntok ? sv[tj * d + cj] : (uint16_t)0;
                }
                uint32_t pk[4], pv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pk[j] = (uint32_t)xk[2 * j] | ((uint32_t)xk[2 * j + 1] << 16);
                    pv[j] = (uint32_t)xv[2 * j] | ((uint32_t)xv[2 * j + 1] << 16);
                }
                *reinterpret_cast<uint4*>(dk + o) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
                *reinterpret_cast<uint4*>(dv + o) = make_uint4(pv[0], pv[1], pv[2], pv[3]);
            }
        }
    }
}

// The migrations of a routing event in one launch: the pack items, each followed by the fill
// item that reuses its source page at this event (if any: a promotion may take a page that a
// demotion frees, and must write it only after the pack has read it); then the other fill
// items, which touch no page a pack reads.
template <int W, int d, int QB>
__global__ void __launch_bounds__(PK_THREADS) k_migrate(Geo g, Bufs bf, int layer, int n_units,
                                                        const uint16_t* __restrict__ kp,
                                                        const uint16_t* __restrict__ vp) {
    __shared__ MigSmem sm;
    const int tid = threadIdx.x;
    // the list: all pack items (unit by unit), then all fill items; each unit's counts are
    // read once, and both running sums kept in LDS
    {
        constexpr int MAXPER = (MIG_MAX_UNITS + PK_THREADS - 1) / PK_THREADS;
        const int lane = tid & 63, wave = tid >> 6;
        const int per = (n_units + PK_THREADS - 1) / PK_THREADS, u0 = tid * per;
        int cp[MAXPER], cf[MAXPER], sp = 0, sf = 0;
#pragma unroll
        for (int k = 0; k < MAXPER; ++k) {
            cp[k] = cf[k] = 0;
            if (k < per && u0 + k < n_units) {
                int b;
                const UnitHdr* hd = bf.hdr + mig_unit(g, layer, u0 + k, b);
                cp[k] = hd->n_pack * g.h_kv;
                cf[k] = hd->n_fill * g.h_kv;
            }
            sp += cp[k];
            sf += cf[k];
        }
        const int ip = (int)wave_scan_incl((unsigned)sp), jf = (int)wave_scan_incl((unsigned)sf);
        if (lane == 63) {
            sm.wtot[wave] = ip;
            sm.wtot2[wave] = jf;
        }
        __syncthreads();
        int rp = ip - sp, rf = jf - sf;
        for (int q = 0; q < wave; ++q) {
            rp += sm.wtot[q];
            rf += sm.wtot2[q];
        }
#pragma unroll
        for (int k = 0; k < MAXPER; ++k) {
            if (k < per && u0 + k < n_units) {
                sm.pre[u0 + k] = rp;
                sm.pre_f[u0 + k] = rf;
            }
            rp += cp[k];
            rf += cf[k];
        }
        if (tid == PK_THREADS - 1) {
            sm.pre[n_units] = rp;
            sm.pre_f[n_units] = rf;
        }
        __syncthreads();
    }
    const int tp = sm.pre[n_units], tf = sm.pre_f[n_units];
    // (a barrier opens every item but the first: one closing each item would also wait for
    // the item's global stores)
    bool first = true;
    auto open_item = [&]() {
        if (!first) __syncthreads();
        first = false;
    };
    for (int it_all = blockIdx.x; it_all < tp + tf; it_all += gridDim.x) {
        const bool is_pack = it_all < tp;
        const int* pre = is_pack ? sm.pre : sm.pre_f;
        const int ia = is_pack ? it_all : it_all - tp;
        const int ub = mig_find(pre, n_units, ia), it = ia - pre[ub];
        int b;
        const int64_t u = mig_unit(g, layer, ub, b);
        const int h = it % g.h_kv;
        FillItem fi;
        bool do_fill;
        if (is_pack) {
            const PackItem pi = bf.pack[u * g.n_windows + it / g.h_kv];
            open_item();
            pack_item<W, d, QB>(g, bf, u, b, pi, h, kp, vp, sm);
            do_fill = pi.then_fill >= 0;
            if (do_fill) fi = bf.fill[u * g.n_windows + pi.then_fill];
        } else {
            fi = bf.fill[u * g.n_windows + it / g.h_kv];
            do_fill = !fi.after_pack;
        }
        if (do_fill) {
            open_item();   // (after a pack: also, every read of its page is done)
            fill_item<W, d, QB>(g, bf, u, b, fi, h, kp, vp, sm);
        }
    }
}

template <int W, int d, int QB>
static void launch_mig_t(dim3 grid, const Geo& g, const Bufs& bf, int layer, int units, const uint16_t* kp,
                         const uint16_t* vp, hipStream_t s, hipEvent_t ev1) {
    hipExtLaunchKernelGGL((k_migrate<W, d, QB>), grid, dim3(PK_THREADS), 0, s, nullptr, ev1, 0, g, bf, layer, units, kp,
                          vp);
}
template <int W, int d>
static void launch_mig_q(dim3 grid, const Geo& g, const Bufs& bf, int layer, int units, const uint16_t* kp,
                         const uint16_t* vp, hipStream_t s, hipEvent_t ev1) {
    if (g.qbits == 4) launch_mig_t<W, d, 4>(grid, g, bf, layer, units, kp, vp, s, ev1);
    else launch_mig_t<W, d, 2>(grid, g, bf, layer, units, kp, vp, s, ev1);
}
template <int W>
static void launch_mig_d(dim3 grid, const Geo& g, const Bufs& bf, int layer, int units, const uint16_t* kp,
                         const uint16_t* vp, hipStream_t s, hipEvent_t ev1) {
    if (g.d == 64) launch_mig_q<W, 64>(grid, g, bf, layer, units, kp, vp, s, ev1);
    else launch_mig_q<W, 128>(grid, g, bf, layer, units, kp, vp, s, ev1);
}
// (the shapes the configuration accepts: W 16 / 32 / 64, d 64 / 128, 2 / 4 code bits)
static void launch_mig(dim3 grid, const Geo& g, const Bufs& bf, int layer, int units, const uint16_t* kp,
                       const uint16_t* vp, hipStream_t s, hipEvent_t ev1) {
    if (g.W == 16) launch_mig_d<16>(grid, g, bf, layer, units, kp, vp, s, ev1);
    else if (g.W == 32) launch_mig_d<32>(grid, g, bf, layer, units, kp, vp, s, ev1);
    else launch_mig_d<64>(grid, g, bf, layer, units, kp, vp, s, ev1);
}

// Routing (every unit of the layer, or of all layers with layer = -1) and the migrations it
// decides: k_route (which also writes the new list's split blocks), then k_migrate (packs and fills).
hipError_t launch_route(const Geo& g, const Bufs& bf, int layer, int mode, const uint16_t* kp, const uint16_t* vp,
                        hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    const int units = layer >= 0 ? g.B : g.B * g.L;
    if (units > MIG_MAX_UNITS || g.n_windows > rt1024::RT_MAXW) return hipErrorInvalidValue;
    // units of at most 1024 windows: 256-thread workgroups, eight per CU instead of two
    if (g.n_windows <= rt256::RT_MAXW)
        hipExtLaunchKernelGGL(rt256::k_route, dim3(units), dim3(rt256::RT_THREADS), sizeof(rt256::RouteSmem), s, ev0,
                              nullptr, 0, g, bf, layer, mode);
    else
        hipExtLaunchKernelGGL(rt1024::k_route, dim3(units), dim3(rt1024::RT_THREADS), sizeof(rt1024::RouteSmem), s,
                              ev0, nullptr, 0, g, bf, layer, mode);
    // workgroups: a prefill (one layer, every prompt window) spreads its items over 1024;
    // a routing event moves a few windows per unit
    const int nb = layer >= 0 ? 1024 : std::min(1024, std::max(256, 8 * units));
    launch_mig(dim3(nb), g, bf, layer, units, kp, vp, s, ev1);
    return hipGetLastError();
}

}  // namespace qv
