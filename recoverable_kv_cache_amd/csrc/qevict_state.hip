// State kernels: arena initialisation, prefill setup, the
// window router (candidate pool + two-stage TopK + migration bookkeeping +
// chronological compaction) and the INT2 pack / dequantize-promote kernels.
//
// Source: "QEvict: Recoverable Quantized KV Eviction for Attention-Drift-Robust
// Long-Context Decoding", §4.3 (Eq. 3 capacities, "Migration-Stable
// Quantization", Eqs. 4-6), Appendix A Algorithm 1.
#include "qevict_common.h"
#include "qevict_internal.h"
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
constexpr int RT_THREADS = 1024;
constexpr int RT_MAXW = 4096;           // windows per unit handled by one workgroup
constexpr int RT_PER = RT_MAXW / RT_THREADS;

// Sum over the 64 lanes of a wave (every lane gets it) with DPP moves and the gfx950 row
// swaps: no LDS traffic.  Every DPP pattern reads a lane of the same row, so bound_ctrl
// changes no value.
__device__ __forceinline__ int wave_sum_i32(int x) {
    x += __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);    // quad [1,0,3,2]
    x += __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);    // quad [2,3,0,1]
    x += __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);   // row_half_mirror
    x += __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true);   // row_mirror
    const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    x = (int)(a[0] + a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return (int)(c[0] + c[1]);
}

// Exclusive scan of a[0..RT_MAXW) in LDS; returns the total.  All threads call.  Two counts
// may share an element as 16-bit fields (lo + (hi << 16)): the fields add independently
// while each total stays below 2^16 (at most RT_MAXW here).
__device__ int block_scan_excl(int* a, int* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int v[RT_PER];
    int s = 0;
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) {
        v[i] = a[tid * RT_PER + i];
        s += v[i];
    }
    int incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    if (wave == 0) {     // exclusive scan of the wave totals by the first wave
        constexpr int NWV = RT_THREADS / 64;
        const int t = lane < NWV ? wsum[lane] : 0;
        int inc = t;
#pragma unroll
        for (int o = 1; o < NWV; o <<= 1) {
            const int y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        if (lane < NWV) wsum[lane] = inc - t;
        if (lane == NWV - 1) wsum[NWV] = inc;
    }
    __syncthreads();
    int run = wsum[wave] + incl - s;
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) {
        a[tid * RT_PER + i] = run;
        run += v[i];
    }
    const int total = wsum[RT_THREADS / 64];
    __syncthreads();
    return total;
}

struct RouteSmem {
    unsigned long long work[RT_MAXW];   // scratch: key-norm sums, tier selection, then flag arrays
    int idx[RT_MAXW];
    int8_t newst[RT_MAXW];
    int wsum[RT_THREADS / 64 + 1];
    int misc[8];
};

// Bytes one accessible entry makes the decode kernel read per KV head; splits are
// balanced on them.  (Weighting bf16 pages by their compute time instead, which is
// only ~2.3x that of an INT2 window against ~6x the bytes, measured slower: with the
// cache streamed from HBM the page loads dominate.)
__device__ __forceinline__ int per_head_cost(const Geo& g, int kind) {
    if (kind == EK_SINK) return 4 * g.n_sink * g.d;
    if (kind == EK_PAGE) return 4 * g.W * g.d;
    return g.slot_head_bytes;
}

// Total order of doubles as unsigned integers, ascending; -0 counts as +0 (so equal
// scores tie and fall to the window index).  Rank keys of every ranker, negative ones
// (key-norm) included.
__device__ inline unsigned long long ord_key(double s) {
    const unsigned long long bits = (unsigned long long)__double_as_longlong(s + 0.0);
    return (bits >> 63) ? ~bits : (bits | (1ull << 63));
}
// ---------------------------------------------------------------- tier selection (Eq. 5)
// Only tier membership matters: Full = the K_f first candidates in rank order (score
// descending, window index ascending), Quantized = the next K_q.  Each candidate has the
// composite key C = (~ord_key(score) << 12) | window, distinct and ascending in rank order;
// a tier boundary is the composite of rank k (the k-th smallest).  It is found by radix
// selection: 11-bit digits of C from the top; per pass a digit histogram of the candidates
// that share the prefix found so far (LDS atomics), then the bin holding rank k (every
// thread takes two bins; block prefix sum) extends the prefix.  Once that bin holds at most
// 64 candidates they are gathered and one wave ranks them exactly.  Two selections (member
// sets and ranks) run side by side.  The loop state is block-uniform and kept in scalar
// registers.
using u128 = unsigned __int128;
constexpr int SEL_BITS = 76;             // 64 key bits + 12 window bits (RT_MAXW = 4096)
constexpr int SEL_D = 11, SEL_BINS = 1 << SEL_D, SEL_FIN = 64;
constexpr int SEL_PASSES = (SEL_BITS + SEL_D - 1) / SEL_D;
constexpr int RT_WAVES = RT_THREADS / 64;
static_assert(RT_MAXW <= 4096, "window index must fit the 12 low bits of the composite key");
static_assert(SEL_BINS == 2 * RT_THREADS, "the bin search takes two bins per thread");

struct SelSmem {
    int wtot[2][RT_WAVES];                 // per-wave totals (counts, then bin sums)
    unsigned hist[2][SEL_BINS];
    unsigned long long gk_hi[2][SEL_FIN], gk_lo[2][SEL_FIN];   // gathered composites
    unsigned long long t_hi[2], t_lo[2];   // the rank-k composites
    int bin[2], cnt[2], rem[2], gcnt[2];
};
enum { SEL_NONE = 0, SEL_ALL = 1, SEL_THR = 2, SEL_SEARCH = 3, SEL_GATHER = 4 };

__device__ __forceinline__ u128 sel_composite(double s, int w) {
    return ((u128)~ord_key(s) << 12) | (u128)(unsigned)w;
}
// top p bits of c (p in [0, SEL_BITS])
__device__ __forceinline__ u128 sel_prefix(u128 c, int p) { return p == 0 ? (u128)0 : c >> (SEL_BITS - p); }
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

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
// sum of a[0..RT_WAVES) and of its first `upto` entries (LDS, 16-byte aligned)
__device__ __forceinline__ void wave_totals(const int* a, int upto, int& all, int& before) {
    all = 0;
    before = 0;
#pragma unroll
    for (int q = 0; q < RT_WAVES; q += 4) {
        const int4 x = *reinterpret_cast<const int4*>(a + q);
        all += x.x + x.y + x.z + x.w;
        before += (q < upto ? x.x : 0) + (q + 1 < upto ? x.y : 0) + (q + 2 < upto ? x.z : 0) + (q + 3 < upto ? x.w : 0);
    }
}

// For each target t in {0, 1}: members mem[t] (bit e: element e of this thread), rank k[t].
// On return in[t] bit e says that element e is a member of rank <= k[t] among the members.
// Every pass adds SEL_D bits to the prefix, so at most SEL_PASSES passes run; false (and no
// element selected) if a selection were still open after them, which the invariants exclude.
// All threads call; ss aliases free LDS.
__device__ bool select_two(const u128 (&c)[RT_PER], const int (&mem)[2], const int (&k)[2], int (&in)[2],
                           SelSmem& ss) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int st[2], p[2] = {0, 0}, rem[2] = {k[0], k[1]};
    u128 pv[2] = {0, 0}, thr[2] = {0, 0};
    {   // member counts (two 16-bit fields: at most RT_MAXW each)
        const int v = wave_sum_i32(__popc(mem[0]) | (__popc(mem[1]) << 16));
        if (lane == 0) ss.wtot[0][wave] = v;
        if (tid < 2) ss.gcnt[tid] = 0;
        __syncthreads();
        int tot, unused;
        wave_totals(ss.wtot[0], 0, tot, unused);
        tot = uni(tot);
        const int n[2] = {tot & 0xFFFF, tot >> 16};
#pragma unroll
        for (int t = 0; t < 2; ++t) st[t] = k[t] <= 0 ? SEL_NONE : (k[t] >= n[t] ? SEL_ALL : SEL_SEARCH);
    }
    bool ok = true;
    for (int pass = 0;; ++pass) {
        if (st[0] != SEL_SEARCH && st[1] != SEL_SEARCH) break;
        if (pass == SEL_PASSES) {
            ok = false;
            st[0] = st[1] = SEL_NONE;
            break;
        }
        for (int i = tid; i < 2 * SEL_BINS; i += RT_THREADS) (&ss.hist[0][0])[i] = 0;
        __syncthreads();
        // histogram of the next digit over the members that share the prefix
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (st[t] != SEL_SEARCH) continue;
            const int dd = min(SEL_D, SEL_BITS - p[t]), sh = SEL_BITS - p[t] - dd;
#pragma unroll
            for (int e = 0; e < RT_PER; ++e)
                if (((mem[t] >> e) & 1) && sel_prefix(c[e], p[t]) == pv[t])
                    atomicAdd(&ss.hist[t][(unsigned)(c[e] >> sh) & ((1u << dd) - 1)], 1u);
        }
        __syncthreads();
        // the bin of rank rem: bins 2 tid and 2 tid + 1 on thread tid, block prefix sum
        unsigned h0[2], h1[2], incl[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (st[t] != SEL_SEARCH) continue;
            const uint2 hh = *reinterpret_cast<const uint2*>(&ss.hist[t][2 * tid]);
            h0[t] = hh.x;
            h1[t] = hh.y;
            incl[t] = wave_scan_incl(hh.x + hh.y);
            if (lane == 63) ss.wtot[t][wave] = (int)incl[t];
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (st[t] != SEL_SEARCH) continue;
            int all, wp;
            wave_totals(ss.wtot[t], wave, all, wp);
            const unsigned r = (unsigned)rem[t];
            const unsigned before = (unsigned)wp + incl[t] - h0[t] - h1[t];
            if (before < r && r <= (unsigned)wp + incl[t]) {      // exactly one thread
                const bool first = before + h0[t] >= r;
                ss.bin[t] = 2 * tid + (first ? 0 : 1);
                ss.cnt[t] = (int)(first ? h0[t] : h1[t]);
                ss.rem[t] = (int)(r - (first ? before : before + h0[t]));
            }
        }
        __syncthreads();
        bool gather = false;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (st[t] != SEL_SEARCH) continue;
            const int dd = min(SEL_D, SEL_BITS - p[t]);
            pv[t] = (pv[t] << dd) | (u128)(unsigned)uni(ss.bin[t]);
            p[t] += dd;
            rem[t] = uni(ss.rem[t]);
            if (uni(ss.cnt[t]) <= SEL_FIN || p[t] == SEL_BITS) {
                st[t] = SEL_GATHER;
                gather = true;
            }
        }
        if (!gather) continue;
        // gather the at most SEL_FIN members of the final bin, then rank them in one wave
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (st[t] != SEL_GATHER) continue;
#pragma unroll
            for (int e = 0; e < RT_PER; ++e)
                if (((mem[t] >> e) & 1) && sel_prefix(c[e], p[t]) == pv[t]) {
                    const int at = atomicAdd(&ss.gcnt[t], 1);
                    if (at < SEL_FIN) {     // (always: the bin holds at most SEL_FIN members)
                        ss.gk_hi[t][at] = (unsigned long long)(c[e] >> 64);
                        ss.gk_lo[t][at] = (unsigned long long)c[e];
                    }
                }
        }
        __syncthreads();
        if (wave < 2 && st[wave] == SEL_GATHER) {
            const int t = wave, m = min(ss.gcnt[t], SEL_FIN);
            if (lane < m) {
                const u128 mine = ((u128)ss.gk_hi[t][lane] << 64) | ss.gk_lo[t][lane];
                int r = 0;
                for (int j = 0; j < m; ++j) r += (((u128)ss.gk_hi[t][j] << 64) | ss.gk_lo[t][j]) < mine;
                if (r == rem[t] - 1) {
                    ss.t_hi[t] = ss.gk_hi[t][lane];
                    ss.t_lo[t] = ss.gk_lo[t][lane];
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 2; ++t)
            if (st[t] == SEL_GATHER) {
                thr[t] = ((u128)ss.t_hi[t] << 64) | ss.t_lo[t];
                st[t] = SEL_THR;
            }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        int bits = 0;
#pragma unroll
        for (int e = 0; e < RT_PER; ++e)
            if (((mem[t] >> e) & 1) && (st[t] == SEL_ALL || (st[t] == SEL_THR && c[e] <= thr[t]))) bits |= 1 << e;
        in[t] = bits;
    }
    __syncthreads();   // (ss may be reused)
    return ok;
}

// One workgroup per (sequence, layer).
__global__ void __launch_bounds__(RT_THREADS) k_route(Geo g, Bufs bf, int layer, int mode) {
    extern __shared__ unsigned char smem_raw[];
    RouteSmem& sm = *reinterpret_cast<RouteSmem*>(smem_raw);
    const int tid = threadIdx.x;
    const int b = layer >= 0 ? blockIdx.x : blockIdx.x / g.L;
    const int l = layer >= 0 ? layer : blockIdx.x % g.L;
    const int64_t u = unit_of(g, b, l);
    UnitHdr* hdr = bf.hdr + u;
    WinRec* win = bf.win + u * g.n_windows;
    double* score = bf.score + u * g.n_windows;
    int8_t* target = bf.target + u * g.n_windows;
    const int n = hdr->n;
    const int K_f = hdr->K_f, K_q = hdr->K_q;
    const int NW = g.n_windows;
    int* flag = (int*)sm.work;               // (used after the tier selection)

    // ---- 0. the last decode step's window-mass shares entered the scores in k_route_fold
    if (tid == 0 && hdr->mass_pending) hdr->mass_pending = 0;
    // ---- 0b. decay / p-norm rankers (Appendix J, Eqs. 22-23): at each decode-time routing
    //          event the interval's mass enters the rank key and starts again from 0
    if (mode == RM_ROUTE && rank_interval(g)) {
        double* ua = bf.uacc + u * g.n_windows;
        for (int w = tid; w < NW; w += RT_THREADS) {
            const double x = ua[w];
            score[w] = (g.flags & QEVICT_F_RANK_DECAY) ? __dadd_rn(__dmul_rn(RANK_DECAY_LAMBDA, score[w]), x)
                                                       : __dadd_rn(score[w], __dmul_rn(__dmul_rn(x, x), x));
            ua[w] = 0.0;
        }
        __syncthreads();
    }
    // ---- 0c. key-norm ranker (Eq. 24): each recent window that ages at this event gets
    //          its rank key from the keys in its page (prompt windows got theirs at prefill)
    if (mode == RM_ROUTE && (g.flags & QEVICT_F_RANK_KEYNORM)) {
        int* list = sm.idx;                          // (scratch before the sort)
        double* tokn = reinterpret_cast<double*>(sm.work);
        if (tid == 0) sm.misc[0] = 0;
        __syncthreads();
        for (int w = tid; w < NW; w += RT_THREADS)
            if (win[w].state == ST_LOCAL && g.n_sink + (w + 1) * g.W <= n - g.n_local) list[atomicAdd(&sm.misc[0], 1)] = w;
        __syncthreads();
        const int nl = sm.misc[0];
        for (int k = 0; k < nl; ++k) {
            const int w = list[k];
            if (win[w].page < 0) continue;           // (a recent window always has its page)
            const uint16_t* pg = bf.pages + u * (int64_t)g.n_pages * g.page_elems + (int64_t)win[w].page * g.page_elems;
            const double r = key_norm_block(g, g.W, [&](int i, int hk, int c) {
                return __uint_as_float((uint32_t)pg[(int64_t)(2 * hk) * g.W * g.d + lay_k(i, c, g.d, g.W)] << 16);
            }, tokn);
            if (tid == 0) score[w] = r;
        }
        __syncthreads();
    }

    // the window records of this thread's windows w = tid + i * RT_THREADS, read once
    WinRec rec[RT_PER];
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) {
        const int w = tid + i * RT_THREADS;
        rec[i] = w < NW ? win[w] : WinRec{ST_NONE, -1, -1, 0};
    }
    // ---- 1. candidate pool (Eq. 4): previous Full ∪ previous Quantized ∪ aged recent windows
    int candm = 0;               // bit i: window tid + i * RT_THREADS is a candidate
    u128 ckey[RT_PER];
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) {
        const int w = tid + i * RT_THREADS;
        int c = 0;
        if (w < NW) {
            const int st = rec[i].state;
            const bool aged = g.n_sink + (w + 1) * g.W <= n - g.n_local;
            if (mode == RM_ROUTE || mode == RM_PREFILL)
                c = (st == ST_FULL || st == ST_QUANT || ((st == ST_LOCAL || st == ST_PROMPT) && aged));
            else if (mode == RM_FORCE_Q)
                c = target[w] != 0 && (st == ST_FULL || (st == ST_LOCAL && aged));
            else
                c = target[w] != 0 && st == ST_QUANT;
        }
        candm |= c << i;
        ckey[i] = sel_composite(c && (mode == RM_ROUTE || mode == RM_PREFILL) ? score[w] : 0.0, w);
    }
    // ---- 2. tiers of the candidates (Eq. 5): Full = rank <= K_f, Quantized = the next K_q
    const bool one_way = (g.flags & QEVICT_F_NO_PROMOTE) != 0;
    int isF = 0, isQ = 0;
    if (mode == RM_ROUTE || mode == RM_PREFILL) {
        static_assert(sizeof(SelSmem) <= sizeof(RouteSmem::work), "selection scratch");
        SelSmem& ss = *reinterpret_cast<SelSmem*>(sm.work);
        int in[2];
        bool sel_ok;
        if (!one_way) {
            const int mem[2] = {candm, candm}, kk[2] = {K_f, K_f + K_q};
            sel_ok = select_two(ckey, mem, kk, in, ss);
            isF = in[0];
            isQ = in[1] & ~in[0];
        } else {
            // one-way: Full = the best K_f candidates that are not Quantized before the event;
            // Quantized = the next K_q of all other candidates, in the same order
            int notq = 0;
#pragma unroll
            for (int i = 0; i < RT_PER; ++i) notq |= (rec[i].state != ST_QUANT) << i;
            const int mem[2] = {candm & notq, 0}, kk[2] = {K_f, 0};
            sel_ok = select_two(ckey, mem, kk, in, ss);
            isF = in[0];
            const int mem2[2] = {candm & ~isF, 0}, kk2[2] = {K_q, 0};
            sel_ok = select_two(ckey, mem2, kk2, in, ss) && sel_ok;
            isQ = in[0];
        }
        if (!sel_ok && tid == 0) atomicOr(&hdr->status, QEVICT_DEV_E_SELECT);
    }
    // ---- 3. new state of every window
    const int forced_st = mode == RM_FORCE_Q ? ST_QUANT : ST_FULL;
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) {
        const int w = tid + i * RT_THREADS;
        int ns = ST_NONE;
        if (w < NW) {
            const int st = rec[i].state;
            ns = st;
            if (st == ST_PROMPT) ns = ST_LOCAL;  // non-aged prompt windows enter the recent region
            if (st == ST_NONE && g.n_sink + w * g.W < n + g.omega) ns = ST_LOCAL;   // prepare
            if ((candm >> i) & 1) {
                if (mode == RM_ROUTE || mode == RM_PREFILL)
                    ns = ((isF >> i) & 1) ? ST_FULL : (((isQ >> i) & 1) ? ST_QUANT : ST_EVICTED);
                else
                    ns = forced_st;
            }
        }
        sm.newst[w] = (int8_t)ns;
    }
    __syncthreads();

    // ---- 4. migration actions (Algorithm 1 steps 5-20).  Per window:
    // bit0 free page, bit1 need page, bit2 free slot, bit3 need slot, bit4 pack, bit5 fill
    int act[RT_PER];
    int ctr[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) {
        const int w = tid + i * RT_THREADS;
        int a = 0;
        if (w < NW) {
            const WinRec r = rec[i];
            const int os = r.state, ns = sm.newst[w];
            const bool cand = (candm >> i) & 1;
            if (cand && (os == ST_LOCAL || os == ST_PROMPT)) ctr[C_AGED]++;
            if (os == ST_LOCAL || os == ST_FULL) {
                if (ns == ST_QUANT) {
                    a |= 1;
                    if (r.flags & WF_LEDGER) ctr[C_REACTIVATED]++;
                    else { a |= 8 | 16; ctr[C_PACKED]++; }
                    ctr[C_DEMOTED]++;
                } else if (ns == ST_EVICTED) {
                    a |= 1;
                    if (r.flags & WF_LEDGER) a |= 4;
                    ctr[C_EVICTED]++;
                }
            } else if (os == ST_QUANT) {
                if (ns == ST_FULL) { a |= 2 | 32; ctr[C_PROMOTED]++; }
                else if (ns == ST_EVICTED) { a |= 4; ctr[C_EVICTED]++; }
            } else if (os == ST_PROMPT) {
                if (ns == ST_FULL || ns == ST_LOCAL) a |= 2 | 32;
                else if (ns == ST_QUANT) { a |= 8 | 16; ctr[C_PACKED]++; ctr[C_DEMOTED]++; }
                else if (ns == ST_EVICTED) ctr[C_EVICTED]++;
            } else if (os == ST_NONE && ns == ST_LOCAL) {
                a |= 2 | 32;          // fresh recent-region page, zero-filled
            }
            if (ns == ST_FULL) ctr[C_NFULL]++;
            if (ns == ST_QUANT) ctr[C_NQUANT]++;
        }
        act[i] = a;
    }
    // counters: block reduction through LDS atomics
    if (tid < 8) sm.misc[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 8; c += 2) {  // wave sums first (two counters per word, 16-bit fields:
                                      // a wave's count is at most 4 * 64), one LDS atomic per wave
        const int v = wave_sum_i32(ctr[c] | (ctr[c + 1] << 16));
        if ((tid & 63) == 0 && v) {
            atomicAdd(&sm.misc[c], v & 0xFFFF);
            atomicAdd(&sm.misc[c + 1], v >> 16);
        }
    }
    __syncthreads();
    if (tid < 8) hdr->ctr[tid] = sm.misc[tid];

    // ---- 5. slot allocation: push freed slots, then pop for new packs
    int32_t* fslot = bf.free_slots + u * g.n_slots;
    int32_t* fpage = bf.free_pages + u * g.n_pages;
    int nslot_free0 = hdr->n_free_slots, npage_free0 = hdr->n_free_pages;
    int my_slot[RT_PER], my_page[RT_PER];
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) {
        const int w = tid + i * RT_THREADS;
        my_slot[i] = w < NW ? rec[i].slot : -1;
        my_page[i] = w < NW ? rec[i].page : -1;
    }
    __syncthreads();
    int* pushed = sm.idx;     // ids pushed at this event, by stack position - cnt0 (sm.idx is free after step 3)
    for (int pass = 0; pass < 2; ++pass) {      // pass 0: slots, pass 1: pages
        const int fbit = pass == 0 ? 4 : 1, nbit = pass == 0 ? 8 : 2;
        int32_t* stack = pass == 0 ? fslot : fpage;
        const int cap = pass == 0 ? g.n_slots : g.n_pages;
        const int cnt0 = pass == 0 ? nslot_free0 : npage_free0;
        // one scan for both counts: freed ids (low field) and needed ids (high field)
#pragma unroll
        for (int i = 0; i < RT_PER; ++i)
            flag[tid + i * RT_THREADS] = ((act[i] & fbit) ? 1 : 0) | ((act[i] & nbit) ? 0x10000 : 0);
        __syncthreads();
        const int tot = block_scan_excl(flag, sm.wsum);
        const int n_freed = tot & 0xFFFF, n_need = tot >> 16;
#pragma unroll
        for (int i = 0; i < RT_PER; ++i) {
            if (act[i] & fbit) {
                const int pos = cnt0 + (flag[tid + i * RT_THREADS] & 0xFFFF);
                const int id = pass == 0 ? my_slot[i] : my_page[i];
                if (pos < cap && id >= 0) stack[pos] = id;
                pushed[pos - cnt0] = id;
                if (pass == 0) my_slot[i] = -1;
                else my_page[i] = -1;
            }
        }
        __syncthreads();
        const int avail = min(cnt0 + n_freed, cap);
#pragma unroll
        for (int i = 0; i < RT_PER; ++i) {
            if (act[i] & nbit) {
                const int k = flag[tid + i * RT_THREADS] >> 16;
                const int at = avail - 1 - k;
                const int id = k >= avail ? -1 : (at >= cnt0 ? pushed[at - cnt0] : stack[at]);
                if (pass == 0) my_slot[i] = id;
                else my_page[i] = id;
            }
        }
        if (tid == 0) {
            int left = avail - n_need;
            if (left < 0) {
                atomicOr(&hdr->status, QEVICT_DEV_E_POOL);
                left = 0;
            }
            if (pass == 0) hdr->n_free_slots = left;
            else hdr->n_free_pages = left;
        }
        __syncthreads();
    }

    // ---- 6. work lists: pack (quantize once) and fill (promote / copy prompt)
#pragma unroll
    for (int i = 0; i < RT_PER; ++i)   // pack count (low field), fill count (high field)
        flag[tid + i * RT_THREADS] = ((act[i] & 16) ? 1 : 0) | ((act[i] & 32) ? 0x10000 : 0);
    __syncthreads();
    const int tot_pf = block_scan_excl(flag, sm.wsum);
    const int n_pack = tot_pf & 0xFFFF, n_fill = tot_pf >> 16;
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) {
        const int w = tid + i * RT_THREADS;
        if (w >= NW) continue;
        const WinRec r = rec[i];
        if (act[i] & 16) {
            PackItem it;
            it.win = w;
            it.src_prompt = r.state == ST_PROMPT ? 1 : 0;
            it.src_page = r.page;
            it.dst_slot = my_slot[i];
            bf.pack[u * g.n_windows + (flag[w] & 0xFFFF)] = it;
        }
        if (act[i] & 32) {
            FillItem it;
            it.win = w;
            it.dst_page = my_page[i];
            it.src_slot = r.state == ST_QUANT ? r.slot : (r.state == ST_PROMPT ? -1 : -2);
            it.pad = 0;
            bf.fill[u * g.n_windows + (flag[w] >> 16)] = it;
        }
    }
    if (tid == 0) {
        hdr->n_pack = n_pack;
        hdr->n_fill = n_fill;
    }
    __syncthreads();
    // ---- 7. commit the new window records
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) {
        const int w = tid + i * RT_THREADS;
        if (w >= NW) continue;
        WinRec r = rec[i];
        const int ns = sm.newst[w];
        int flags = r.flags;
        if (ns == ST_EVICTED) flags = 0;
        else if (r.state == ST_QUANT && ns == ST_FULL) flags |= WF_DORMANT;
        else if (ns == ST_QUANT) flags = WF_LEDGER;           // new or reactivated record is active
        r.state = ns;
        r.flags = flags;
        r.slot = (ns == ST_QUANT || (flags & WF_LEDGER)) ? my_slot[i] : -1;
        r.page = (ns == ST_FULL || ns == ST_LOCAL) ? my_page[i] : -1;
        win[w] = r;
        if (mode == RM_FORCE_Q || mode == RM_FORCE_F) target[w] = 0;
    }
    __syncthreads();
    // ---- 8. accessible list (Algorithm 1 step 21) and byte-balanced splits.  The bf16
    //      pages and the Quantized slots, each in chronological order, are merged so that
    //      the pages fall evenly among the slots (by rank fraction, (2r + 1) / 2count, pages
    //      first on ties): every byte-balanced split then holds a like share of both kinds,
    //      whose costs per byte differ.  Attention does not depend on the order.
    for (int w = tid; w < RT_MAXW; w += RT_THREADS) {   // page (low field), slot (high field)
        const int ns = w < NW ? sm.newst[w] : ST_NONE;
        flag[w] = ((ns == ST_LOCAL || ns == ST_FULL) ? 1 : 0) | (ns == ST_QUANT ? 0x10000 : 0);
    }
    __syncthreads();
    const int tot_ps = block_scan_excl(flag, sm.wsum);   // flag[w]: rank among the pages / the slots
    const int n_pg = tot_ps & 0xFFFF, n_sl = tot_ps >> 16;
    auto list_pos = [&](int w, bool page) -> int {   // (counts <= RT_MAXW: 32-bit products)
        const int P = n_pg, S = n_sl;
        if (page) {
            const int r = flag[w] & 0xFFFF, X = (2 * r + 1) * S - P;   // slots strictly before
            const int c = X > 0 ? (int)(((unsigned)X + 2u * P - 1u) / (2u * P)) : 0;
            return r + (c < S ? c : S);
        }
        const int r = flag[w] >> 16, Y = (2 * r + 1) * P - S;   // pages before or tied
        const int c = Y >= 0 ? (int)((unsigned)Y / (2u * S)) + 1 : 0;
        return r + (c < P ? c : P);
    };
    const int n_winacc = n_pg + n_sl;
    const int base = 1;   // entry 0 is the sink prefix
    int n_acc = base + n_winacc;
    if (n_acc > g.n_acc_max) {
        if (tid == 0) atomicOr(&hdr->status, QEVICT_DEV_E_LIST);
        n_acc = g.n_acc_max;
    }
    AccEntry* acc = bf.acc + u * g.n_acc_max;
    int* cost = sm.idx;
    for (int e = tid; e < RT_MAXW; e += RT_THREADS) cost[e] = 0;
    __syncthreads();
    if (tid == 0) {
        acc[0] = AccEntry{EK_SINK, 0, -1, 0};
        cost[0] = per_head_cost(g, EK_SINK);
    }
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) {
        const int w = tid + i * RT_THREADS;
        if (w >= NW) continue;
        const int ns = sm.newst[w];
        if (!(ns == ST_LOCAL || ns == ST_FULL || ns == ST_QUANT)) continue;
        const int e = base + list_pos(w, ns != ST_QUANT);
        if (e >= n_acc) continue;
        AccEntry en;
        en.kind = ns == ST_QUANT ? EK_SLOT : EK_PAGE;
        en.idx = ns == ST_QUANT ? my_slot[i] : my_page[i];
        en.win = w;
        en.start = g.n_sink + w * g.W;
        acc[e] = en;
        cost[e] = per_head_cost(g, en.kind);
    }
    __syncthreads();
    const int total = block_scan_excl(cost, sm.wsum);   // cost[e] = bytes before entry e
    int32_t* splits = bf.splits + u * (g.n_splits + 1);
    for (int s = tid; s <= g.n_splits; s += RT_THREADS) {
        int pos;
        if (s == 0) pos = 0;
        else if (s == g.n_splits) pos = n_acc;
        else {
            const long long tgt = (long long)total * s / g.n_splits;
            int lo = 0, hi = n_acc;       // first e with cost[e] >= tgt
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (cost[mid] < tgt) lo = mid + 1;
                else hi = mid;
            }
            pos = lo;
        }
        splits[s] = pos;
    }
    // (the split blocks are copied by k_split_blocks)
    if (tid == 0) {
        hdr->n_acc = n_acc;
        int nwin = 0;
        const int lim = n + g.omega - g.n_sink;
        if (lim > 0) nwin = (lim + g.W - 1) / g.W;
        hdr->n_win = nwin < NW ? nwin : NW;
        const int lastprep = nwin;
        if (lastprep > NW) atomicOr(&hdr->status, QEVICT_DEV_E_LIST);
    }
}

// The last decode step's pending window-mass shares, folded into the scores before routing:
// one thread per accessible entry, spread over many workgroups (a single workgroup would take
// microseconds to bring in one unit's log-sum-exp rows).  k_route then clears the flag.
__global__ void __launch_bounds__(256) k_route_fold(Geo g, Bufs bf, int layer) {
    const int ub = blockIdx.y;
    const int b = layer >= 0 ? ub : ub / g.L;
    const int l = layer >= 0 ? layer : ub % g.L;
    const int64_t u = unit_of(g, b, l);
    const UnitHdr* hdr = bf.hdr + u;
    if (!hdr->mass_pending) return;
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    const int n_acc = hdr->n_acc;
    apply_mass_range(g, bf, u, hdr->n - 1, e, e < n_acc ? e + 1 : e, 1);   // the step at position n - 1
}

// Each split's block: header {entries, first entry, -1, 0} and its first SPLIT_BLOCK - 1
// accessible-list entries, copied after k_route has rebuilt the list and the split offsets.
__global__ void __launch_bounds__(SPLIT_BLOCK) k_split_blocks(Geo g, Bufs bf, int layer) {
    const int ub = blockIdx.y;
    const int b = layer >= 0 ? ub : ub / g.L;
    const int l = layer >= 0 ? layer : ub % g.L;
    const int64_t u = unit_of(g, b, l);
    const int s = blockIdx.x, x = threadIdx.x;
    const int32_t* splits = bf.splits + u * (g.n_splits + 1);
    const int e0 = splits[s], cnt = splits[s + 1] - e0;
    AccEntry v = AccEntry{EK_PAGE, -1, -1, 0};
    if (x == 0) v = AccEntry{cnt, e0, -1, 0};
    else if (x - 1 < cnt) v = bf.acc[u * g.n_acc_max + e0 + x - 1];
    bf.split_blk[(u * g.n_splits + s) * SPLIT_BLOCK + x] = v;
}

hipError_t launch_route(const Geo& g, const Bufs& bf, int layer, int mode, hipStream_t s) {
    const int units = layer >= 0 ? g.B : g.B * g.L;
    hipLaunchKernelGGL(k_route_fold, dim3((g.n_acc_max + 255) / 256, units), dim3(256), 0, s, g, bf, layer);
    const size_t smem = sizeof(RouteSmem);
    hipLaunchKernelGGL(k_route, dim3(units), dim3(RT_THREADS), smem, s, g, bf, layer, mode);
    hipLaunchKernelGGL(k_split_blocks, dim3(g.n_splits, units), dim3(SPLIT_BLOCK), 0, s, g, bf, layer);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------ pack (INT2 / INT4, once)
// Keys: per (head, channel) over the window's tokens; values: per (head, token)
// over channels.  With L = 2^b - 1 levels (b = 2, or 4 for the INT4 tier):
// off = RD_fp16(min), scl = RU_fp16((max - off)/L), code =
// #{k in 1..L : 2(x - off) >= (2k-1) scl}, 0 when scl == 0.  All comparisons in
// fp64, where they are exact for bf16 x and fp16 off/scl.
constexpr int PK_THREADS = 256;
constexpr int PK_MAXE = 64 * 128;   // W * d

// #{k in 1..L : t >= (2k - 1) scl} for t = 2(x - off) >= 0: the nearest of the levels
// 0..L, ties up.  A quotient gives the estimate; exact fp64 comparisons with the
// thresholds on either side settle it.
__device__ inline int nearest_level(double t, double scl, int L) {
    if (scl == 0.0) return 0;
    int k = (int)floor((t / scl + 1.0) * 0.5);
    k = k < 0 ? 0 : (k > L ? L : k);
    while (k < L && t >= (double)(2 * k + 1) * scl) ++k;
    while (k > 0 && t < (double)(2 * k - 1) * scl) --k;
    return k;
}

__global__ void __launch_bounds__(PK_THREADS) k_pack(Geo g, Bufs bf, int layer, const uint16_t* __restrict__ kp,
                                                     const uint16_t* __restrict__ vp) {
    __shared__ uint16_t sk[PK_MAXE], sv[PK_MAXE];
    __shared__ uint8_t ck[PK_MAXE], cv[PK_MAXE];
    __shared__ double p_off[128 + 64], p_scl[128 + 64];   // key channels, then value tokens
    const int l = layer >= 0 ? layer : blockIdx.x % g.L;
    const int b = layer >= 0 ? blockIdx.x : blockIdx.x / g.L;
    const int64_t u = unit_of(g, b, l);
    UnitHdr* hdr = bf.hdr + u;
    const int n_items = hdr->n_pack * g.h_kv;
    const int W = g.W, d = g.d;
    for (int it = blockIdx.y; it < n_items; it += gridDim.y) {
        const PackItem pi = bf.pack[u * g.n_windows + it / g.h_kv];
        const int h = it % g.h_kv;
        const int start = g.n_sink + pi.win * W;
        const uint16_t *srck, *srcv;
        if (pi.src_prompt) {
            srck = kp + (((int64_t)b * g.h_kv + h) * g.S_max + start) * d;
            srcv = vp + (((int64_t)b * g.h_kv + h) * g.S_max + start) * d;
        } else {
            const uint16_t* pg = bf.pages + u * (int64_t)g.n_pages * g.page_elems + (int64_t)pi.src_page * g.page_elems;
            srck = pg + (int64_t)(2 * h) * W * d;
            srcv = pg + (int64_t)(2 * h + 1) * W * d;
        }
        const bool from_page = !pi.src_prompt;
        if (pi.dst_slot < 0 || (!pi.src_prompt && pi.src_page < 0)) {
            if (threadIdx.x == 0) atomicOr(&hdr->status, QEVICT_DEV_E_POOL);
            continue;
        }
        // staged in batches of SB elements per thread, every load of a batch issued before
        // the first LDS store (clamped addresses; positions past W*d are not stored)
        constexpr int SB = 8;
        for (int e0 = threadIdx.x; e0 < W * d; e0 += SB * PK_THREADS) {
            uint16_t xk[SB], xv[SB];
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                const int e = min(e0 + k * PK_THREADS, W * d - 1), t = e / d, c = e % d;
                xk[k] = srck[from_page ? lay_k(t, c, d, W) : e];
                xv[k] = srcv[from_page ? lay_v(t, c, d, W) : e];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                const int e = e0 + k * PK_THREADS;
                if (e < W * d) {
                    sk[e] = xk[k];
                    sv[e] = xv[k];
                }
            }
        }
        __syncthreads();
        uint8_t* slot = bf.slots + u * (int64_t)g.n_slots * g.slot_bytes + (int64_t)pi.dst_slot * g.slot_bytes +
                        (int64_t)h * g.slot_head_bytes;
        const int qb = g.qbits, P = 8 / qb, L = (1 << qb) - 1, cbytes = lay_code_bytes(W, d, qb);
        uint16_t* offK = (uint16_t*)(slot + 2 * cbytes);
        uint16_t* sclK = offK + d;
        uint16_t* offV = sclK + d;
        uint16_t* sclV = offV + W;
        bool bad = false;
        // keys as quantized: the stored (bf16) values, or in RoPE mode those values turned
        // back to the pre-RoPE domain at their positions (exact products, one rounding)
        const bool rope = (g.flags & QEVICT_F_ROPE) != 0;
        const int hd = d / 2;
        auto key_at = [&](int t, int c) -> double {
            if (!rope) return (double)bf16_to_f32(sk[t * d + c]);
            const int i = c < hd ? c : c - hd;
            const float2 cs = bf.rope[(int64_t)(start + t) * hd + i];
            const double a = (double)bf16_to_f32(sk[t * d + i]), b = (double)bf16_to_f32(sk[t * d + i + hd]);
            return c < hd ? __dadd_rn(__dmul_rn(a, (double)cs.x), __dmul_rn(b, (double)cs.y))
                          : __dsub_rn(__dmul_rn(b, (double)cs.x), __dmul_rn(a, (double)cs.y));
        };
        // parameters: threads [0, d) take a key channel each (over the W tokens), threads
        // [d, d + W) a value token each (over the d channels)
        const int tid = threadIdx.x;
        if (tid < d + W) {
            const bool key = tid < d;
            const int gi = key ? tid : tid - d;
            const int n_el = key ? W : d;
            auto elem = [&](int i) -> double {
                return key ? key_at(i, gi) : (double)bf16_to_f32(sv[gi * d + i]);
            };
            double mn = elem(0), mx = mn;
            for (int i = 1; i < n_el; ++i) {
                const double x = elem(i);
                mn = fmin(mn, x);
                mx = fmax(mx, x);
            }
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
            p_off[tid] = off;
            p_scl[tid] = scl;
        }
        __syncthreads();
        // codes: every element on its own thread
        for (int e = tid; e < W * d; e += PK_THREADS) {
            const int i = e / d, c = e % d;
            ck[e] = (uint8_t)nearest_level(2.0 * (key_at(i, c) - p_off[c]), p_scl[c], L);
            cv[e] = (uint8_t)nearest_level(2.0 * ((double)bf16_to_f32(sv[e]) - p_off[d + i]), p_scl[d + i], L);
        }
        if (bad) atomicOr(&hdr->status, QEVICT_DEV_E_RANGE);
        __syncthreads();
        // K codes: P consecutive channels of one token per byte (lay_kc_byte)
        for (int e = threadIdx.x; e < cbytes; e += PK_THREADS) {
            const int i = e / (d / P), c0 = P * (e % (d / P));
            uint32_t byte = 0;
            for (int x = 0; x < P; ++x) byte |= (uint32_t)ck[i * d + c0 + x] << (qb * x);
            slot[lay_kc_byte(i, c0, d, W, qb, rope)] = (uint8_t)byte;
        }
        // V codes: one byte = P consecutive tokens of one channel (lay_vc_byte)
        for (int e = threadIdx.x; e < cbytes; e += PK_THREADS) {
            const int c = e % d, t0 = P * (e / d);
            uint32_t byte = 0;
            for (int x = 0; x < P; ++x) byte |= (uint32_t)cv[(t0 + x) * d + c] << (qb * x);
            slot[cbytes + lay_vc_byte(t0, c, d, W, qb)] = (uint8_t)byte;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------ fill (promote / copy)
// Promotion writes bf16(off + code*scl), rounded once from the exact fp64 value
// (§4.3: promotion reconstructs the same low-bit approximation in the execution
// datatype).  Prefill copies prompt tokens into pages.
__global__ void __launch_bounds__(PK_THREADS) k_fill(Geo g, Bufs bf, int layer, const uint16_t* __restrict__ kp,
                                                     const uint16_t* __restrict__ vp) {
    const int l = layer >= 0 ? layer : blockIdx.x % g.L;
    const int b = layer >= 0 ? blockIdx.x : blockIdx.x / g.L;
    const int64_t u = unit_of(g, b, l);
    UnitHdr* hdr = bf.hdr + u;
    const int n_items = hdr->n_fill * g.h_kv;
    const int W = g.W, d = g.d;
    const int S = hdr->prompt_len;
    for (int it = blockIdx.y; it < n_items; it += gridDim.y) {
        const FillItem fi = bf.fill[u * g.n_windows + it / g.h_kv];
        const int h = it % g.h_kv;
        if (fi.dst_page < 0) {
            if (threadIdx.x == 0) atomicOr(&hdr->status, QEVICT_DEV_E_POOL);
            continue;
        }
        uint16_t* pg = bf.pages + u * (int64_t)g.n_pages * g.page_elems + (int64_t)fi.dst_page * g.page_elems;
        uint16_t* dk = pg + (int64_t)(2 * h) * W * d;
        uint16_t* dv = pg + (int64_t)(2 * h + 1) * W * d;
        const int start = g.n_sink + fi.win * W;
        if (fi.src_slot >= 0) {
            const uint8_t* slot = bf.slots + u * (int64_t)g.n_slots * g.slot_bytes +
                                  (int64_t)fi.src_slot * g.slot_bytes + (int64_t)h * g.slot_head_bytes;
            const int qb = g.qbits, mask = (1 << qb) - 1, cbytes = lay_code_bytes(W, d, qb);
            const uint16_t* offK = (const uint16_t*)(slot + 2 * cbytes);
            const uint16_t* sclK = offK + d;
            const uint16_t* offV = sclK + d;
            const uint16_t* sclV = offV + W;
            const bool rope = (g.flags & QEVICT_F_ROPE) != 0;
            const int hd = d / 2;
            auto khat = [&](int i, int c) -> double {   // dequantized key (exact in fp64)
                const int kc = (slot[lay_kc_byte(i, c, d, W, qb, rope)] >> lay_kc_shift(c, qb)) & mask;
                return (double)fp16_bits_to_f32(offK[c]) + kc * (double)fp16_bits_to_f32(sclK[c]);
            };
            for (int e = threadIdx.x; e < W * d; e += PK_THREADS) {
                const int i = e / d, c = e % d;
                const int vc = (slot[cbytes + lay_vc_byte(i, c, d, W, qb)] >> lay_vc_shift(i, qb)) & mask;
                const int vp = lay_vp(i, W);
                double kx = khat(i, c);
                if (rope) {   // RoPE re-applied at the window's positions, then one bf16 rounding
                    const int pi = c < hd ? c : c - hd;
                    const float2 cs = bf.rope[(int64_t)(start + i) * hd + pi];
                    const double xp = khat(i, c < hd ? c + hd : c - hd);
                    kx = c < hd ? __dsub_rn(__dmul_rn(kx, (double)cs.x), __dmul_rn(xp, (double)cs.y))
                                : __dadd_rn(__dmul_rn(kx, (double)cs.x), __dmul_rn(xp, (double)cs.y));
                }
                const double vx = (double)fp16_bits_to_f32(offV[vp]) + vc * (double)fp16_bits_to_f32(sclV[vp]);
                dk[lay_k(i, c, d, W)] = f64_to_bf16(kx);
                dv[lay_v(i, c, d, W)] = f64_to_bf16(vx);
            }
        } else if (fi.src_slot == -1) {
            const uint16_t* sk = kp + (((int64_t)b * g.h_kv + h) * g.S_max + start) * d;
            const uint16_t* sv = vp + (((int64_t)b * g.h_kv + h) * g.S_max + start) * d;
            int ntok = S - start;
            if (ntok > W) ntok = W;
            for (int e = threadIdx.x; e < W * d; e += PK_THREADS) {
                const int i = e / d, c = e % d;
                dk[lay_k(i, c, d, W)] = i < ntok ? sk[e] : (uint16_t)0;
                dv[lay_v(i, c, d, W)] = i < ntok ? sv[e] : (uint16_t)0;
            }
        } else {
            for (int e = threadIdx.x; e < W * d; e += PK_THREADS) {
                dk[e] = 0;
                dv[e] = 0;
            }
        }
    }
}

hipError_t launch_migrate(const Geo& g, const Bufs& bf, int layer, const uint16_t* kp, const uint16_t* vp,
                          hipStream_t s) {
    const int units = layer >= 0 ? g.B : g.B * g.L;
    // workgroups per unit: a prefill (one layer, every prompt window) spreads its items over
    // about 1024 workgroups in all; a routing event over all layers moves few per unit
    const int nb = layer >= 0 ? std::max(64, 1024 / std::max(g.B, 1)) : 64;
    hipLaunchKernelGGL(k_pack, dim3(units, nb), dim3(PK_THREADS), 0, s, g, bf, layer, kp, vp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_fill, dim3(units, nb), dim3(PK_THREADS), 0, s, g, bf, layer, kp, vp);
    return hipGetLastError();
}

}  // namespace qv
