// Router of one (sequence, layer) unit per workgroup, compiled once per workgroup size:
// qevict_state.hip includes this file inside a namespace per instance, with QV_RT_THREADS set
// (1024 threads for up to 4096 windows per unit, 256 for up to 1024: four windows per thread).
// Source: "QEvict: Recoverable Quantized KV Eviction for Attention-Drift-Robust Long-Context
// Decoding", §4.2 Eq. 1, §4.3 Eqs. 3-6 and Algorithm 1 (routing, migration, reconstruction of
// the accessible set).
constexpr int RT_THREADS = QV_RT_THREADS;
constexpr int RT_MAXW = 4 * RT_THREADS;  // windows per unit handled by one workgroup
constexpr int RT_PER = RT_MAXW / RT_THREADS;
constexpr int RT_WAVES = RT_THREADS / 64;

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

// Exclusive scan of a[0..RT_MAXW) in LDS; returns the total.  All threads call.  Two counts
// may share an element as 16-bit fields (lo + (hi << 16)): the fields add independently
// while each total stays below 2^16 (at most RT_MAXW here).  wsum: RT_WAVES ints of LDS,
// 16-byte aligned.
__device__ int block_scan_excl(int* a, int* wsum) {
    static_assert(RT_PER == 4, "four elements per thread");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int4 v = *reinterpret_cast<const int4*>(a + tid * RT_PER);
    const int s = v.x + v.y + v.z + v.w;
    const int incl = (int)wave_scan_incl((unsigned)s);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int all, before;
    wave_totals(wsum, wave, all, before);
    int4 o;
    o.x = before + incl - s;
    o.y = o.x + v.x;
    o.z = o.y + v.y;
    o.w = o.z + v.z;
    *reinterpret_cast<int4*>(a + tid * RT_PER) = o;
    __syncthreads();
    return all;
}

struct RouteSmem {
    unsigned long long work[RT_MAXW];   // scratch: key-norm sums, tier selection, then flag arrays
    int idx[RT_MAXW];
    int8_t newst[RT_MAXW];
    alignas(16) int wsum[RT_WAVES];
    int misc[8];
};

// ---------------------------------------------------------------- tier selection (Eq. 5)
// Only tier membership matters: Full = the K_f first candidates in rank order (score
// descending, window index ascending), Quantized = the next K_q.  Each candidate has the
// composite key C = (~ord_key(score) << 12) | window, distinct and ascending in rank order;
// a tier boundary is the composite of rank k (the k-th smallest).  It is found by radix
// selection: digits of C from the top (11 bits with 1024 threads, 9 with 256); per pass a
// digit histogram of the candidates that share the prefix found so far (LDS atomics), then
// the bin holding rank k (every thread takes two bins; block prefix sum) extends the
// prefix.  Once that bin holds at most
// 64 candidates they are gathered and one wave ranks them exactly.  Two selections (member
// sets and ranks) run side by side.  The loop state is block-uniform and kept in scalar
// registers.
using u128 = unsigned __int128;
constexpr int SEL_BITS = 76;             // 64 key bits + 12 window bits (RT_MAXW <= 4096)
constexpr int SEL_D = RT_THREADS == 1024 ? 11 : RT_THREADS == 512 ? 10 : 9;   // two bins per thread
constexpr int SEL_BINS = 1 << SEL_D, SEL_FIN = 64;
constexpr int SEL_PASSES = (SEL_BITS + SEL_D - 1) / SEL_D;
static_assert(RT_MAXW <= 4096, "window index must fit the 12 low bits of the composite key");
static_assert(SEL_BINS == 2 * RT_THREADS, "the bin search takes two bins per thread");

struct SelSmem {
    int wtot[2][RT_WAVES];                 // per-wave totals (counts, then bin sums)
    unsigned wand[RT_WAVES], wor[RT_WAVES];
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
    {   // member counts (two 16-bit fields: at most RT_MAXW each), and the bits that all
        // members share at the top of their composites (AND == OR over the top 32 bits):
        // the first digit starts below them
        unsigned ka = ~0u, ko = 0u;
#pragma unroll
        for (int e = 0; e < RT_PER; ++e)
            if (((mem[0] | mem[1]) >> e) & 1) {
                const unsigned top = (unsigned)(c[e] >> (SEL_BITS - 32));
                ka &= top;
                ko |= top;
            }
        const int v = wave_sum_i32(__popc(mem[0]) | (__popc(mem[1]) << 16));
        ka = wave_and_u32(ka);
        ko = wave_or_u32(ko);
        if (lane == 0) {
            ss.wtot[0][wave] = v;
            ss.wand[wave] = ka;
            ss.wor[wave] = ko;
        }
        if (tid < 2) ss.gcnt[tid] = 0;
        __syncthreads();
        int tot, unused;
        wave_totals(ss.wtot[0], 0, tot, unused);
        tot = uni(tot);
        const int n[2] = {tot & 0xFFFF, tot >> 16};
#pragma unroll
        for (int q = 0; q < RT_WAVES; ++q) {
            ka &= ss.wand[q];
            ko |= ss.wor[q];
        }
        const unsigned diff = (unsigned)uni((int)(ka ^ ko)), kau = (unsigned)uni((int)ka);
        const int p0 = diff == 0 ? 32 : __clz(diff);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            st[t] = k[t] <= 0 ? SEL_NONE : (k[t] >= n[t] ? SEL_ALL : SEL_SEARCH);
            p[t] = p0;
            pv[t] = p0 == 0 ? (u128)0 : (u128)(kau >> (32 - p0));
        }
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
    const int NW = g.n_windows;
    // Loads that depend on nothing read here go first, with the header's, so that they share
    // one round trip: the accessible entry this thread folds first, and the window records
    // and rank keys of its windows w = tid + i * RT_THREADS (the rank keys again below when
    // a ranker rewrites them in memory first).  Every load is unconditional, from a clamped
    // index, and out-of-range values are replaced afterwards: a load under a per-thread
    // condition would be waited for on the spot, one round trip each.
    const int e_first = 1 + tid;
    const AccEntry en_first = bf.acc[u * g.n_acc_max + (e_first < g.n_acc_max ? e_first : g.n_acc_max - 1)];
    WinRec rec[RT_PER];
    double sc[RT_PER];
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) {
        const int w = tid + i * RT_THREADS, wc = w < NW ? w : NW - 1;
        rec[i] = win[wc];
        sc[i] = score[wc];
    }
    const UnitHdr hd = *hdr;             // (one batch of scalar loads)
    const int n = hd.n;
    const int K_f = hd.K_f, K_q = hd.K_q;
    const int n_acc_old = hd.n_acc;
    const bool fold = hd.mass_pending != 0;
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) {
        const bool in = tid + i * RT_THREADS < NW;
        rec[i].state = in ? rec[i].state : ST_NONE;
        rec[i].page = in ? rec[i].page : -1;
        rec[i].slot = in ? rec[i].slot : -1;
        rec[i].flags = in ? rec[i].flags : 0;
        sc[i] = in ? sc[i] : 0.0;
    }
    int* flag = (int*)sm.work;               // (used after the tier selection)

    // ---- 0. the last decode step's window-mass shares (Eq. 1), folded before routing: one
    //         thread per accessible entry, the entry's mass to LDS by window.  With the
    //         cumulative ranker the sums join the rank keys as they are read (below);
    //         the other rankers take them in global memory first.
    const bool cum_fold = fold && !rank_interval(g) && !(g.flags & QEVICT_F_RANK_KEYNORM);
    double* mwin = reinterpret_cast<double*>(sm.work);      // RT_MAXW doubles
    // (entry 0: the sinks, no window.)  The mass of an entry is computed whether or not it has
    // a window (or a fold is pending), so that its row's loads wait for neither; the first
    // entry's loads (from a clamped row, unconditional) are in flight while the table is cleared.
    const float* lwin = bf.lse_win + lse_win_off(g, u, (n - 1) & 1);   // the step at position n - 1
    const float* lg = bf.lse_glob + lse_glob_off(g, u, (n - 1) & 1);
    const double m_row = entry_mass(lwin + (int64_t)(e_first < g.n_acc_max ? e_first : g.n_acc_max - 1) * g.h_q, lg,
                                    g.h_q) / g.h_q;
    if (fold) {
        const int n_acc = n_acc_old;
        const double m_first = e_first < n_acc ? m_row : 0.0;
        for (int w = tid; w < RT_MAXW; w += RT_THREADS) mwin[w] = 0.0;
        __syncthreads();
        if (e_first < n_acc && en_first.win >= 0 && en_first.win < NW) mwin[en_first.win] = m_first;
        for (int e = e_first + RT_THREADS; e < n_acc; e += RT_THREADS) {
            const AccEntry en = bf.acc[u * g.n_acc_max + e];
            const double m = entry_mass(lwin + (int64_t)e * g.h_q, lg, g.h_q) / g.h_q;
            if (en.win >= 0 && en.win < NW) mwin[en.win] = m;
        }
        __syncthreads();
        if (tid == 0) hdr->mass_pending = 0;
        if (!cum_fold) {
            double* tgt = mass_target(g, bf) + u * NW;
            for (int w = tid; w < NW; w += RT_THREADS)
                if (mwin[w] != 0.0) tgt[w] += mwin[w];
            __syncthreads();
        }
    }
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

    if (mode == RM_ROUTE && (rank_interval(g) || (g.flags & QEVICT_F_RANK_KEYNORM))) {
#pragma unroll
        for (int i = 0; i < RT_PER; ++i) {   // (rewritten above)
            const int w = tid + i * RT_THREADS;
            sc[i] = w < NW ? score[w] : 0.0;
        }
    }
    if (cum_fold) {   // S_bar(w) += the step's mass (windows with an entry)
#pragma unroll
        for (int i = 0; i < RT_PER; ++i) {
            const int w = tid + i * RT_THREADS;
            const double m = w < NW ? mwin[w] : 0.0;
            if (m != 0.0) {
                sc[i] += m;
                score[w] = sc[i];
            }
        }
        __syncthreads();   // (mwin aliases the selection scratch)
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
        ckey[i] = sel_composite(c && (mode == RM_ROUTE || mode == RM_PREFILL) ? sc[i] : 0.0, w);
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

    // ---- 4. migration actions (Algorithm 1: promotion, demotion, eviction).  Per window:
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
                a |= 2;               // fresh recent-region page (not cleared: decode reads only its written rows)
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
    int* pushed = sm.idx;     // ids pushed at this event, by stack position - cnt0 (sm.idx is free after phase 3)
    // pages: the window that took each page pushed at this event (-1: none), by push position
    int* taker = flag + RT_MAXW;
    constexpr int PACKED = 0x40000000;   // (pages) pushed by a window packed at this event
    int my_push[RT_PER], my_taken_from[RT_PER];
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) my_push[i] = my_taken_from[i] = -1;
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
                pushed[pos - cnt0] = id | (pass == 1 && (act[i] & 16) && id >= 0 ? PACKED : 0);
                if (pass == 1) {
                    taker[pos - cnt0] = -1;
                    my_push[i] = pos - cnt0;
                }
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
                int id = k >= avail ? -1 : (at >= cnt0 ? pushed[at - cnt0] : stack[at]);
                if (id >= 0 && (id & PACKED)) {   // a page the pack of its window reads at this event
                    id &= ~PACKED;
                    if (act[i] & 32) {            // ... and a fill writes (a fresh recent page is
                        taker[at - cnt0] = tid + i * RT_THREADS;   // written only by later steps)
                        my_taken_from[i] = at - cnt0;
                    }
                }
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

    // ---- 6. work lists: pack (quantize once) and fill (promote / copy prompt).  A page freed by
    //      a window packed at this event and taken by a promotion at this event is written only
    //      after that pack has read it: the fill item runs as the pack item's second half.
    int my_taker[RT_PER];
#pragma unroll
    for (int i = 0; i < RT_PER; ++i) my_taker[i] = my_push[i] >= 0 && (act[i] & 16) ? taker[my_push[i]] : -1;
    __syncthreads();   // (taker lives in the upper half of the scan array)
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
            it.then_fill = my_taker[i] >= 0 ? (flag[my_taker[i]] >> 16) : -1;
            it.pad[0] = it.pad[1] = it.pad[2] = 0;
            bf.pack[u * g.n_windows + (flag[w] & 0xFFFF)] = it;
        }
        if (act[i] & 32) {
            FillItem it;
            it.win = w;
            it.dst_page = my_page[i];
            it.src_slot = r.state == ST_QUANT ? r.slot : -1;   // promote, or copy the prompt tokens
            it.after_pack = my_taken_from[i] >= 0 ? 1 : 0;
            bf.fill[u * g.n_windows + (flag[w] >> 16)] = it;
            if (it.after_pack) atomicAdd(&hdr->paired, 1);
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
    // ---- 8. accessible list (Algorithm 1: the accessible set after migration) and its splits.  The bf16
    //      pages and the Quantized slots, each in chronological order, are merged so that
    //      the pages fall evenly among the slots (by rank fraction, (2r + 1) / 2count, pages
    //      first on ties): every split then holds a like share of both kinds, whose costs
    //      per byte differ.  Attention does not depend on the order.  The splits cut the
    //      list at equal shares of the entries' job costs (per_head_cost).
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
    const int total = block_scan_excl(cost, sm.wsum);   // cost[e] = cost of the entries before e
    int32_t* splits = bf.splits + u * (g.n_splits + 1);
    int* spos = flag + RT_MAXW;    // the boundaries, for the split blocks below (flag is free here)
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
            // the boundary nearer the target (cost[n_acc] would be the total)
            const long long c_hi = lo < n_acc ? cost[lo] : total;
            if (lo > 0 && tgt - cost[lo - 1] < c_hi - tgt) lo -= 1;
            pos = lo;
        }
        splits[s] = pos;
        spos[s] = pos;
    }
    __syncthreads();   // (also: the list entries above are visible to the whole workgroup)
    // each split's block: header {entries, first entry, -1, 0}, then its first SPLIT_BLOCK - 1
    // entries (padding past them), one entry per thread
    for (int k = tid; k < g.n_splits * SPLIT_BLOCK; k += RT_THREADS) {
        const int sp = k / SPLIT_BLOCK, x = k % SPLIT_BLOCK, e0 = spos[sp], cnt = spos[sp + 1] - e0;
        AccEntry v = AccEntry{EK_PAGE, -1, -1, 0};
        if (x == 0) v = AccEntry{cnt, e0, -1, 0};
        else if (x - 1 < cnt) v = acc[e0 + x - 1];
        bf.split_blk[(u * g.n_splits + sp) * SPLIT_BLOCK + x] = v;
    }
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


