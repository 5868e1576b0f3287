// Folding the window-mass shares of the last decode step into the cumulative
// window score (Eq. 1 of "QEvict: Recoverable Quantized KV Eviction for
// Attention-Drift-Robust Long-Context Decoding", §4.2): S_bar(w) += (1/H_q)
// sum_h share_h(w), with share_h(w) = 2^(window log-sum-exp - row log-sum-exp)
// of head h (log2 domain, fp32), summed in head order in fp64.  The inputs are the
// step's window log-sum-exps (by parity of its position) and its row log-sum-exps.
// With the decay / p-norm rankers the mass goes to the interval accumulator instead
// (Appendix J, Eq. 20), which each routing event folds into the rank key.
#pragma once

#include "qevict_internal.h"

namespace qv {

// one head's share of an entry's window mass
__device__ __forceinline__ float mass_share(float lse_w, float lse_row) { return __builtin_amdgcn_exp2f(lse_w - lse_row); }

// sum over the h_q heads, in head order (fp64), of one entry's shares: row = the entry's
// window log-sum-exps [h_q], lg = the step's row log-sum-exps [h_q].  With h_q a multiple
// of 4 the loads go in batches of 32 heads, each batch issued before its first use
// (clamped addresses; heads past h_q add 0), so a batch costs one round trip.
__device__ __forceinline__ double entry_mass(const float* __restrict__ row, const float* __restrict__ lg, int h_q) {
    double sm = 0.0;
    if ((h_q & 3) == 0) {
        constexpr int HB = 8;
        for (int h0 = 0; h0 < h_q; h0 += 4 * HB) {
            float4 v[HB], l[HB];
#pragma unroll
            for (int k = 0; k < HB; ++k) {
                const int h = h0 + 4 * k < h_q - 4 ? h0 + 4 * k : h_q - 4;
                v[k] = *reinterpret_cast<const float4*>(row + h);
                l[k] = *reinterpret_cast<const float4*>(lg + h);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < HB; ++k) {
                const bool in = h0 + 4 * k < h_q;
                sm += in ? (double)mass_share(v[k].x, l[k].x) : 0.0;
                sm += in ? (double)mass_share(v[k].y, l[k].y) : 0.0;
                sm += in ? (double)mass_share(v[k].z, l[k].z) : 0.0;
                sm += in ? (double)mass_share(v[k].w, l[k].w) : 0.0;
            }
        }
    } else {
        for (int h = 0; h < h_q; ++h) sm += (double)mass_share(row[h], lg[h]);
    }
    return sm;
}

// adds the pending shares of accessible entries first + k*step (k = 0, 1, ...), e < last,
// of the decode step at position pos; the sink entry (index 0) has no window and is skipped
__device__ inline void apply_mass_range(const Geo& g, const Bufs& bf, int64_t u, int pos, int first, int last,
                                        int step) {
    const float* lwin = bf.lse_win + lse_win_off(g, u, pos & 1);
    const float* lg = bf.lse_glob + lse_glob_off(g, u, pos & 1);
    for (int e = first; e < last; e += step) {
        if (e == 0) continue;
        const AccEntry en = bf.acc[u * g.n_acc_max + e];
        const double sm = entry_mass(lwin + (int64_t)e * g.h_q, lg, g.h_q);
        if (en.win >= 0) mass_target(g, bf)[u * g.n_windows + en.win] += sm / g.h_q;
    }
}

// sum over the 64 lanes in a fixed order (every lane gets the result)
__device__ inline double wave_sum_f64(double x) {
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
// The key-norm rank key of window w from its bf16 keys (Eq. 24): minus the mean over its
// W tokens of the L2 norm of the token's key over all KV heads' channels.  Token norms
// are computed by whole waves (lanes over (head, channel), fixed order), then summed in
// token order by one thread; `tokn` is LDS scratch for W doubles.  All threads call.
template <typename KeyAt>
__device__ double key_norm_block(const Geo& g, int Wn, KeyAt key_at, double* tokn) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x / 64;
    for (int i = wave; i < Wn; i += nwaves) {
        double ss = 0.0;
        for (int e = lane; e < g.h_kv * g.d; e += 64) {
            const double x = (double)key_at(i, e / g.d, e % g.d);
            ss += x * x;
        }
        ss = wave_sum_f64(ss);
        if (lane == 0) tokn[i] = sqrt(ss);
    }
    __syncthreads();
    double r = 0.0;
    if (tid == 0) {
        double t = 0.0;
        for (int i = 0; i < Wn; ++i) t += tokn[i];
        r = -(t / Wn);
    }
    __syncthreads();
    return r;   // (valid in thread 0)
}

}  // namespace qv
