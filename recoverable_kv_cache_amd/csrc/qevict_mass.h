// Folding the window-mass shares of the last decode step into the cumulative
// window score (Eq. 1 of "QEvict: Recoverable Quantized KV Eviction for
// Attention-Drift-Robust Long-Context Decoding", §4.2): S_bar(w) += (1/H_q)
// sum_h share_h(w), with share_h(w) = 2^(window log-sum-exp - row log-sum-exp)
// of head h (log2 domain, fp32), summed in head order in fp64.  The inputs are the
// step's window log-sum-exps (by parity of its position) and its row log-sum-exps.
#pragma once

#include "qevict_internal.h"

namespace qv {

// one head's share of an entry's window mass
__device__ __forceinline__ float mass_share(float lse_w, float lse_row) { return __builtin_amdgcn_exp2f(lse_w - lse_row); }

// adds the pending shares of accessible entries first + k*step (k = 0, 1, ...), e < last,
// of the decode step at position pos; the sink entry (index 0) has no window and is skipped
__device__ inline void apply_mass_range(const Geo& g, const Bufs& bf, int64_t u, int pos, int first, int last,
                                        int step) {
    const float* lwin = bf.lse_win + lse_win_off(g, u, pos & 1);
    const float* lg = bf.lse_glob + u * g.h_q;
    for (int e = first; e < last; e += step) {
        if (e == 0) continue;
        const AccEntry en = bf.acc[u * g.n_acc_max + e];
        const float* row = lwin + (int64_t)e * g.h_q;
        double sm = 0.0;
        for (int h = 0; h < g.h_q; ++h) sm += (double)mass_share(row[h], lg[h]);
        if (en.win >= 0) bf.score[u * g.n_windows + en.win] += sm / g.h_q;
    }
}

}  // namespace qv
