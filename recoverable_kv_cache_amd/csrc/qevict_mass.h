// Folding the window-mass shares of the last decode step into the cumulative
// window score (Eq. 1 of "QEvict: Recoverable Quantized KV Eviction for
// Attention-Drift-Robust Long-Context Decoding", §4.2): S_bar(w) += (1/H_q)
// sum_h share_h(w), with share_h(w) = exp of (window log-sum-exp - row
// log-sum-exp) of head h, summed in head order in fp64.
#pragma once

#include "qevict_internal.h"

namespace qv {

// adds the pending shares of accessible entries first + k*step (k = 0, 1, ...), e < last;
// the sink entry (index 0) has no window and is skipped
__device__ inline void apply_mass_range(const Geo& g, const Bufs& bf, int64_t u, int first, int last, int step) {
    for (int e = first; e < last; e += step) {
        if (e == 0) continue;
        const AccEntry en = bf.acc[u * g.n_acc_max + e];
        const float* row = bf.mass_part + (u * g.n_acc_max + e) * (int64_t)g.h_q;
        double sm = 0.0;
        for (int h = 0; h < g.h_q; ++h) sm += (double)row[h];
        if (en.win >= 0) bf.score[u * g.n_windows + en.win] += sm / g.h_q;
    }
}

}  // namespace qv
