// Host-only stand-ins for the HIP runtime and the kernel launchers, so that the C-ABI host
// code (validation, byte accounting, arena layout, bookkeeping, export) can run under
// AddressSanitizer on a machine without a GPU.  The "device" is host memory: copies are
// memcpy, kernels do nothing.  Test infrastructure only.
#include <hip/hip_runtime_api.h>

#include <cstring>

#include "qevict_internal.h"

extern "C" {
hipError_t hipGetDevice(int* d) {
    *d = 0;
    return hipSuccess;
}
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "host stand-in error"; }
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
    if (n) std::memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
    if (n) std::memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
}

namespace qv {
hipError_t launch_step_mass(const Geo&, const Bufs&, int, int, double*, hipStream_t) { return hipSuccess; }
hipError_t launch_rope_prompt(const Geo&, const Bufs&, const uint16_t* qp, const uint16_t* kp, void*,
                              const uint16_t** qr, const uint16_t** kr, hipStream_t) {
    *qr = qp;
    *kr = kp;
    return hipSuccess;
}
// A plausible state for the export to walk: every unit holds its prompt, its windows cycle
// through Full (a page), Quantized with a ledger (a slot), Evicted and recent (a page).
hipError_t launch_init(const Geo& g, const Bufs& bf, const int32_t* plens, const int32_t* kf, const int32_t* kq,
                       hipStream_t) {
    for (int64_t u = 0; u < (int64_t)g.B * g.L; ++u) {
        const int b = (int)(u / g.L);
        UnitHdr h;
        std::memset(&h, 0, sizeof h);
        h.prompt_len = plens[b];
        h.n = plens[b];
        h.K_f = kf[b];
        h.K_q = kq[b];
        bf.hdr[u] = h;
        for (int w = 0; w < g.n_windows; ++w) {
            const int k = w % 4;
            const int st = k == 0 ? ST_FULL : k == 1 ? ST_QUANT : k == 2 ? ST_EVICTED : ST_LOCAL;
            const int page = (st == ST_FULL || st == ST_LOCAL) ? w % g.n_pages : -1;
            const int slot = st == ST_QUANT ? w % g.n_slots : -1;
            bf.win[u * g.n_windows + w] = WinRec{st, page, slot, st == ST_QUANT ? WF_LEDGER : 0};
            bf.score[u * g.n_windows + w] = 0.5 * w;
        }
        for (int s = 0; s <= g.n_splits; ++s) bf.splits[u * (g.n_splits + 1) + s] = 0;
    }
    return hipSuccess;
}
hipError_t launch_decode(const Geo&, const Bufs&, int, const uint16_t*, const uint16_t*, const uint16_t*, float*, int,
                         hipStream_t, hipEvent_t, hipEvent_t) {
    return hipSuccess;
}
hipError_t launch_finish(const Geo&, const Bufs&, int, float*, const uint16_t*, const uint16_t*, int, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_flush_mass(const Geo&, const Bufs&, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_route(const Geo&, const Bufs&, int, int, const uint16_t*, const uint16_t*, hipStream_t, hipEvent_t,
                        hipEvent_t) {
    return hipSuccess;
}
hipError_t launch_force_targets(const Geo&, const Bufs&, int, const int32_t*, int, int, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_prefill_setup(const Geo&, const Bufs&, int, const uint16_t*, const uint16_t*, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_prefill_scores(const Geo&, const Bufs&, int, const uint16_t*, const uint16_t*, const double*, void*,
                                 hipStream_t) {
    return hipSuccess;
}
hipError_t launch_stream_read(const void*, uint32_t, uint32_t*, hipStream_t, hipEvent_t, hipEvent_t) {
    return hipSuccess;
}
}  // namespace qv
