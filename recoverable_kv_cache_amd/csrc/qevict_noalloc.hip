// Allocation-free variant of the prefill entry point.  The prompt-attention column sums
// (row log-sum-exps, then per-head column sums) need a device workspace; this entry point
// takes it from a static device array of the library instead of from the caller, for callers
// that cannot allocate device memory.  Each GPU the library runs on holds its own copy of the
// array until the process ends, and every call on that GPU shares it.
#include <cstdio>
#include <mutex>

#include "qevict_internal.h"

namespace {

constexpr size_t kScratchBytes = QEVICT_NOALLOC_WS_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` on each device, once looked up

// Device address of the array on the current device `dev`: looked up once per device with that
// device current.  The array's name in host code is a host-side stand-in, never a device address.
hipError_t scratch_on(int dev, void** out) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" qevict_status qevict_prefill_init_noalloc(qevict_state* st, int32_t layer, const void* q_prompt,
                                                     const void* k_prompt, const void* v_prompt,
                                                     const double* score_init, void* stream) {
    if (!st) return qv::set_error(QEVICT_E_INVALID, "null state");
    const size_t need = qv::state_prefill_ws_bytes(st);
    if (need > kScratchBytes) {
        char msg[200];
        snprintf(msg, sizeof msg, "prefill workspace of %zu bytes exceeds the static %zu-byte array; "
                 "use qevict_prefill_init with a caller workspace", need, kScratchBytes);
        return qv::set_error(QEVICT_E_CAPACITY, msg);
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return qv::set_error(QEVICT_E_HIP, "hipGetDevice failed");
    if (dev != qv::state_device(st))
        return qv::set_error(QEVICT_E_STATE, "the state's device must be current");
    if (dev < 0 || dev >= kMaxDevices) return qv::set_error(QEVICT_E_INVALID, "device index out of range");
    void* ws = nullptr;
    const hipError_t e = scratch_on(dev, &ws);
    if (e != hipSuccess) {
        char msg[200];
        snprintf(msg, sizeof msg, "hipGetSymbolAddress: %s", hipGetErrorString(e));
        return qv::set_error(QEVICT_E_HIP, msg);
    }
    return qevict_prefill_init(st, layer, q_prompt, k_prompt, v_prompt, score_init, ws, kScratchBytes, stream);
}
