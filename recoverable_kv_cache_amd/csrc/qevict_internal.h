// Device-side layout of the QEvict state and the kernel entry points.
// All persistent state of one (sequence b, layer l) "unit" lives in per-unit
// slices of a few arrays carved out of one caller-allocated arena.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qevict.h"

namespace qv {

// window states (tiers of §4.1 plus the protected recent region and the
// transient "still in the caller's prompt buffer" state used during prefill)
enum : int32_t { ST_NONE = 0, ST_LOCAL = 1, ST_FULL = 2, ST_QUANT = 3, ST_EVICTED = 4, ST_PROMPT = 5 };
enum : int32_t { WF_LEDGER = 1, WF_DORMANT = 2 };
// accessible-list entry kinds
enum : int32_t { EK_SINK = 0, EK_PAGE = 1, EK_SLOT = 2 };
// route modes
enum : int32_t { RM_ROUTE = 0, RM_PREFILL = 1, RM_FORCE_Q = 2, RM_FORCE_F = 3 };
// counters of the last event
enum : int32_t { C_AGED = 0, C_PROMOTED, C_PACKED, C_REACTIVATED, C_DEMOTED, C_EVICTED, C_NFULL, C_NQUANT };

struct WinRec {
    int32_t state;
    int32_t page;    // bf16 page id or -1
    int32_t slot;    // INT2 slot id or -1
    int32_t flags;   // WF_LEDGER | WF_DORMANT
};

struct AccEntry {
    int32_t kind;    // EK_*
    int32_t idx;     // page or slot id
    int32_t win;     // window id (-1 for the sinks)
    int32_t start;   // first position
};

struct PackItem {    // quantize a window once: source bf16 -> slot
    int32_t win;
    int32_t src_prompt;  // 1: caller prompt buffer, 0: page
    int32_t src_page;
    int32_t dst_slot;
};

struct FillItem {    // write a bf16 page: promote from a slot, or copy from the prompt
    int32_t win;
    int32_t dst_page;
    int32_t src_slot;    // >= 0: promote (dequantize); -1: copy prompt tokens
    int32_t pad;
};

struct UnitHdr {
    int32_t n;            // tokens in the cache (next position)
    int32_t prompt_len;
    int32_t n_acc;        // accessible-list length
    int32_t n_win;        // windows with a record (created or prepared)
    int32_t n_free_pages;
    int32_t n_free_slots;
    uint32_t status;      // QEVICT_DEV_E_* bits
    int32_t n_pack;
    int32_t n_fill;
    int32_t K_f;
    int32_t K_q;
    int32_t ctr[8];
    int32_t pad0;
    double sink_mass;     // prefill: head-averaged attention mass on the sink prefix
    int32_t pad[10];      // 128 bytes in all
};
static_assert(sizeof(UnitHdr) == 128, "UnitHdr layout");

// Geometry shared by all kernels (passed by value).
struct Geo {
    int32_t B, L, h_q, h_kv, d, W, n_sink, n_local, omega;
    int32_t S_max;        // prompt buffer row stride
    int32_t n_windows, n_pages, n_slots, n_acc_max, n_splits;
    int32_t page_elems;   // bf16 elements per page = h_kv * 2 * W * d
    int32_t slot_head_bytes;  // W*d/2 + 4d + 4W
    int32_t slot_bytes;   // h_kv * slot_head_bytes
    int32_t sink_elems;   // h_kv * 2 * n_sink * d
    uint32_t flags;
};

// Device pointers to the per-unit arrays (index by unit = b * L + l).
struct Bufs {
    UnitHdr* hdr;           // [U]
    WinRec* win;            // [U][n_windows]
    double* score;          // [U][n_windows]
    AccEntry* acc;          // [U][n_acc_max]
    int32_t* splits;        // [U][n_splits + 1]
    int32_t* free_pages;    // [U][n_pages]
    int32_t* free_slots;    // [U][n_slots]
    PackItem* pack;         // [U][n_windows]
    FillItem* fill;         // [U][n_windows]
    int8_t* target;         // [U][n_windows] forced targets
    float* lse_win;         // [U][n_acc_max][h_q]   log2 domain
    float* lse_glob;        // [U][h_q]              log2 domain
    float2* part_ml;        // [U][n_splits][h_q]    (m, l), log2 domain
    float* part_acc;        // [U][n_splits][h_q][d]
    uint16_t* pages;        // [U][n_pages][h_kv][2][W][d]   bf16
    uint8_t* slots;         // [U][n_slots][h_kv][slot_head_bytes]
    uint16_t* sinks;        // [U][h_kv][2][n_sink][d]       bf16
};

__host__ __device__ inline int64_t unit_of(const Geo& g, int b, int l) { return (int64_t)b * g.L + l; }

// ---------------------------------------------------------------- launchers (host side)
hipError_t launch_init(const Geo& g, const Bufs& bf, const int32_t* prompt_lens_dev, const int32_t* kf_dev,
                       const int32_t* kq_dev, hipStream_t s);
hipError_t launch_append(const Geo& g, const Bufs& bf, int layer, const uint16_t* k, const uint16_t* v, hipStream_t s);
hipError_t launch_decode(const Geo& g, const Bufs& bf, int layer, const uint16_t* q, hipStream_t s);
hipError_t launch_combine(const Geo& g, const Bufs& bf, int layer, float* out, hipStream_t s);
hipError_t launch_mass(const Geo& g, const Bufs& bf, int layer, hipStream_t s);
hipError_t launch_route(const Geo& g, const Bufs& bf, int layer, int mode, hipStream_t s);
hipError_t launch_force_targets(const Geo& g, const Bufs& bf, int layer, const int32_t* win_ids, int n, int target,
                                hipStream_t s);
hipError_t launch_migrate(const Geo& g, const Bufs& bf, int layer, const uint16_t* kp, const uint16_t* vp,
                          hipStream_t s);
hipError_t launch_prefill_setup(const Geo& g, const Bufs& bf, int layer, const uint16_t* kp, const uint16_t* vp,
                                hipStream_t s);
hipError_t launch_prefill_scores(const Geo& g, const Bufs& bf, int layer, const uint16_t* qp, const uint16_t* kp,
                                 const double* score_init, void* ws, hipStream_t s);
size_t prefill_ws_bytes(const Geo& g);

}  // namespace qv
