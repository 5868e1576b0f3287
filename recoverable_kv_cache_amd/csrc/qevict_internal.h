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
    int32_t then_fill;   // >= 0: the fill item that reuses src_page at this event (runs after this pack)
    int32_t pad[3];
};

struct FillItem {    // write a bf16 page: promote from a slot, or copy from the prompt
    int32_t win;
    int32_t dst_page;
    int32_t src_slot;    // >= 0: promote (dequantize); -1: copy prompt tokens
    int32_t after_pack;  // 1: dst_page was freed by a window packed at this event (run by that pack item)
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
    int32_t paired;       // fill items run as the second half of a pack item (reused page), since creation
    double sink_mass;     // prefill: head-averaged attention mass on the sink prefix
    int32_t mass_pending; // 1: the last decode step's window-mass shares are not yet in score[]
    int32_t pos;          // decode: position of the step's token (written by the split kernel)
    int32_t tok_at;       // decode: position whose block the split kernel found (== pos when found)
    int32_t tok_page;     // decode: page holding that position (-2: the sink block)
    int32_t pad[6];       // 128 bytes in all
};
static_assert(sizeof(UnitHdr) == 128, "UnitHdr layout");

// Geometry shared by all kernels (passed by value).
struct Geo {
    int32_t B, L, h_q, h_kv, d, W, n_sink, n_local, omega;
    int32_t S_max;        // prompt buffer row stride
    int32_t n_windows, n_pages, n_slots, n_acc_max, n_splits;
    int32_t page_elems;   // bf16 elements per page = h_kv * 2 * W * d
    int32_t slot_head_bytes;  // 2 * code_bytes + 4d + 4W
    int32_t slot_bytes;   // h_kv * slot_head_bytes
    int32_t sink_elems;   // h_kv * 2 * Ws * d, Ws = sink_width(n_sink)
    uint32_t flags;
    int32_t qbits;        // bits per Quantized-tier code: 2, or 4 with QEVICT_F_INT4
    int32_t n_rope;       // rows of the RoPE table (0 without QEVICT_F_ROPE)
    int32_t fuse;         // 1: one split per group, and the split kernel also finishes the step
};

// Device pointers to the per-unit arrays (index by unit = b * L + l).
struct Bufs {
    UnitHdr* hdr;           // [U]
    WinRec* win;            // [U][n_windows]
    double* score;          // [U][n_windows]        the rank key (S, or P for the p-norm ranker)
    double* uacc;           // [U][n_windows]        decay / p-norm rankers: mass since the previous routing event
    AccEntry* acc;          // [U][n_acc_max]
    int32_t* splits;        // [U][n_splits + 1]
    AccEntry* split_blk;    // [U][n_splits][SPLIT_BLOCK]: {entries, first entry, -1, 0}, then the split's entries
    int32_t* free_pages;    // [U][n_pages]
    int32_t* free_slots;    // [U][n_slots]
    PackItem* pack;         // [U][n_windows]
    FillItem* fill;         // [U][n_windows]
    int8_t* target;         // [U][n_windows] forced targets
    float* lse_win;         // [U][2][n_acc_max][h_q] log2 domain, by parity of the step's position
    float* lse_glob;        // [U][2][h_q]           log2 domain, by parity of the step's position
    float2* part_ml;        // [U][n_splits][h_q]    (m, l), log2 domain
    float* part_acc;        // [U][n_splits][h_q][d]
    uint16_t* pages;        // [U][n_pages][h_kv][2][W][d]   bf16
    uint8_t* slots;         // [U][n_slots][h_kv][slot_head_bytes]
    uint16_t* sinks;        // [U][h_kv] pages of Ws tokens (same layout as a window page)
    const float2* rope;     // RoPE mode: (cos, sin) [n_rope][d/2], n_rope >= max(32, max_prompt + max_new)
    uint16_t* krot;         // RoPE mode: [U][h_kv][d] the step's key after RoPE (split kernel -> finish)
    uint32_t* unit_arr;     // [U]  one split per group: the unit's workgroups done with a step
};

__host__ __device__ inline int64_t unit_of(const Geo& g, int b, int l) { return (int64_t)b * g.L + l; }
// window log-sum-exps of the decode step at a position of parity par: the next step reads
// them (to fold this step's window mass) while writing its own to the other half
__host__ __device__ inline int64_t lse_win_off(const Geo& g, int64_t u, int par) {
    return (u * 2 + par) * (int64_t)g.n_acc_max * g.h_q;
}
// the heads' log-sum-exps of the step at a position of parity par (same double buffering: a
// split kernel that finishes the step itself writes them while its other workgroups still
// read the previous step's)
__host__ __device__ inline int64_t lse_glob_off(const Geo& g, int64_t u, int par) {
    return (u * 2 + par) * (int64_t)g.h_q;
}

// Each split's header and first SPLIT_BLOCK - 1 accessible-list entries, copied by the
// router to a fixed place so that a decode wave gets them in one load (one per lane).
constexpr int SPLIT_BLOCK = 64;
// (sequence, layer) units one routing launch may cover (batch * n_layers)
constexpr int MIG_MAX_UNITS = 4096;

// ------------------------------------------------------------------ in-HBM layouts
// The decode kernel feeds MFMA tiles straight from HBM, so pages and
// slots are stored in the order a lane consumes them.  One head of a window of
// W tokens (NT = W/16 tiles of 16 tokens), D channels, CQ = D/4 channels per
// lane group, MB = D/16 channel blocks.  t = 16*tile + r, c = CQ*qg + cc.
//
// A "chunk" is up to 32 tokens (TPC = min(W, 32)/16 tiles); NCH = W/TPC/16 chunks.
// bf16 page of one head: K block (W*D) then V block (W*D).
//   K (t, c): (((ch*16 + r)*4 + qg)*TPC + tc)*CQ + cc        t = 32*ch + 16*tc + r
//             (a lane reads the CQ channels of its token row for every tile of a chunk)
//   V (t, c): ((((c%16)*4 + r/4)*NT + tile)*MB + c/16)*4 + r%4
//             (a lane reads, per tile, 4 tokens x MB channel blocks of one channel row)
// Quantized slot of one head, b-bit codes (b = 2 or 4, P = 8/b codes per byte; same byte
// count as the canonical record):
//   K codes [W*D*b/8]: code (t, c) in byte (((ch*16 + r)*4 + qg)*TPC + tc)*(CQ/P) + cc/P, bits b*(cc%P)
//             ((qg, cc) from lay_kc_pos: c = CQ*qg + cc, or the RoPE pairing)
//   V codes [W*D*b/8]: code (t, c) in byte (((((ch*16 + c%16)*4 + r/4)*MB + c/16)*TPC + tc)*(4/P) + (r%4)/P,
//             bits b*(r%P) (a lane reads, per chunk, MB x TPC x 4/P bytes: the 4 tokens of row group
//             r/4 of each tile of the chunk, per channel block; each chunk's codes are contiguous)
//   K offset [D], K scale [D] (fp16, channel order), V offset [W], V scale [W] (fp16) with
//   token t at ((r/4)*NT + tile)*4 + r%4.
__host__ __device__ inline int lay_tpc(int W) { return (W < 32 ? W : 32) / 16; }
__host__ __device__ inline int lay_k(int t, int c, int D, int W) {
    const int CQ = D / 4, TPC = lay_tpc(W);
    const int ch = t / (16 * TPC), tc = (t / 16) % TPC, r = t & 15;
    return (((ch * 16 + r) * 4 + c / CQ) * TPC + tc) * CQ + c % CQ;
}
__host__ __device__ inline int lay_v(int t, int c, int D, int W) {
    const int NT = W / 16, MB = D / 16;
    return ((((c & 15) * 4 + (t & 15) / 4) * NT + (t >> 4)) * MB + c / 16) * 4 + (t & 3);
}
// Key channel c -> (lane group qg, position cc in the group's CQ channels).  In RoPE mode
// a group holds CQ/2 channels of the first half and their RoPE partners c + D/2, so that
// a lane rotates its keys without exchanging values.
__host__ __device__ inline void lay_kc_pos(int c, int D, bool rope, int& qg, int& cc) {
    const int CQ = D / 4;
    if (!rope) {
        qg = c / CQ;
        cc = c % CQ;
    } else if (c < D / 2) {
        qg = c / (CQ / 2);
        cc = c % (CQ / 2);
    } else {
        qg = (c - D / 2) / (CQ / 2);
        cc = CQ / 2 + (c - D / 2) % (CQ / 2);
    }
}
__host__ __device__ inline int lay_kc_byte(int t, int c, int D, int W, int b, bool rope = false) {
    const int CQ = D / 4, TPC = lay_tpc(W), P = 8 / b;
    const int ch = t / (16 * TPC), tc = (t / 16) % TPC, r = t & 15;
    int qg, cc;
    lay_kc_pos(c, D, rope, qg, cc);
    return (((ch * 16 + r) * 4 + qg) * TPC + tc) * (CQ / P) + cc / P;
}
__host__ __device__ inline int lay_kc_shift(int c, int b) { return b * (c % (8 / b)); }
__host__ __device__ inline int lay_vc_byte(int t, int c, int D, int W, int b) {
    const int TPC = lay_tpc(W), MB = D / 16, P = 8 / b;
    const int tile = t >> 4;
    return (((((tile / TPC) * 16 + (c & 15)) * 4 + (t & 15) / 4) * MB + c / 16) * TPC + tile % TPC) * (4 / P) +
           (t & 3) / P;
}
__host__ __device__ inline int lay_vc_shift(int t, int b) { return b * (t % (8 / b)); }
// bytes of one tensor's codes of one head
__host__ __device__ inline int lay_code_bytes(int W, int D, int b) { return W * D * b / 8; }
__host__ __device__ inline int lay_vp(int t, int W) {
    const int NT = W / 16;
    return (((t & 15) / 4) * NT + (t >> 4)) * 4 + (t & 3);
}
// tokens held by the sink block: n_sink rounded up to a supported window size
__host__ __device__ inline int sink_width(int n_sink) { return n_sink <= 16 ? 16 : (n_sink <= 32 ? 32 : 64); }

constexpr double RANK_DECAY_LAMBDA = 0.99;   // Eq. 22
// rankers that fold an interval's mass at each routing event
__host__ __device__ inline bool rank_interval(const Geo& g) {
    return (g.flags & (QEVICT_F_RANK_DECAY | QEVICT_F_RANK_PNORM)) != 0;
}
// where a decode step's window-mass shares go
__host__ __device__ inline double* mass_target(const Geo& g, const Bufs& bf) {
    return rank_interval(g) ? bf.uacc : bf.score;
}

// ---------------------------------------------------------------- launchers (host side)
hipError_t launch_step_mass(const Geo& g, const Bufs& bf, int layer, int b, double* out, hipStream_t s);
size_t rope_ws_offset(const Geo& g);
size_t rope_ws_bytes(const Geo& g);
hipError_t launch_rope_prompt(const Geo& g, const Bufs& bf, const uint16_t* qp, const uint16_t* kp, void* ws,
                              const uint16_t** qr, const uint16_t** kr, hipStream_t s);
hipError_t launch_init(const Geo& g, const Bufs& bf, const int32_t* prompt_lens_dev, const int32_t* kf_dev,
                       const int32_t* kq_dev, hipStream_t s);
// ev0 / ev1 (optional): events stamped by the split kernel's own dispatch at its start and end.
// With g.fuse (one split per group) the split kernel also finishes the step (out, score_now as
// for launch_finish); otherwise launch_finish follows.
hipError_t launch_decode(const Geo& g, const Bufs& bf, int layer, const uint16_t* q, const uint16_t* k_new,
                         const uint16_t* v_new, float* out, int score_now, hipStream_t s, hipEvent_t ev0 = nullptr,
                         hipEvent_t ev1 = nullptr);
hipError_t launch_finish(const Geo& g, const Bufs& bf, int layer, float* out, const uint16_t* k_new,
                         const uint16_t* v_new, int score_now, hipStream_t s);
hipError_t launch_flush_mass(const Geo& g, const Bufs& bf, int layer, int b, hipStream_t s);
// ev0 / ev1 (optional): stamped by the dispatch of the routing kernel at its start and of the
// migration kernel at its end
hipError_t launch_route(const Geo& g, const Bufs& bf, int layer, int mode, const uint16_t* kp, const uint16_t* vp,
                        hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_force_targets(const Geo& g, const Bufs& bf, int layer, const int32_t* win_ids, int n, int target,
                                hipStream_t s);
hipError_t launch_prefill_setup(const Geo& g, const Bufs& bf, int layer, const uint16_t* kp, const uint16_t* vp,
                                hipStream_t s);
hipError_t launch_prefill_scores(const Geo& g, const Bufs& bf, int layer, const uint16_t* qp, const uint16_t* kp,
                                 const double* score_init, void* ws, hipStream_t s);
size_t prefill_ws_bytes(const Geo& g);
// accessors of the host-side state for entry points in other sources
qevict_status set_error(qevict_status s, const char* msg);   // message for qevict_last_error; returns s
size_t state_prefill_ws_bytes(const qevict_state* st);
int state_device(const qevict_state* st);
// measurement aid: one streaming read of [buf, buf + bytes), bytes a multiple of 1024;
// sink receives one XOR word per workgroup (STREAM_READ_WGS of them)
constexpr int STREAM_READ_WGS = 1024;
hipError_t launch_stream_read(const void* buf, uint32_t bytes, uint32_t* sink, hipStream_t s, hipEvent_t ev0,
                              hipEvent_t ev1);

}  // namespace qv
