// Host side of the C ABI: validation, byte accounting (Eq. 3), arena layout,
// kernel launch order.  No device allocation happens here.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "qevict_internal.h"

using namespace qv;

namespace {

thread_local std::string g_err;

qevict_status fail(qevict_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

#define HIP_TRY(expr)                                                                      \
    do {                                                                                   \
        hipError_t e_ = (expr);                                                            \
        if (e_ != hipSuccess) return fail(QEVICT_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Shape checks for the byte accounting alone (any positive geometry).
qevict_status validate_accounting(const qevict_config* c) {
    if (!c) return fail(QEVICT_E_INVALID, "null config");
    if (c->h_kv < 1 || c->d_head < 4 || c->d_head % 4 || c->window < 1 || c->n_sink < 0 || c->n_local < 0)
        return fail(QEVICT_E_INVALID, "bad geometry");
    if (!(c->quant_frac >= 0.0 && c->quant_frac <= 1.0)) return fail(QEVICT_E_INVALID, "quant_frac must be in [0, 1]");
    if (!(c->budget_frac > 0.0)) return fail(QEVICT_E_INVALID, "budget_frac must be > 0");
    if (c->max_new < 0) return fail(QEVICT_E_INVALID, "max_new must be >= 0");
    return QEVICT_OK;
}

// Shapes the kernels support.
qevict_status validate(const qevict_config* c) {
    if (!c) return fail(QEVICT_E_INVALID, "null config");
    if (c->batch < 1 || c->n_layers < 1) return fail(QEVICT_E_INVALID, "batch and n_layers must be >= 1");
    if ((int64_t)c->batch * c->n_layers > MIG_MAX_UNITS)
        return fail(QEVICT_E_INVALID, "batch * n_layers must be <= %d", MIG_MAX_UNITS);
    if (c->h_kv < 1 || c->h_q < c->h_kv || c->h_q % c->h_kv) return fail(QEVICT_E_INVALID, "h_q must be a multiple of h_kv");
    int G = c->h_q / c->h_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return fail(QEVICT_E_INVALID, "h_q / h_kv must be 1, 2, 4 or 8");
    if (c->h_q > 64) return fail(QEVICT_E_INVALID, "h_q must be <= 64");
    if (c->d_head != 64 && c->d_head != 128) return fail(QEVICT_E_INVALID, "d_head must be 64 or 128");
    if (c->window != 16 && c->window != 32 && c->window != 64) return fail(QEVICT_E_INVALID, "window must be 16, 32 or 64");
    if (c->n_sink < 0 || c->n_sink > 64) return fail(QEVICT_E_INVALID, "n_sink must be in [0, 64]");
    if (c->n_local < 0) return fail(QEVICT_E_INVALID, "n_local must be >= 0");
    if (c->omega < 1) return fail(QEVICT_E_INVALID, "omega must be >= 1");
    {
        const uint32_t rk = c->flags & (QEVICT_F_RANK_DECAY | QEVICT_F_RANK_PNORM | QEVICT_F_RANK_KEYNORM);
        if (rk & (rk - 1)) return fail(QEVICT_E_INVALID, "at most one ranker flag");
    }
    if (!(c->quant_frac >= 0.0 && c->quant_frac <= 1.0)) return fail(QEVICT_E_INVALID, "quant_frac must be in [0, 1]");
    if (!(c->budget_frac > 0.0)) return fail(QEVICT_E_INVALID, "budget_frac must be > 0");
    if (c->max_prompt < 0 || c->max_new < 0) return fail(QEVICT_E_INVALID, "max_prompt / max_new must be >= 0");
    if (c->n_splits < 0) return fail(QEVICT_E_INVALID, "n_splits must be >= 0");
    return QEVICT_OK;
}

struct Caps {
    int32_t K_f, K_q;
    double B_total, B_hist;
    int64_t M_f, M_q;
};

qevict_status caps_of(const qevict_config* c, int32_t prompt_len, Caps* out) {
    const int64_t b_tok = 4LL * c->h_kv * c->d_head;
    const double B_total = c->budget_frac * (double)b_tok * (double)(prompt_len + c->max_new);
    const double B_hist = B_total - (double)((int64_t)(c->n_sink + c->n_local) * b_tok);
    const int64_t W = c->window, H = c->h_kv, d = c->d_head;
    const int64_t M_f = W * b_tok + 8;
    const int64_t qb = (c->flags & QEVICT_F_INT4) ? 4 : 2;   // bits per code
    const int64_t M_q = 2 * W * H * d * qb / 8 + 4 * H * d + 4 * W * H + 4 + 16;
    out->B_total = B_total;
    out->B_hist = B_hist;
    out->M_f = M_f;
    out->M_q = M_q;
    if (B_hist < 0) return fail(QEVICT_E_BUDGET, "B_hist = %.1f < 0: the protected regions exceed the budget", B_hist);
    out->K_f = (int32_t)std::floor((1.0 - c->quant_frac) * B_hist / (double)M_f);
    out->K_q = (int32_t)std::floor(c->quant_frac * B_hist / (double)M_q);
    return QEVICT_OK;
}

constexpr int O_COUNT_MAX = 32;
struct Layout {
    Geo g;
    size_t off[O_COUNT_MAX];
    size_t total;
    size_t export_bytes;
    int32_t max_kf, max_kq;
};

enum { O_HDR, O_WIN, O_SCORE, O_ACC, O_SPLITS, O_FPAGE, O_FSLOT, O_PACK, O_FILL, O_TARGET, O_LSEW, O_LSEG,
       O_PML, O_PACC, O_PAGES, O_SLOTS, O_SINKS, O_PLENS, O_KF, O_KQ, O_SBLK, O_UACC, O_ROPE, O_KROT, O_UARR,
       O_COUNT };

qevict_status make_layout(const qevict_config* c, const int32_t* prompt_lens, Layout* lay) {
    qevict_status s = validate(c);
    if (s) return s;
    if (!prompt_lens) return fail(QEVICT_E_INVALID, "null prompt_lens");
    int32_t max_kf = 0, max_kq = 0;
    for (int b = 0; b < c->batch; ++b) {
        if (prompt_lens[b] < 0 || prompt_lens[b] > c->max_prompt)
            return fail(QEVICT_E_INVALID, "prompt_lens[%d] = %d outside [0, %d]", b, prompt_lens[b], c->max_prompt);
        Caps cp;
        s = caps_of(c, prompt_lens[b], &cp);
        if (s) return s;
        max_kf = cp.K_f > max_kf ? cp.K_f : max_kf;
        max_kq = cp.K_q > max_kq ? cp.K_q : max_kq;
    }
    Geo& g = lay->g;
    g.B = c->batch; g.L = c->n_layers; g.h_q = c->h_q; g.h_kv = c->h_kv; g.d = c->d_head; g.W = c->window;
    g.n_sink = c->n_sink; g.n_local = c->n_local; g.omega = c->omega; g.S_max = c->max_prompt; g.flags = c->flags;
    const int64_t span = (int64_t)c->max_prompt + c->max_new + c->omega - c->n_sink;
    g.n_windows = (int32_t)((span > 0 ? (span + g.W - 1) / g.W : 0) + 1);
    if (g.n_windows > 4096) return fail(QEVICT_E_INVALID, "%d windows per unit exceed the router's 4096", g.n_windows);
    const int32_t n_local_pages = (c->n_local + c->omega + g.W - 1) / g.W + 2;
    g.n_pages = max_kf + n_local_pages + 1;
    g.n_slots = max_kq + max_kf + 1;
    g.n_acc_max = 1 + max_kf + max_kq + n_local_pages + 1;
    if (g.n_acc_max > 4096) return fail(QEVICT_E_INVALID, "accessible list of %d exceeds 4096", g.n_acc_max);
    int32_t ns = c->n_splits;
    if (ns == 0) {
        const int32_t par = g.B * g.h_kv;
        ns = (512 + par - 1) / par;
        int32_t cap = g.n_acc_max / 4;
        if (cap < 1) cap = 1;
        if (ns > cap) ns = cap;
        if (ns < 1) ns = 1;
    }
    // the finish kernel stages (m, l) of every split of a head in LDS: at most 512
    const int32_t ns_max = 512;
    if (ns > ns_max) ns = ns_max;
    g.n_splits = ns;
    g.page_elems = g.h_kv * 2 * g.W * g.d;
    g.qbits = (c->flags & QEVICT_F_INT4) ? 4 : 2;
    // one split per (sequence, KV head): the split kernel finishes the step itself
    g.fuse = g.n_splits == 1 && !(c->flags & QEVICT_F_SEPARATE_FINISH);
    g.n_rope = (c->flags & QEVICT_F_ROPE) ? std::max(32, c->max_prompt + c->max_new) : 0;
    g.slot_head_bytes = 2 * lay_code_bytes(g.W, g.d, g.qbits) + 4 * g.d + 4 * g.W;
    g.slot_bytes = g.h_kv * g.slot_head_bytes;
    g.sink_elems = g.h_kv * 2 * sink_width(g.n_sink) * g.d;
    const size_t U = (size_t)g.B * g.L;
    size_t sz[O_COUNT];
    sz[O_HDR] = U * sizeof(UnitHdr);
    sz[O_WIN] = U * g.n_windows * sizeof(WinRec);
    sz[O_SCORE] = U * g.n_windows * sizeof(double);
    sz[O_UACC] = U * g.n_windows * sizeof(double);
    sz[O_ACC] = U * g.n_acc_max * sizeof(AccEntry);
    sz[O_SPLITS] = U * (g.n_splits + 1) * sizeof(int32_t);
    sz[O_FPAGE] = U * g.n_pages * sizeof(int32_t);
    sz[O_FSLOT] = U * g.n_slots * sizeof(int32_t);
    sz[O_PACK] = U * g.n_windows * sizeof(PackItem);
    sz[O_FILL] = U * g.n_windows * sizeof(FillItem);
    sz[O_TARGET] = U * g.n_windows;
    sz[O_LSEW] = U * 2 * g.n_acc_max * g.h_q * sizeof(float);   // two halves by position parity
    sz[O_LSEG] = U * 2 * g.h_q * sizeof(float);                  // two halves by position parity
    sz[O_PML] = U * g.n_splits * g.h_q * sizeof(float2);
    sz[O_PACC] = U * g.n_splits * g.h_q * g.d * sizeof(float);
    sz[O_PAGES] = U * g.n_pages * (size_t)g.page_elems * 2;
    sz[O_SLOTS] = U * g.n_slots * (size_t)g.slot_bytes;
    sz[O_SINKS] = U * (size_t)g.sink_elems * 2;
    sz[O_PLENS] = sz[O_KF] = sz[O_KQ] = g.B * sizeof(int32_t);
    sz[O_SBLK] = U * (size_t)g.n_splits * SPLIT_BLOCK * sizeof(AccEntry);
    sz[O_ROPE] = (size_t)g.n_rope * (g.d / 2) * sizeof(float2);
    sz[O_KROT] = g.n_rope ? U * g.h_kv * (size_t)g.d * 2 : 0;
    sz[O_UARR] = U * sizeof(uint32_t);
    size_t at = 0;
    for (int i = 0; i < O_COUNT; ++i) {
        lay->off[i] = at;
        at += align256(sz[i]);
    }
    lay->total = at;
    lay->export_bytes = 80 + (size_t)g.n_windows * 24 + (size_t)g.n_acc_max * sizeof(AccEntry) +
                        (size_t)(g.n_splits + 1) * 4 + (size_t)g.n_windows * 8 +
                        (size_t)g.n_windows * g.slot_bytes + (size_t)g.n_windows * g.page_elems * 2 +
                        (size_t)g.sink_elems * 2;
    lay->max_kf = max_kf;
    lay->max_kq = max_kq;
    return QEVICT_OK;
}

Bufs bind_bufs(const Layout& lay, void* arena) {
    char* a = (char*)arena;
    Bufs b;
    b.hdr = (UnitHdr*)(a + lay.off[O_HDR]);
    b.win = (WinRec*)(a + lay.off[O_WIN]);
    b.score = (double*)(a + lay.off[O_SCORE]);
    b.uacc = (double*)(a + lay.off[O_UACC]);
    b.acc = (AccEntry*)(a + lay.off[O_ACC]);
    b.splits = (int32_t*)(a + lay.off[O_SPLITS]);
    b.free_pages = (int32_t*)(a + lay.off[O_FPAGE]);
    b.free_slots = (int32_t*)(a + lay.off[O_FSLOT]);
    b.pack = (PackItem*)(a + lay.off[O_PACK]);
    b.fill = (FillItem*)(a + lay.off[O_FILL]);
    b.target = (int8_t*)(a + lay.off[O_TARGET]);
    b.lse_win = (float*)(a + lay.off[O_LSEW]);
    b.lse_glob = (float*)(a + lay.off[O_LSEG]);
    b.part_ml = (float2*)(a + lay.off[O_PML]);
    b.part_acc = (float*)(a + lay.off[O_PACC]);
    b.pages = (uint16_t*)(a + lay.off[O_PAGES]);
    b.slots = (uint8_t*)(a + lay.off[O_SLOTS]);
    b.sinks = (uint16_t*)(a + lay.off[O_SINKS]);
    b.split_blk = (AccEntry*)(a + lay.off[O_SBLK]);
    b.rope = lay.g.n_rope ? (const float2*)(a + lay.off[O_ROPE]) : nullptr;
    b.krot = lay.g.n_rope ? (uint16_t*)(a + lay.off[O_KROT]) : nullptr;
    b.unit_arr = (uint32_t*)(a + lay.off[O_UARR]);
    return b;
}

}  // namespace

namespace qv {
// prefill workspace: row log-sum-exps fp32 [B][h_q][S_max], column sums fp64 [B][h_q][S_max]
size_t prefill_ws_bytes(const Geo& g) {
    const size_t n = (size_t)g.B * g.h_q * g.S_max;
    size_t at = ((n * 4 + 255) & ~size_t(255)) + ((n * 8 + 255) & ~size_t(255));
    if (g.n_rope) at += rope_ws_bytes(g);
    return at;
}

// the RoPE-mode prompt copies in the workspace: queries [B][h_q][S_max][d], then keys
// [B][h_kv][S_max][d] (bf16, rotated)
size_t rope_ws_offset(const Geo& g) {
    const size_t n = (size_t)g.B * g.h_q * g.S_max;
    return ((n * 4 + 255) & ~size_t(255)) + ((n * 8 + 255) & ~size_t(255));
}
size_t rope_ws_bytes(const Geo& g) {
    const size_t nq = (size_t)g.B * g.h_q * g.S_max * g.d * 2, nk = (size_t)g.B * g.h_kv * g.S_max * g.d * 2;
    return ((nq + 255) & ~size_t(255)) + ((nk + 255) & ~size_t(255));
}
}  // namespace qv

struct qevict_state {
    qevict_config cfg;
    Layout lay;
    Bufs bf;
    char* arena;
    std::vector<int32_t> prompt_lens, K_f, K_q;
    std::vector<int32_t> steps;
    std::vector<uint8_t> prefilled;
    std::vector<uint8_t> step_fresh;                      // per layer: a decode step and no routing since
    bool rope_set = false;                                // RoPE mode: table copied in
    hipEvent_t ev_before = nullptr, ev_after = nullptr;   // one-shot timing of the split kernel
    hipEvent_t rev_before = nullptr, rev_after = nullptr; // one-shot timing of a routing event
    int device = -1;                                      // the device current at qevict_create
};

namespace qv {
qevict_status set_error(qevict_status s, const char* msg) { return fail(s, "%s", msg); }
size_t state_prefill_ws_bytes(const qevict_state* st) { return prefill_ws_bytes(st->lay.g); }
int state_device(const qevict_state* st) { return st->device; }
}  // namespace qv

extern "C" {

const char* qevict_last_error(void) { return g_err.c_str(); }

const char* qevict_decode_kernel_name(void) { return "qevict_decode_split"; }

qevict_status qevict_capacities(const qevict_config* cfg, int32_t prompt_len, int32_t* K_f, int32_t* K_q,
                                double* B_total, double* B_hist, int64_t* M_f, int64_t* M_q) {
    qevict_status s = validate_accounting(cfg);
    if (s) return s;
    if (prompt_len < 0) return fail(QEVICT_E_INVALID, "prompt_len < 0");
    Caps c;
    s = caps_of(cfg, prompt_len, &c);
    if (B_total) *B_total = c.B_total;
    if (B_hist) *B_hist = c.B_hist;
    if (M_f) *M_f = c.M_f;
    if (M_q) *M_q = c.M_q;
    if (s) return s;
    if (K_f) *K_f = c.K_f;
    if (K_q) *K_q = c.K_q;
    return QEVICT_OK;
}

qevict_status qevict_plan(const qevict_config* cfg, const int32_t* prompt_lens, qevict_plan_info* out) {
    if (!out) return fail(QEVICT_E_INVALID, "null output");
    Layout lay;
    qevict_status s = make_layout(cfg, prompt_lens, &lay);
    if (s) return s;
    out->arena_bytes = lay.total;
    out->prefill_ws_bytes = prefill_ws_bytes(lay.g);
    out->export_bytes = lay.export_bytes;
    out->n_windows = lay.g.n_windows;
    out->n_pages = lay.g.n_pages;
    out->n_slots = lay.g.n_slots;
    out->n_acc_max = lay.g.n_acc_max;
    out->n_splits = lay.g.n_splits;
    out->max_K_f = lay.max_kf;
    out->max_K_q = lay.max_kq;
    out->combine_in_kernel = lay.g.fuse;
    return QEVICT_OK;
}

qevict_status qevict_create(const qevict_config* cfg, const int32_t* prompt_lens, void* arena, size_t arena_bytes,
                            void* stream, qevict_state** out) {
    if (!out) return fail(QEVICT_E_INVALID, "null output handle");
    *out = nullptr;
    Layout lay;
    qevict_status s = make_layout(cfg, prompt_lens, &lay);
    if (s) return s;
    if (!arena) return fail(QEVICT_E_INVALID, "null arena");
    if ((uintptr_t)arena % 256) return fail(QEVICT_E_INVALID, "arena must be 256-byte aligned");
    if (arena_bytes < lay.total)
        return fail(QEVICT_E_CAPACITY, "arena of %zu bytes < %zu required", arena_bytes, lay.total);
    int device = -1;
    HIP_TRY(hipGetDevice(&device));
    qevict_state* st = new qevict_state();
    st->device = device;
    st->cfg = *cfg;
    st->lay = lay;
    st->arena = (char*)arena;
    st->bf = bind_bufs(lay, arena);
    st->prompt_lens.assign(prompt_lens, prompt_lens + cfg->batch);
    st->K_f.resize(cfg->batch);
    st->K_q.resize(cfg->batch);
    for (int b = 0; b < cfg->batch; ++b) {
        Caps c;
        caps_of(cfg, prompt_lens[b], &c);
        st->K_f[b] = c.K_f;
        st->K_q[b] = c.K_q;
    }
    st->steps.assign(cfg->n_layers, 0);
    st->prefilled.assign(cfg->n_layers, 0);
    st->step_fresh.assign(cfg->n_layers, 0);
    hipStream_t hs = (hipStream_t)stream;
    char* a = (char*)arena;
    hipError_t e = hipMemcpyAsync(a + lay.off[O_PLENS], st->prompt_lens.data(), cfg->batch * 4, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess)
        e = hipMemcpyAsync(a + lay.off[O_KF], st->K_f.data(), cfg->batch * 4, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess)
        e = hipMemcpyAsync(a + lay.off[O_KQ], st->K_q.data(), cfg->batch * 4, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess)
        e = launch_init(lay.g, st->bf, (const int32_t*)(a + lay.off[O_PLENS]), (const int32_t*)(a + lay.off[O_KF]),
                        (const int32_t*)(a + lay.off[O_KQ]), hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);   // host vectors above are pageable
    if (e != hipSuccess) {
        delete st;
        return fail(QEVICT_E_HIP, "init: %s", hipGetErrorString(e));
    }
    *out = st;
    return QEVICT_OK;
}

void qevict_destroy(qevict_state* st) { delete st; }

static qevict_status check_layer(qevict_state* st, int32_t layer, bool allow_all) {
    if (!st) return fail(QEVICT_E_INVALID, "null state");
    if (allow_all && layer == -1) return QEVICT_OK;
    if (layer < 0 || layer >= st->cfg.n_layers) return fail(QEVICT_E_INVALID, "layer %d out of range", layer);
    return QEVICT_OK;
}

qevict_status qevict_prefill_init(qevict_state* st, int32_t layer, const void* q_prompt, const void* k_prompt,
                                  const void* v_prompt, const double* score_init, void* workspace, size_t ws_bytes,
                                  void* stream) {
    qevict_status s = check_layer(st, layer, false);
    if (s) return s;
    if (st->prefilled[layer]) return fail(QEVICT_E_STATE, "layer %d already initialised", layer);
    if (st->cfg.max_prompt > 0 && (!k_prompt || !v_prompt))
        return fail(QEVICT_E_INVALID, "null prompt key/value buffer");
    const Geo& g = st->lay.g;
    const bool rope = (g.flags & QEVICT_F_ROPE) != 0;
    if (rope && !st->rope_set) return fail(QEVICT_E_STATE, "RoPE mode: qevict_set_rope must come before prefill");
    if (!score_init && st->cfg.max_prompt > 0 && !q_prompt) return fail(QEVICT_E_INVALID, "null prompt query buffer");
    if (!score_init || rope) {
        if (ws_bytes < prefill_ws_bytes(g) || (!workspace && prefill_ws_bytes(g)))
            return fail(QEVICT_E_CAPACITY, "prefill workspace of %zu bytes < %zu required", ws_bytes,
                        prefill_ws_bytes(g));
    }
    hipStream_t hs = (hipStream_t)stream;
    const uint16_t *qp = (const uint16_t*)q_prompt, *kp = (const uint16_t*)k_prompt;
    if (rope) HIP_TRY(launch_rope_prompt(g, st->bf, score_init ? nullptr : qp, kp, workspace, &qp, &kp, hs));
    HIP_TRY(launch_prefill_setup(g, st->bf, layer, kp, (const uint16_t*)v_prompt, hs));
    HIP_TRY(launch_prefill_scores(g, st->bf, layer, qp, kp, score_init, workspace, hs));
    HIP_TRY(launch_route(g, st->bf, layer, RM_PREFILL, kp, (const uint16_t*)v_prompt, hs));
    st->prefilled[layer] = 1;
    st->steps[layer] = 0;
    return QEVICT_OK;
}

qevict_status qevict_decode_attn(qevict_state* st, int32_t layer, const void* q, const void* k_new, const void* v_new,
                                 float* out, void* stream) {
    qevict_status s = check_layer(st, layer, false);
    if (s) return s;
    if (!st->prefilled[layer]) return fail(QEVICT_E_STATE, "layer %d has no prefill", layer);
    if (!q || !k_new || !v_new || !out) return fail(QEVICT_E_INVALID, "null decode buffer");
    if (st->steps[layer] >= st->cfg.max_new)
        return fail(QEVICT_E_CAPACITY, "layer %d already decoded max_new = %d tokens", layer, st->cfg.max_new);
    hipStream_t hs = (hipStream_t)stream;
    const Geo& g = st->lay.g;
    // Eq. 1 accumulates every step; with QEVICT_F_SCORE_ROUTE_ONLY only on the steps that end
    // a routing interval
    const int j = st->steps[layer];
    const int score_now = (!(g.flags & QEVICT_F_SCORE_ROUTE_ONLY) || (j + 1) % g.omega == 0) &&
                          !(g.flags & QEVICT_F_RANK_KEYNORM);   // the key-norm ranker uses no mass
    HIP_TRY(launch_decode(g, st->bf, layer, (const uint16_t*)q, (const uint16_t*)k_new, (const uint16_t*)v_new, out,
                          score_now, hs, st->ev_before, st->ev_after));
    st->ev_before = st->ev_after = nullptr;
    if (!g.fuse)
        HIP_TRY(launch_finish(g, st->bf, layer, out, (const uint16_t*)k_new, (const uint16_t*)v_new, score_now, hs));
    st->steps[layer] += 1;
    st->step_fresh[layer] = 1;
    return QEVICT_OK;
}

qevict_status qevict_set_rope(qevict_state* st, const float* cos_sin, int32_t n_pos, void* stream) {
    if (!st) return fail(QEVICT_E_INVALID, "null state");
    const Geo& g = st->lay.g;
    if (!(g.flags & QEVICT_F_ROPE)) return fail(QEVICT_E_STATE, "the state was created without QEVICT_F_ROPE");
    if (!cos_sin) return fail(QEVICT_E_INVALID, "null RoPE table");
    if (n_pos < g.n_rope)
        return fail(QEVICT_E_INVALID, "RoPE table of %d positions < %d needed (max(32, max_prompt + max_new))", n_pos,
                    g.n_rope);
    HIP_TRY(hipMemcpyAsync(st->arena + st->lay.off[O_ROPE], cos_sin, (size_t)g.n_rope * (g.d / 2) * sizeof(float2),
                           hipMemcpyDefault, (hipStream_t)stream));
    st->rope_set = true;
    return QEVICT_OK;
}

qevict_status qevict_stream_read(const void* buf, size_t bytes, void* sink, void* ev_before, void* ev_after,
                                 void* stream) {
    if (!buf || !sink) return fail(QEVICT_E_INVALID, "null buffer or sink");
    if (bytes == 0 || bytes % 1024 != 0 || bytes >= ((size_t)1 << 31))
        return fail(QEVICT_E_INVALID, "bytes must be a positive multiple of 1024 below 2^31 (got %zu)", bytes);
    if (((uintptr_t)buf & 15) != 0) return fail(QEVICT_E_INVALID, "buffer not 16-byte aligned");
    if ((ev_before == nullptr) != (ev_after == nullptr)) return fail(QEVICT_E_INVALID, "give both events or neither");
    HIP_TRY(launch_stream_read(buf, (uint32_t)bytes, (uint32_t*)sink, (hipStream_t)stream, (hipEvent_t)ev_before,
                               (hipEvent_t)ev_after));
    return QEVICT_OK;
}

qevict_status qevict_time_next_decode(qevict_state* st, void* ev_before, void* ev_after) {
    if (!st) return fail(QEVICT_E_INVALID, "null state");
    if ((ev_before == nullptr) != (ev_after == nullptr)) return fail(QEVICT_E_INVALID, "give both events or neither");
    st->ev_before = (hipEvent_t)ev_before;
    st->ev_after = (hipEvent_t)ev_after;
    return QEVICT_OK;
}

qevict_status qevict_time_next_route(qevict_state* st, void* ev_before, void* ev_after) {
    if (!st) return fail(QEVICT_E_INVALID, "null state");
    if ((ev_before == nullptr) != (ev_after == nullptr)) return fail(QEVICT_E_INVALID, "give both events or neither");
    st->rev_before = (hipEvent_t)ev_before;
    st->rev_after = (hipEvent_t)ev_after;
    return QEVICT_OK;
}

qevict_status qevict_step_bytes(qevict_state* st, int32_t layer, int64_t* kv_bytes, int64_t* io_bytes, void* stream) {
    qevict_status s = check_layer(st, layer, false);
    if (s) return s;
    if (!kv_bytes || !io_bytes) return fail(QEVICT_E_INVALID, "null output");
    const Geo& g = st->lay.g;
    HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
    int64_t kv = 0;
    std::vector<WinRec> win(g.n_windows);
    for (int b = 0; b < g.B; ++b) {
        const int64_t u = unit_of(g, b, layer);
        UnitHdr hdr;
        HIP_TRY(hipMemcpy(&hdr, st->bf.hdr + u, sizeof hdr, hipMemcpyDeviceToHost));
        HIP_TRY(hipMemcpy(win.data(), st->bf.win + u * g.n_windows, win.size() * sizeof(WinRec), hipMemcpyDeviceToHost));
        const int n = hdr.n + 1;   // the next step attends over one more token
        const int64_t tok = 4LL * g.h_kv * g.d;
        kv += (int64_t)(n < g.n_sink ? n : g.n_sink) * tok;
        for (int w = 0; w < g.n_windows; ++w) {
            const int start = g.n_sink + w * g.W;
            if (start >= n) break;
            const int ntok = n - start < g.W ? n - start : g.W;
            if (win[w].state == ST_LOCAL || win[w].state == ST_FULL) kv += (int64_t)ntok * tok;
            else if (win[w].state == ST_QUANT) kv += g.slot_bytes;
        }
        kv += 32LL * hdr.n_acc;    // accessible-list entry (16 B) + window score read and write (fp64)
    }
    *kv_bytes = kv;
    *io_bytes = (int64_t)g.B * g.h_q * g.d * (2 + 4) + 2LL * g.B * g.h_kv * g.d * 2;   // q in, o out, k/v in
    return QEVICT_OK;
}

qevict_status qevict_route(qevict_state* st, int32_t layer, void* stream) {
    qevict_status s = check_layer(st, layer, true);
    if (s) return s;
    for (int l = 0; l < st->cfg.n_layers; ++l)
        if ((layer == -1 || layer == l) && !st->prefilled[l]) return fail(QEVICT_E_STATE, "layer %d has no prefill", l);
    hipStream_t hs = (hipStream_t)stream;
    HIP_TRY(launch_route(st->lay.g, st->bf, layer, RM_ROUTE, nullptr, nullptr, hs, st->rev_before, st->rev_after));
    st->rev_before = st->rev_after = nullptr;
    for (int l = 0; l < st->cfg.n_layers; ++l)
        if (layer == -1 || layer == l) st->step_fresh[l] = 0;
    return QEVICT_OK;
}

qevict_status qevict_step_mass(qevict_state* st, int32_t layer, int32_t b, double* out, void* stream) {
    qevict_status s = check_layer(st, layer, false);
    if (s) return s;
    if (b < 0 || b >= st->cfg.batch) return fail(QEVICT_E_INVALID, "sequence %d outside [0, %d)", b, st->cfg.batch);
    if (!out) return fail(QEVICT_E_INVALID, "null output");
    if (!st->step_fresh[layer])
        return fail(QEVICT_E_STATE, "layer %d: no decode step since the last prefill / routing", layer);
    HIP_TRY(launch_step_mass(st->lay.g, st->bf, layer, b, out, (hipStream_t)stream));
    return QEVICT_OK;
}

static qevict_status forced(qevict_state* st, int32_t layer, const int32_t* win_ids, int32_t n, int mode,
                            void* stream) {
    qevict_status s = check_layer(st, layer, false);
    if (s) return s;
    if (!st->prefilled[layer]) return fail(QEVICT_E_STATE, "layer %d has no prefill", layer);
    if (n < 0 || (n > 0 && !win_ids)) return fail(QEVICT_E_INVALID, "bad window list");
    if (n == 0) return QEVICT_OK;
    hipStream_t hs = (hipStream_t)stream;
    HIP_TRY(launch_force_targets(st->lay.g, st->bf, layer, win_ids, n, mode == RM_FORCE_Q ? ST_QUANT : ST_FULL, hs));
    HIP_TRY(launch_route(st->lay.g, st->bf, layer, mode, nullptr, nullptr, hs));
    st->step_fresh[layer] = 0;
    return QEVICT_OK;
}

qevict_status qevict_pack_int2(qevict_state* st, int32_t layer, const int32_t* win_ids, int32_t n, void* stream) {
    return forced(st, layer, win_ids, n, RM_FORCE_Q, stream);
}

qevict_status qevict_promote(qevict_state* st, int32_t layer, const int32_t* win_ids, int32_t n, void* stream) {
    return forced(st, layer, win_ids, n, RM_FORCE_F, stream);
}

qevict_status qevict_poll_status(qevict_state* st, uint32_t* status, void* stream) {
    if (!st || !status) return fail(QEVICT_E_INVALID, "null argument");
    const Geo& g = st->lay.g;
    const size_t U = (size_t)g.B * g.L;
    std::vector<UnitHdr> h(U);
    HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
    HIP_TRY(hipMemcpy(h.data(), st->bf.hdr, U * sizeof(UnitHdr), hipMemcpyDeviceToHost));
    uint32_t acc = 0;
    for (auto& x : h) acc |= x.status;
    *status = acc;
    return QEVICT_OK;
}

qevict_status qevict_export_unit(qevict_state* st, int32_t layer, int32_t b, void* host_buf, size_t bytes,
                                 size_t* written, void* stream) {
    qevict_status s = check_layer(st, layer, false);
    if (s) return s;
    if (b < 0 || b >= st->cfg.batch) return fail(QEVICT_E_INVALID, "sequence %d out of range", b);
    if (!host_buf) return fail(QEVICT_E_INVALID, "null host buffer");
    if (bytes < st->lay.export_bytes) return fail(QEVICT_E_CAPACITY, "export buffer < %zu bytes", st->lay.export_bytes);
    const Geo& g = st->lay.g;
    const int64_t u = unit_of(g, b, layer);
    HIP_TRY(launch_flush_mass(g, st->bf, layer, b, (hipStream_t)stream));
    HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
    UnitHdr hdr;
    std::vector<WinRec> win(g.n_windows);
    std::vector<double> score(g.n_windows);
    std::vector<uint8_t> slots((size_t)g.n_slots * g.slot_bytes);
    std::vector<uint16_t> pages((size_t)g.n_pages * g.page_elems);
    std::vector<uint16_t> sinks(g.sink_elems);
    HIP_TRY(hipMemcpy(&hdr, st->bf.hdr + u, sizeof hdr, hipMemcpyDeviceToHost));
    HIP_TRY(hipMemcpy(win.data(), st->bf.win + u * g.n_windows, win.size() * sizeof(WinRec), hipMemcpyDeviceToHost));
    HIP_TRY(hipMemcpy(score.data(), st->bf.score + u * g.n_windows, score.size() * 8, hipMemcpyDeviceToHost));
    HIP_TRY(hipMemcpy(slots.data(), st->bf.slots + u * (size_t)g.n_slots * g.slot_bytes, slots.size(),
                      hipMemcpyDeviceToHost));
    HIP_TRY(hipMemcpy(pages.data(), st->bf.pages + u * (size_t)g.n_pages * g.page_elems, pages.size() * 2,
                      hipMemcpyDeviceToHost));
    HIP_TRY(hipMemcpy(sinks.data(), st->bf.sinks + u * (size_t)g.sink_elems, sinks.size() * 2, hipMemcpyDeviceToHost));
    const int32_t n_acc = hdr.n_acc < 0 ? 0 : (hdr.n_acc > g.n_acc_max ? g.n_acc_max : hdr.n_acc);
    std::vector<AccEntry> acc(n_acc);
    std::vector<int32_t> splits(g.n_splits + 1);
    if (n_acc)
        HIP_TRY(hipMemcpy(acc.data(), st->bf.acc + u * g.n_acc_max, n_acc * sizeof(AccEntry), hipMemcpyDeviceToHost));
    HIP_TRY(hipMemcpy(splits.data(), st->bf.splits + u * (g.n_splits + 1), splits.size() * 4, hipMemcpyDeviceToHost));

    // the records index the host copies of the pools below: a page or slot id outside its pool
    // (a device state that no kernel of this library writes) is reported, not followed
    for (int w = 0; w < g.n_windows; ++w)
        if (win[w].page < -1 || win[w].page >= g.n_pages || win[w].slot < -1 || win[w].slot >= g.n_slots)
            return fail(QEVICT_E_STATE, "device state of layer %d, sequence %d: window %d names page %d / slot %d",
                        layer, b, w, win[w].page, win[w].slot);
    char* o = (char*)host_buf;
    size_t at = 0;
    auto put = [&](const void* p, size_t nb) {
        memcpy(o + at, p, nb);
        at += nb;
    };
    // windows created = those whose first position is below n
    int32_t n_created = 0;
    if (hdr.n > g.n_sink) n_created = (hdr.n - g.n_sink + g.W - 1) / g.W;
    if (n_created > g.n_windows) n_created = g.n_windows;
    int32_t head[20] = {0x58564551, hdr.n, n_created, hdr.K_f, hdr.K_q, (int32_t)hdr.status};
    for (int i = 0; i < 8; ++i) head[6 + i] = hdr.ctr[i];
    head[14] = hdr.n_acc;
    head[15] = hdr.prompt_len;
    memcpy(&head[16], &hdr.sink_mass, 8);
    head[18] = hdr.paired;
    put(head, sizeof head);
    for (int w = 0; w < n_created; ++w) {
        int32_t rec[4] = {win[w].state, (win[w].flags & WF_LEDGER) ? 1 : 0, (win[w].flags & WF_DORMANT) ? 1 : 0,
                          g.n_sink + w * g.W};
        put(rec, sizeof rec);
        put(&score[w], 8);
    }
    // the accessible list as the decode kernels read it, its split offsets, and the page /
    // slot id of every created window (so that each entry can be checked against its window)
    for (const AccEntry& e : acc) {
        int32_t rec[4] = {e.kind, e.idx, e.win, e.start};
        put(rec, sizeof rec);
    }
    put(splits.data(), splits.size() * 4);
    for (int w = 0; w < n_created; ++w) {
        int32_t ids[2] = {win[w].page, win[w].slot};
        put(ids, sizeof ids);
    }
    std::vector<uint8_t> canon(g.slot_bytes);
    for (int w = 0; w < n_created; ++w)
        if ((win[w].flags & WF_LEDGER) && win[w].slot >= 0) {
            const uint8_t* sl = slots.data() + (size_t)win[w].slot * g.slot_bytes;
            std::fill(canon.begin(), canon.end(), 0);
            for (int h = 0; h < g.h_kv; ++h) {
                const uint8_t* src = sl + (size_t)h * g.slot_head_bytes;
                uint8_t* dst = canon.data() + (size_t)h * g.slot_head_bytes;
                const int qb = g.qbits, P = 8 / qb, mask = (1 << qb) - 1;
                const int cb = lay_code_bytes(g.W, g.d, qb);
                for (int t = 0; t < g.W; ++t)
                    for (int c = 0; c < g.d; ++c) {
                        const int kc = (src[lay_kc_byte(t, c, g.d, g.W, qb, (g.flags & QEVICT_F_ROPE) != 0)] >>
                                        lay_kc_shift(c, qb)) & mask;
                        const int vc = (src[cb + lay_vc_byte(t, c, g.d, g.W, qb)] >> lay_vc_shift(t, qb)) & mask;
                        dst[t * (g.d / P) + c / P] |= (uint8_t)(kc << (qb * (c % P)));
                        dst[cb + t * (g.d / P) + c / P] |= (uint8_t)(vc << (qb * (c % P)));
                    }
                memcpy(dst + 2 * cb, src + 2 * cb, (size_t)4 * g.d);     // K offset, K scale
                const uint16_t* ov = (const uint16_t*)(src + 2 * cb + 4 * g.d);
                uint16_t* dv = (uint16_t*)(dst + 2 * cb + 4 * g.d);
                for (int t = 0; t < g.W; ++t) {
                    dv[t] = ov[lay_vp(t, g.W)];
                    dv[g.W + t] = ov[g.W + lay_vp(t, g.W)];
                }
            }
            put(canon.data(), g.slot_bytes);
        }
    // pages: device layout -> [K/V][h][W][d], tokens >= ntok zeroed
    std::vector<uint16_t> tmp(g.page_elems);
    const int Ws = sink_width(g.n_sink);
    auto unpage = [&](const uint16_t* pg, int Wp, int ntok, uint16_t* dst) {
        for (int kv = 0; kv < 2; ++kv)
            for (int h = 0; h < g.h_kv; ++h) {
                const uint16_t* blk = pg + (size_t)(h * 2 + kv) * Wp * g.d;
                for (int i = 0; i < Wp; ++i)
                    for (int c = 0; c < g.d; ++c) {
                        const int o = kv == 0 ? lay_k(i, c, g.d, Wp) : lay_v(i, c, g.d, Wp);
                        dst[((size_t)(kv * g.h_kv + h) * Wp + i) * g.d + c] = i < ntok ? blk[o] : 0;
                    }
            }
    };
    for (int w = 0; w < n_created; ++w) {
        const int st_ = win[w].state;
        if ((st_ == ST_LOCAL || st_ == ST_FULL) && win[w].page >= 0) {
            int ntok = hdr.n - (g.n_sink + w * g.W);
            if (ntok > g.W) ntok = g.W;
            unpage(pages.data() + (size_t)win[w].page * g.page_elems, g.W, ntok, tmp.data());
            put(tmp.data(), (size_t)g.page_elems * 2);
        }
    }
    {
        std::vector<uint16_t> sk((size_t)2 * g.h_kv * Ws * g.d);
        unpage(sinks.data(), Ws, hdr.n < g.n_sink ? hdr.n : g.n_sink, sk.data());
        // keep the first n_sink tokens of each block
        std::vector<uint16_t> out((size_t)2 * g.h_kv * g.n_sink * g.d);
        for (int b2 = 0; b2 < 2 * g.h_kv; ++b2)
            memcpy(out.data() + (size_t)b2 * g.n_sink * g.d, sk.data() + (size_t)b2 * Ws * g.d,
                   (size_t)g.n_sink * g.d * 2);
        put(out.data(), out.size() * 2);
    }
    if (written) *written = at;
    return QEVICT_OK;
}

}  // extern "C"
