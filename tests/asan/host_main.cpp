// Driver for the host-side AddressSanitizer / UBSan run of the C ABI (host code only: the
// kernels are stand-ins that do nothing and the "device" arena is host memory).  It walks
// the validation, byte accounting, state bookkeeping and export paths, once over a zeroed
// arena and once over an arena of random bytes (a corrupted device state must not make the
// host read or write out of bounds).  Exits non-zero on a wrong status; the sanitizers
// abort on a memory error or leak.  Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "qevict.h"

static int failures = 0;
#define EXPECT(cond)                                                               \
    do {                                                                           \
        if (!(cond)) {                                                             \
            std::fprintf(stderr, "FAILED %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, \
                         qevict_last_error());                                     \
            ++failures;                                                            \
        }                                                                          \
    } while (0)

static qevict_config base_config() {
    qevict_config c;
    std::memset(&c, 0, sizeof c);
    c.batch = 2;
    c.n_layers = 2;
    c.h_q = 4;
    c.h_kv = 1;
    c.d_head = 64;
    c.window = 16;
    c.n_sink = 4;
    c.n_local = 64;
    c.omega = 8;
    c.quant_frac = 0.7;
    c.budget_frac = 0.4;
    c.max_prompt = 512;
    c.max_new = 64;
    c.flags = 0;
    c.n_splits = 0;
    return c;
}

static void check_plans() {
    const int32_t lens[2] = {512, 300};
    qevict_plan_info info;
    qevict_config c = base_config();
    EXPECT(qevict_plan(&c, lens, &info) == QEVICT_OK);
    EXPECT(info.arena_bytes > 0 && info.export_bytes > 0 && info.n_windows > 0 && info.n_splits > 0);
    // a decode step is one launch exactly when each (sequence, KV head) has one split, unless
    // the flag asks for the finish launch
    EXPECT(info.combine_in_kernel == (info.n_splits == 1));
    {
        qevict_config x = c;
        x.n_splits = 6;
        EXPECT(qevict_plan(&x, lens, &info) == QEVICT_OK && info.combine_in_kernel == 0);
        x.n_splits = 1;
        EXPECT(qevict_plan(&x, lens, &info) == QEVICT_OK && info.combine_in_kernel == 1);
        x.flags = QEVICT_F_SEPARATE_FINISH;
        EXPECT(qevict_plan(&x, lens, &info) == QEVICT_OK && info.combine_in_kernel == 0);
    }
    // every field outside what the kernels support
    struct Bad {
        const char* what;
        void (*edit)(qevict_config&);
    } bad[] = {
        {"d_head", [](qevict_config& x) { x.d_head = 96; }},
        {"window", [](qevict_config& x) { x.window = 24; }},
        {"gqa", [](qevict_config& x) { x.h_q = 6; x.h_kv = 4; }},
        {"n_sink", [](qevict_config& x) { x.n_sink = 65; }},
        {"omega", [](qevict_config& x) { x.omega = 0; }},
        {"quant_frac", [](qevict_config& x) { x.quant_frac = 1.5; }},
        {"budget_frac", [](qevict_config& x) { x.budget_frac = 0.0; }},
        {"batch", [](qevict_config& x) { x.batch = 0; }},
        {"units", [](qevict_config& x) { x.batch = 4097; x.n_layers = 2; }},
        {"rankers", [](qevict_config& x) { x.flags = QEVICT_F_RANK_DECAY | QEVICT_F_RANK_PNORM; }},
    };
    for (auto& b : bad) {
        qevict_config x = base_config();
        b.edit(x);
        std::vector<int32_t> l(x.batch > 0 && x.batch < 5000 ? x.batch : 1, 100);
        const qevict_status s = qevict_plan(&x, l.data(), &info);
        if (s == QEVICT_OK) std::fprintf(stderr, "accepted: %s\n", b.what);
        EXPECT(s != QEVICT_OK);
    }
    const int32_t too_long[2] = {513, 10};
    EXPECT(qevict_plan(&c, too_long, &info) != QEVICT_OK);
    EXPECT(qevict_plan(nullptr, lens, &info) == QEVICT_E_INVALID);
    // capacities: a budget below the protected regions
    int32_t kf, kq;
    double bt, bh;
    int64_t mf, mq;
    qevict_config tight = base_config();
    tight.budget_frac = 0.01;
    EXPECT(qevict_capacities(&tight, 512, &kf, &kq, &bt, &bh, &mf, &mq) == QEVICT_E_BUDGET);
    EXPECT(qevict_capacities(&c, 512, &kf, &kq, &bt, &bh, &mf, &mq) == QEVICT_OK && kf >= 0 && kq >= 0);
}

static void run_state(bool random_fill, uint32_t flags) {
    qevict_config c = base_config();
    c.flags = flags;
    const int32_t lens[2] = {512, 300};
    qevict_plan_info info;
    EXPECT(qevict_plan(&c, lens, &info) == QEVICT_OK);
    void* arena = std::aligned_alloc(256, (info.arena_bytes + 255) / 256 * 256);
    if (random_fill) {
        std::mt19937 rng(1234);
        for (size_t i = 0; i < info.arena_bytes; ++i) static_cast<uint8_t*>(arena)[i] = (uint8_t)rng();
    } else {
        std::memset(arena, 0, info.arena_bytes);
    }
    qevict_state* st = nullptr;
    EXPECT(qevict_create(&c, lens, nullptr, info.arena_bytes, nullptr, &st) == QEVICT_E_INVALID);
    EXPECT(qevict_create(&c, lens, (char*)arena + 16, info.arena_bytes, nullptr, &st) == QEVICT_E_INVALID);
    EXPECT(qevict_create(&c, lens, arena, info.arena_bytes - 1, nullptr, &st) == QEVICT_E_CAPACITY);
    EXPECT(qevict_create(&c, lens, arena, info.arena_bytes, nullptr, &st) == QEVICT_OK && st);
    if (!st) {
        std::free(arena);
        return;
    }
    if (random_fill) {   // the whole arena random again, records included (the stand-in init wrote some)
        std::mt19937 rng(99);
        for (size_t i = 0; i < info.arena_bytes; ++i) static_cast<uint8_t*>(arena)[i] = (uint8_t)rng();
    }
    const size_t S = c.max_prompt, d = c.d_head;
    std::vector<uint16_t> qp(c.batch * c.h_q * S * d), kp(c.batch * c.h_kv * S * d), vp(kp.size());
    std::vector<uint8_t> ws(info.prefill_ws_bytes + 256);
    std::vector<float> rope((size_t)(c.max_prompt + c.max_new + 32) * (d / 2) * 2, 0.5f);
    // out of order: decode and routing before any prefill
    std::vector<uint16_t> q(c.batch * c.h_q * d), k(c.batch * c.h_kv * d), v(k.size());
    std::vector<float> out(c.batch * c.h_q * d);
    EXPECT(qevict_decode_attn(st, 0, q.data(), k.data(), v.data(), out.data(), nullptr) == QEVICT_E_STATE);
    EXPECT(qevict_route(st, -1, nullptr) == QEVICT_E_STATE);
    if (flags & QEVICT_F_ROPE) {
        EXPECT(qevict_prefill_init(st, 0, qp.data(), kp.data(), vp.data(), nullptr, ws.data(), info.prefill_ws_bytes,
                                   nullptr) == QEVICT_E_STATE);
        EXPECT(qevict_set_rope(st, rope.data(), c.max_prompt + c.max_new + 32, nullptr) == QEVICT_OK);
    } else {
        EXPECT(qevict_set_rope(st, rope.data(), 1000, nullptr) == QEVICT_E_STATE);
    }
    EXPECT(qevict_prefill_init(st, 2, qp.data(), kp.data(), vp.data(), nullptr, ws.data(), info.prefill_ws_bytes,
                               nullptr) == QEVICT_E_INVALID);
    EXPECT(qevict_prefill_init(st, 0, qp.data(), kp.data(), vp.data(), nullptr, ws.data(), info.prefill_ws_bytes - 1,
                               nullptr) == QEVICT_E_CAPACITY);
    for (int l = 0; l < c.n_layers; ++l)
        EXPECT(qevict_prefill_init(st, l, qp.data(), kp.data(), vp.data(), nullptr, ws.data(), info.prefill_ws_bytes,
                                   nullptr) == QEVICT_OK);
    std::vector<uint8_t> exp(info.export_bytes);
    std::vector<double> mass((size_t)c.h_q * (info.n_windows + 1));
    for (int j = 0; j < 2 * c.omega; ++j) {
        for (int l = 0; l < c.n_layers; ++l)
            EXPECT(qevict_decode_attn(st, l, q.data(), k.data(), v.data(), out.data(), nullptr) == QEVICT_OK);
        EXPECT(qevict_step_mass(st, 1, 1, mass.data(), nullptr) == QEVICT_OK);
        EXPECT(qevict_step_mass(st, 1, 2, mass.data(), nullptr) == QEVICT_E_INVALID);
        if ((j + 1) % c.omega == 0) EXPECT(qevict_route(st, -1, nullptr) == QEVICT_OK);
    }
    for (int l = 0; l < c.n_layers; ++l)
        for (int b = 0; b < c.batch; ++b) {
            size_t written = 0;
            const qevict_status s = qevict_export_unit(st, l, b, exp.data(), exp.size(), &written, nullptr);
            // (random records name pages / slots outside the pools: reported, not followed)
            EXPECT(random_fill ? (s == QEVICT_OK || s == QEVICT_E_STATE) : s == QEVICT_OK);
            EXPECT(written <= exp.size());
        }
    size_t written = 0;
    EXPECT(qevict_export_unit(st, 0, 0, exp.data(), exp.size() - 1, &written, nullptr) == QEVICT_E_CAPACITY);
    EXPECT(qevict_export_unit(st, 0, 2, exp.data(), exp.size(), &written, nullptr) == QEVICT_E_INVALID);
    uint32_t status = 0;
    EXPECT(qevict_poll_status(st, &status, nullptr) == QEVICT_OK);
    int64_t kvb = 0, iob = 0;
    EXPECT(qevict_step_bytes(st, 0, &kvb, &iob, nullptr) == QEVICT_OK);
    std::vector<int32_t> ids(c.batch * 2, -1);
    ids[0] = 0;
    EXPECT(qevict_pack_int2(st, 0, ids.data(), 2, nullptr) == QEVICT_OK);
    EXPECT(qevict_promote(st, 0, ids.data(), 2, nullptr) == QEVICT_OK);
    EXPECT(qevict_pack_int2(st, 0, nullptr, 2, nullptr) == QEVICT_E_INVALID);
    qevict_destroy(st);
    std::free(arena);
}

int main() {
    check_plans();
    run_state(false, 0);
    run_state(true, 0);
    run_state(false, QEVICT_F_ROPE);
    run_state(true, QEVICT_F_INT4 | QEVICT_F_NO_PROMOTE);
    if (failures) {
        std::fprintf(stderr, "%d failure(s)\n", failures);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
