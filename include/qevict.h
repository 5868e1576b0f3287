/*
 * qevict.h — C ABI of the MI355X (gfx950) QEvict decode hot path.
 *
 * QEvict keeps a per-layer KV cache as a protected sink prefix, a protected
 * recent region and fixed-size windows of W tokens, each window in one of
 * three tiers: Full (bf16), Quantized (INT2, recoverable) or Evicted.
 * Source: "QEvict: Recoverable Quantized KV Eviction for Attention-Drift-Robust
 * Long-Context Decoding" (arXiv 2608.05326), §4.1-§4.3 and Appendix A
 * (Algorithm 1); byte accounting Appendix B.4.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked [host].
 *   - The caller owns all memory.  The library never allocates device memory:
 *     qevict_plan() reports the sizes, the caller allocates them (e.g. with
 *     PyTorch) and passes them in.  Host-side bookkeeping (the qevict_state
 *     object, a few hundred bytes) is the only allocation the library makes.
 *   - Work is enqueued on the caller's `stream` (a hipStream_t, passed as
 *     void*; NULL = the default stream).  Only the calls marked "syncs" wait.
 *   - Argument and shape errors return a negative qevict_status at once and
 *     enqueue nothing; qevict_last_error() then holds a message for the
 *     calling thread.  Errors found on the device (pool overflow, a decode
 *     step that runs past the windows prepared by the last route, an fp16
 *     range overflow while quantizing) set bits of a per-(sequence, layer)
 *     status word that qevict_poll_status() reads.
 *   - bf16 tensors are raw 16-bit bfloat16 values; fp32 outputs are IEEE float.
 *   - Calls for different layers touch disjoint state and may run on different
 *     streams concurrently; calls for one layer must be ordered on one stream.
 */
#ifndef QEVICT_H
#define QEVICT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QEVICT_OK = 0,
    QEVICT_E_INVALID = -1,   /* bad argument, unsupported shape */
    QEVICT_E_BUDGET = -2,    /* protected regions exceed the budget: B_hist < 0 (§4.3 Eq. 3) */
    QEVICT_E_CAPACITY = -3,  /* a buffer is smaller than qevict_plan() requires */
    QEVICT_E_RANGE = -4,     /* value outside the fp16 range of the quantization parameters */
    QEVICT_E_STATE = -5,     /* call out of order (e.g. decode before prefill) */
    QEVICT_E_HIP = -6        /* a HIP runtime call failed */
} qevict_status;

/* device status bits (qevict_poll_status) */
#define QEVICT_DEV_E_POOL   1u   /* page or slot pool exhausted */
#define QEVICT_DEV_E_WINDOW 2u   /* decode wrote past the windows prepared by the last route */
#define QEVICT_DEV_E_RANGE  4u   /* |x| > 65504 in a window being quantized */
#define QEVICT_DEV_E_LIST   8u   /* accessible list or work list overflow */
#define QEVICT_DEV_E_SELECT 16u  /* tier selection left open (internal invariant broken) */

/* flags */
#define QEVICT_F_NO_PROMOTE        1u  /* one-way variant Full -> Quantized -> Evicted (App. K) */
#define QEVICT_F_SCORE_ROUTE_ONLY  2u  /* accumulate Eq. 1 only at the routing step itself */
/* Alternative window rankers (App. J), at most one; default: cumulative mass (Eq. 21).
 * u_r(w) is the window's head-averaged mass since the previous routing event (Eq. 20).
 * DECAY:   S <- 0.99 * S + u_r at each decode-time routing event (Eq. 22).
 * PNORM:   the rank key P <- P + u_r^3 (Eq. 23 with p = 3; P orders the windows as
 *          P^(1/3) does), P_0 = S_0^3 from the prefill initialisation.
 * KEYNORM: S(w) = -(mean over the window's tokens of the L2 norm of the token's key over
 *          all KV heads' channels), set when the window enters the candidate pool (Eq. 24);
 *          no attention mass is accumulated. */
#define QEVICT_F_RANK_DECAY        4u
#define QEVICT_F_RANK_PNORM        8u
#define QEVICT_F_RANK_KEYNORM     16u
/* INT4 recoverable tier (App. G.3): 4-bit codes (16 levels, scl = RU_fp16((max - off)/15)),
 * everything else as for INT2; M_q = W*H_kv*d + 4*H_kv*d + 4*W*H_kv + 20 bytes. */
#define QEVICT_F_INT4             32u
/* RoPE-faithful Quantized tier (§4.3 "Migration-Stable Quantization", "Cache Execution"):
 * queries and keys are handed over BEFORE RoPE and the library rotates them with the
 * table given to qevict_set_rope ("rotate half": channel pair (i, i + d/2) of position p
 * turns by the angle whose cos / sin are table[p][i]).  Cached keys (sinks, recent, Full)
 * are bf16 of the exact rotation at their positions; a window's first demotion quantizes
 * its cached keys rotated back to the pre-RoPE domain (exact fp64); attention re-applies
 * RoPE to the dequantized keys at the ledger's positions, and a promotion writes bf16 of
 * that re-rotation. */
#define QEVICT_F_ROPE             64u
/* With one split per (sequence, KV head) (n_splits = 1, the automatic choice once
 * B * h_kv >= 512) a decode step is one kernel launch: each split-kernel workgroup writes its
 * heads' output and log-sum-exps and the step's token itself, and the last of a sequence's
 * h_kv workgroups advances its token count.  This flag keeps the second (finish) launch that
 * otherwise combines the splits. */
#define QEVICT_F_SEPARATE_FINISH 128u

typedef struct {
    int32_t batch;        /* B sequences */
    int32_t n_layers;     /* L */
    int32_t h_q;          /* query heads; h_q % h_kv == 0, h_q / h_kv in {1,2,4,8} */
    int32_t h_kv;         /* KV heads (GQA groups) */
    int32_t d_head;       /* 64 or 128 */
    int32_t window;       /* W tokens per window: 16, 32 or 64 */
    int32_t n_sink;       /* protected sink prefix, 0 < n_sink <= 64 */
    int32_t n_local;      /* R_loc: protected recent tokens (nominal) */
    int32_t omega;        /* routing interval (generated tokens between routing events) */
    double quant_frac;    /* q: share of the historical budget given to the Quantized tier */
    double budget_frac;   /* rho: KV budget as a fraction of the full bf16 cache */
    int32_t max_prompt;   /* S_max: prompt buffers are [..][S_max][d] */
    int32_t max_new;      /* N_g: generated tokens; B_total covers prompt_len + max_new */
    uint32_t flags;       /* QEVICT_F_* */
    int32_t n_splits;     /* decode splits per (sequence, KV head); 0 = choose; capped at 512 */
} qevict_config;

typedef struct {
    size_t arena_bytes;          /* one device buffer holding all persistent state */
    size_t prefill_ws_bytes;     /* device workspace for qevict_prefill_init (reusable across layers) */
    size_t export_bytes;         /* host buffer size for qevict_export_unit */
    int32_t n_windows;           /* window slots per (sequence, layer) */
    int32_t n_pages;             /* bf16 pages per (sequence, layer) */
    int32_t n_slots;             /* INT2 slots per (sequence, layer) */
    int32_t n_acc_max;           /* accessible-list capacity */
    int32_t n_splits;            /* decode splits actually used */
    int32_t max_K_f, max_K_q;    /* largest capacities over the batch */
    int32_t combine_in_kernel;   /* 1: a decode step is one kernel launch (QEVICT_F_SEPARATE_FINISH) */
} qevict_plan_info;

typedef struct qevict_state qevict_state;

/*
 * Tier capacities of one sequence (§4.3 Eq. 3, budget inequality of §4.1):
 *   b_tok   = 4 * h_kv * d_head                       bf16 K+V bytes per token
 *   B_total = budget_frac * b_tok * (prompt_len + max_new)
 *   B_hist  = B_total - (n_sink + n_local) * b_tok
 *   M_f     = W * b_tok + 8
 *   M_q     = W*h_kv*d/2 (codes) + 4*h_kv*d (K off/scl) + 4*W*h_kv (V off/scl) + 4 + 16
 *   K_f     = floor((1 - q) * B_hist / M_f),  K_q = floor(q * B_hist / M_q)
 * All outputs [host].  Returns QEVICT_E_BUDGET when B_hist < 0.  Accepts any
 * positive geometry (accounting only); qevict_plan checks what the kernels support.
 */
qevict_status qevict_capacities(const qevict_config* cfg, int32_t prompt_len,
                                int32_t* K_f, int32_t* K_q, double* B_total, double* B_hist,
                                int64_t* M_f, int64_t* M_q);

/* Sizes of every buffer for `cfg` and the per-sequence prompt lengths
 * prompt_lens[host][batch] (each in [0, max_prompt]).  out [host]. */
qevict_status qevict_plan(const qevict_config* cfg, const int32_t* prompt_lens,
                          qevict_plan_info* out);

/* Bind a state object to a caller-allocated arena of >= plan.arena_bytes
 * (256-byte aligned).  Enqueues the arena's initialisation on `stream`.
 * *out [host] receives a handle owned by the caller (qevict_destroy). */
qevict_status qevict_create(const qevict_config* cfg, const int32_t* prompt_lens,
                            void* arena, size_t arena_bytes, void* stream, qevict_state** out);
void qevict_destroy(qevict_state* st);

/*
 * Prefill of one layer (§4.2, last paragraph: prompt attention initialises the
 * window scores and the first tier assignment).
 *   q_prompt [B][h_q][S_max][d], k_prompt / v_prompt [B][h_kv][S_max][d] bf16;
 *   rows >= prompt_lens[b] are ignored.
 *   score_init: NULL -> S_bar_0(w) = (1/h_q) sum_h sum_{u} sum_{t in w} P_h[u, t],
 *     the causal prompt-attention column sums (MFMA kernels, fp32 inside a
 *     tile, fp64 across tiles); otherwise a device array [B][n_windows] of
 *     fp64 initial scores supplied by the caller (any ranking estimator; the
 *     hierarchy only needs an order, App. J).
 *   workspace: >= plan.prefill_ws_bytes of device scratch, free after the call
 *     completes on `stream`.  When the column sums run it holds, from offset 0,
 *     the row log-sum-exps in log2 units, fp32 [B][h_q][S_max], then (at the
 *     next 256-byte boundary) the per-head column sums, fp64 [B][h_q][S_max].
 *     With QEVICT_F_ROPE it is required also with score_init (it then holds the
 *     rotated prompt queries and keys after those arrays).
 *   With QEVICT_F_ROPE, q_prompt and k_prompt are before RoPE (qevict_set_rope first).
 * Then routes the aged prompt windows (Eqs. 4-5), packs the Quantized ones
 * (INT2 or INT4, write-once) and copies the Full and recent ones into bf16 pages.
 */
qevict_status qevict_prefill_init(qevict_state* st, int32_t layer,
                                  const void* q_prompt, const void* k_prompt, const void* v_prompt,
                                  const double* score_init, void* workspace, size_t ws_bytes,
                                  void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): qevict_prefill_init with the workspace
 * taken from a static device array inside the library, QEVICT_NOALLOC_WS_BYTES (32 MiB)
 * per GPU, held by each GPU the library runs on until the process ends.  Same arguments,
 * results and ordering as qevict_prefill_init otherwise; allocates nothing.
 *   Errors: QEVICT_E_CAPACITY (nothing enqueued) when plan.prefill_ws_bytes exceeds
 *   QEVICT_NOALLOC_WS_BYTES (e.g. a 32K prompt at batch 1 with 32 query heads needs 12 MiB
 *   and fits; RoPE mode at that size does not); QEVICT_E_STATE unless the device current at
 *   qevict_create is current; then the errors of qevict_prefill_init.
 *   Every call on one GPU shares the array: calls that overlap on one GPU (unordered streams,
 *   threads) race; calls ordered on one stream do not.  Nothing in the array needs to start
 *   at zero (each call writes every word it reads), so it is never cleared.
 */
#define QEVICT_NOALLOC_WS_BYTES ((size_t)32 << 20)
qevict_status qevict_prefill_init_noalloc(qevict_state* st, int32_t layer, const void* q_prompt,
                                          const void* k_prompt, const void* v_prompt,
                                          const double* score_init, void* stream);

/*
 * One decode step of one layer (§4.1 accessible-set attention, §4.2 Eq. 1).
 *   q [B][h_q][d], k_new / v_new [B][h_kv][d] bf16: the new token's query, key, value
 *     (query and key before RoPE with QEVICT_F_ROPE; the library turns them to position n).
 *   out [B][h_q][d] fp32: o = softmax(q K_acc^T / sqrt(d)) V_acc over sinks, the
 *     recent region, Full windows (bf16) and Quantized windows (INT2 values
 *     off + code * scl, dequantized in registers).
 * Appends k_new / v_new at position n (recent region), attends, and adds each
 * accessible window's head-averaged attention mass to its score S_bar(w).
 */
qevict_status qevict_decode_attn(qevict_state* st, int32_t layer, const void* q,
                                 const void* k_new, const void* v_new, float* out, void* stream);

/*
 * Routing event (§4.3 Eqs. 4-6, Algorithm 1), for one layer or all (layer = -1).
 * Candidates = Full ∪ Quantized ∪ recent windows whose end is <= n - n_local;
 * ordered by (S_bar descending, window index ascending); the first K_f become
 * Full, the next K_q Quantized, the rest Evicted.  Q->F dequantizes the ledger
 * into a bf16 page and marks it dormant; a first entry into Q packs INT2 codes
 * once; a dormant ledger is reactivated; Evicted windows release everything.
 * Also prepares recent-region windows for the next omega positions and
 * rebuilds the chronological accessible list.  Call after the decode step
 * j with (j + 1) % omega == 0.
 */
qevict_status qevict_route(qevict_state* st, int32_t layer, void* stream);

/*
 * [QEvict] §4.3 and Algorithm 1 (the demotion steps of the migration: Full or aged
 * recent -> Quantized, the ledger written once and reactivated later).
 * Demote chosen windows to the Quantized tier (first time: pack INT2 codes and
 * create the ledger; dormant ledger: reactivate) and release their bf16 pages.
 * win_ids [B][n] int32 device array, -1 = unused entry; windows must be Full
 * or aged recent windows.  Capacities are not enforced here: this is the
 * migration step alone, for callers with their own policy.
 */
qevict_status qevict_pack_int2(qevict_state* st, int32_t layer, const int32_t* win_ids, int32_t n,
                               void* stream);

/* Promote chosen Quantized windows to Full: bf16(off + code*scl), rounded to
 * nearest-even from the exact value, into a free page; the ledger becomes
 * dormant (write-once, §4.3).  win_ids as for qevict_pack_int2. */
qevict_status qevict_promote(qevict_state* st, int32_t layer, const int32_t* win_ids, int32_t n,
                             void* stream);

/* OR of the device status words of every (sequence, layer) into *status [host].  Syncs. */
qevict_status qevict_poll_status(qevict_state* st, uint32_t* status, void* stream);

/*
 * Canonical export of one (sequence b, layer) unit into host_buf [host] of
 * >= plan.export_bytes.  Syncs `stream`.  Layout (little endian):
 *   header 20 x int32: magic 0x58564551, n, n_windows_created, K_f, K_q,
 *     status, counters[8] of the last routing event (aged, promoted, packed,
 *     reactivated, demoted, evicted, n_full, n_quant), n_acc, prompt_len,
 *     fp64 head-averaged prefill attention mass on the sink prefix (2 words),
 *     the count of promotions that took a page a demotion's pack read at the same
 *     routing event (written after that pack), 1 reserved word
 *   per window w < n_windows_created: int32 state (1 recent, 2 Full,
 *     3 Quantized, 4 Evicted), int32 has_ledger, int32 dormant, int32 start_pos,
 *     fp64 score
 *   the accessible list the decode kernels read (Algorithm 1, last step: the
 *     effective cache): n_acc entries of 4 x int32 (kind: 0 sink prefix, 1 bf16
 *     page, 2 Quantized slot; page or slot id; window, -1 for the sinks; first
 *     position), in the device's order (pages spread among the slots), which
 *     includes the recent windows prepared for the next omega positions
 *   the split offsets: (n_splits + 1) x int32, entries [s_i, s_{i+1}) form split i
 *   per window w < n_windows_created: int32 page id, int32 slot id (-1 if none)
 *   per window with a ledger, in window order: per KV head: K codes [W][d/4],
 *     V codes [W][d/4] (element (i,c) at byte c/4, bits 2(c%4)), K off [d],
 *     K scl [d], V off [W], V scl [W] (fp16)
 *   per window in state 1 or 2, in window order: bf16 K [h_kv][W][d] then V
 *   sink K [h_kv][n_sink][d] then V (bf16)
 * *written [host] receives the byte count.
 */
qevict_status qevict_export_unit(qevict_state* st, int32_t layer, int32_t b, void* host_buf,
                                 size_t bytes, size_t* written, void* stream);

/* Profiling aid: the next qevict_decode_attn call launches its split-K
 * attention kernel so that its own dispatch stamps ev_before (a hipEvent_t
 * created with timing) at the kernel's start and ev_after at its end; then
 * both are forgotten.  Both or neither must be given; NULL disables. */
qevict_status qevict_time_next_decode(qevict_state* st, void* ev_before, void* ev_after);

/* Profiling aid: the next qevict_route call launches its routing kernel so that its
 * dispatch stamps ev_before (a hipEvent_t created with timing) at the kernel's start, and
 * its migration kernel so that that dispatch stamps ev_after at its end: the GPU span of
 * the routing event, without event packets of their own in the stream; then both are
 * forgotten.  Both or neither must be given; NULL disables. */
qevict_status qevict_time_next_route(qevict_state* st, void* ev_before, void* ev_after);

/* Bytes the next decode step of `layer` must move, summed over the batch
 * [host outputs]: kv_bytes = bf16 K/V of the sink, recent and Full tokens
 * (4 * h_kv * d per token) + whole INT2 slots of Quantized windows (codes and
 * fp16 parameters) + 32 B per accessible-list entry (the entry and the fp64
 * window score read and written); io_bytes = q in (bf16), o out (fp32), k/v in
 * (bf16).  Syncs. */
qevict_status qevict_step_bytes(qevict_state* st, int32_t layer, int64_t* kv_bytes, int64_t* io_bytes,
                                void* stream);

/* Diagnostics ([QEvict] Appendix I, Eqs. 12-13): per-head attention mass of the last
 * decode step of (layer, sequence b) on the sinks and on each window.
 *   out [h_q][n_windows + 1] fp64, device: column 0 the sinks, column 1 + w window w
 *   (the step's probabilities summed over the window's tokens), 0 for windows the step
 *   did not attend (Evicted, not yet created).  Each row sums to 1 up to rounding.
 * Valid after qevict_decode_attn and before the next routing of that layer
 * (QEVICT_E_STATE otherwise).  Runs on `stream`. */
qevict_status qevict_step_mass(qevict_state* st, int32_t layer, int32_t b, double* out, void* stream);

/* RoPE mode (QEVICT_F_ROPE): copy the rotary table into the state.
 *   cos_sin: [n_pos][d_head/2][2] fp32 (cos, sin) of position p, pair i (channels i and
 *            i + d_head/2), device or host memory, read before the call returns on `stream`;
 *            rows >= max(32, max_prompt + max_new) are needed.
 * Must come before the first qevict_prefill_init.  Errors: QEVICT_E_STATE without the flag,
 * QEVICT_E_INVALID for a null or short table. */
qevict_status qevict_set_rope(qevict_state* st, const float* cos_sin, int32_t n_pos, void* stream);

/* Measurement aid, not part of the method: one launch of a plain streaming read of
 * `bytes` bytes at device address buf (bytes a positive multiple of 1024 below 2^31,
 * buf 16-byte aligned), every byte read once with 16-byte loads over 1024 workgroups of
 * 256 threads, for comparison with the split-K kernel's achieved bandwidth.  sink
 * (device, 1024 uint32, caller-owned) receives the XOR of the 32-bit words each
 * workgroup read; the XOR of all 1024 equals that of the buffer's words.  With
 * ev_before / ev_after (hipEvent_t with timing; both or neither) the kernel's own
 * dispatch stamps its start and end, as for qevict_time_next_decode.  Enqueues on
 * `stream`; argument errors return QEVICT_E_INVALID before anything is enqueued. */
qevict_status qevict_stream_read(const void* buf, size_t bytes, void* sink, void* ev_before, void* ev_after,
                                 void* stream);

/* Name of the dominant decode kernel (the split-K attention), for profilers. */
const char* qevict_decode_kernel_name(void);

/* Message of the last failed call on this thread ("" if none). */
const char* qevict_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* QEVICT_H */
