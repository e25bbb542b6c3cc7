/*
 * growpage.h - C ABI of the GrowPage capacity-boundary event on MI355X.
 *
 * GrowPage ("GrowPage: On-Demand KV Budgeting for Efficient LLM Reasoning
 * Serving", arXiv 2609.03494) decides at each KV capacity boundary of a
 * request whether to compress its cache in place ("Compress & Hold") or to
 * take one more physical page ("Grow by One Page").  This library runs that
 * boundary event on the GPU for a batch of requests over a paged KV cache.
 * Section, equation and appendix numbers below refer to that paper.
 *
 * Conventions
 *  - Ownership: the caller allocates and owns every buffer (device pool,
 *    query-state pool, block tables, free-page stack, workspace, outputs)
 *    and the stream.  The library borrows raw pointers for the duration of
 *    the enqueue.  gp_create allocates a few bytes of device memory for
 *    counters and an error word; no other call allocates.
 *  - Asynchrony: every gp_* call that takes a stream enqueues kernels on it
 *    and returns after host-side validation; results are valid once the
 *    stream has reached that point.  No call synchronises the device except
 *    gp_get_counters, gp_get_device_errors and gp_profile_read.  The event
 *    calls (gp_update_summaries, gp_demand, gp_grow_page, gp_compress_hold,
 *    gp_decode_attention) enqueue kernels only (no allocation, memset or
 *    copy), so a caller may capture them in a HIP graph; the host-side
 *    validation then runs once, at capture time.
 *  - Errors: host-checkable problems return an error status and enqueue
 *    nothing.  Device-side checks (out-of-range slot, position or page id,
 *    a compress request with fewer than 2 pages) never fault: the offending
 *    item is skipped and a bit is set in the device error word (gp_err_bits),
 *    read with gp_get_device_errors.  A failed HIP launch returns GP_ERR_HIP.
 *  - Threads: one context per host thread.
 *  - Data types: fp32 for queries and query states, bf16 (raw uint16 bits)
 *    for keys and values, int32 for ids and counts.  Device buffers start on
 *    16-byte boundaries (the kernels read and write 16-byte vectors; torch
 *    allocations are aligned far beyond that).
 *
 * Layouts (row-major, outermost first)
 *  - K and V pools: [L][num_pages][Hkv][b][d] bf16.  A page id is shared by
 *    all layers; logical slot i of a request lives in page
 *    block_table[i / b] at offset i % b.
 *  - Query-state pool (Appendix E.1 Eq. 11): [L][M][2][Hq][d] fp32, index 0
 *    of the third axis is the short-timescale summary, 1 the long one.
 *  - Queries: [B][L][Hq][d] fp32, the normalised query before RoPE (§3.2).
 *  - Rotary table: [rope_rows][d] fp32; row p holds cos(p * f_j) for the d/2
 *    frequencies f_j, then sin(p * f_j) (rotate-half pairing (j, j + d/2)).
 *
 * Version 1 limits: d = 128, b = 256, Hq / Hkv = 4, batch <= 1024, at most
 * 2^23 cached tokens (32768 pages) per request for gp_demand and
 * gp_grow_page, at most 65536 tokens (256 pages) per compressed request
 * (a longer one is skipped with GP_DEVERR_LONG).
 */
#ifndef GROWPAGE_H
#define GROWPAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gp_status {
  GP_OK = 0,
  GP_ERR_INVALID_ARG = 1, /* a null pointer, bad shape or inconsistent size */
  GP_ERR_UNSUPPORTED = 2, /* valid but outside the version 1 limits */
  GP_ERR_WORKSPACE = 3,   /* workspace missing, too small or not from gp_demand */
  GP_ERR_HIP = 4          /* a HIP runtime call failed (see gp_last_hip_error) */
} gp_status;

/* Device error bits, OR-ed into the context's device error word. */
enum gp_err_bits {
  GP_DEVERR_SLOT = 1,      /* slot outside [0, max_slots): item skipped */
  GP_DEVERR_POSITION = 2,  /* position outside [0, rope_rows): clamped */
  GP_DEVERR_PAGE = 4,      /* page id outside [0, num_pages): tile skipped */
  GP_DEVERR_SHORT = 8,     /* compress requested with fewer than 2 pages */
  GP_DEVERR_PAGES = 16,    /* device page count outside [1, max_pages] */
  GP_DEVERR_NOPAGE = 32,   /* no free pages to replace a compressing request's
                              shared pages (App. E.2): request left uncompressed */
  GP_DEVERR_LONG = 64      /* compress asked of a request longer than 65536 tokens
                              (the version 1 selection limit): request left as it
                              was, the rest of the batch is compressed */
};

/* Actions and decisions (int8 on the device). */
#define GP_COMPRESS 0
#define GP_GROW 1
#define GP_SHRINK 2 /* GrowPage-Shrink policy only (App. H.1 Eq. 13) */

/* Capacity policies (gp_config.policy). */
#define GP_POLICY_GROWPAGE 0 /* Grow by One Page or Compress & Hold (§3.2-3.3) */
#define GP_POLICY_SHRINK 1   /* adds Shrink below shrink_tau (App. H.1 Eq. 13) */

/* Method parameters; defaults in brackets are the pages'. */
typedef struct gp_config {
  int32_t num_layers;    /* L */
  int32_t num_q_heads;   /* Hq */
  int32_t num_kv_heads;  /* Hkv; query head q uses KV head q / (Hq / Hkv) */
  int32_t head_dim;      /* d [128] */
  int32_t page_size;     /* b, tokens per page [256] (§5.1) */
  int32_t recent_window; /* |R_t|, newest tokens never evicted [16] (§3.3) */
  int32_t local_quota;   /* k_loc, per-block minimum retention [64] (App. D.2); 0 = plain top-k */
  int32_t p_num, p_den;  /* coverage p = p_num / p_den [99/100] (§3.2 Eq. 7) */
  double tau;            /* demand threshold [0] (§3.2, App. D.1) */
  float alpha_short;     /* new-query weight 1 - beta_S [0.1] (§3.2 Eq. 6) */
  float alpha_long;      /* new-query weight 1 - beta_L [0.001] */
  int32_t max_slots;     /* M, query-state slots [512] (App. E.1) */
  int32_t policy;        /* GP_POLICY_GROWPAGE [default] or GP_POLICY_SHRINK */
  double shrink_tau;     /* Shrink iff Delta < shrink_tau [-0.005] (App. H.1 Eq. 13);
                            must be <= tau; used by GP_POLICY_SHRINK only */
  int32_t min_tokens;    /* capacity floor: Shrink only if (P - 1) b >= min_tokens
                            [1024] (App. H.1) */
  int32_t compact_workgroups; /* workgroups (1024 threads) of the compaction kernel; 0 = 2
                                 per CU.  A smaller count leaves CUs to work on other
                                 streams, e.g. decoding beside asynchronous compression
                                 (App. E.3) */
} gp_config;

/* Global page pool (§4.2): K/V storage and the device free-page stack. */
typedef struct gp_pool {
  uint16_t* k_pool;     /* device bf16 [L][num_pages][Hkv][b][d] */
  uint16_t* v_pool;     /* device bf16, same layout */
  int32_t num_pages;    /* pages in the pool */
  int32_t* free_stack;  /* device int32 [num_pages]; free ids in [0, free_count) */
  int32_t* free_count;  /* device int32 [1]; top of stack is free_stack[free_count - 1] */
  int32_t* refcount;    /* device int32 [num_pages] references per page (prefix sharing,
                           App. E.2), or NULL: every page referenced once */
} gp_pool;

/* A batch of requests at their capacity boundary (N = P * b for each). */
typedef struct gp_batch {
  int32_t batch;                 /* B */
  int32_t max_pages;             /* row stride of block_table */
  int32_t* block_table;          /* device int32 [B][max_pages] page ids */
  int32_t* num_pages;            /* device int32 [B] P (gp_grow_page increments,
                                    gp_compress_hold decrements on Shrink) */
  int32_t* num_tokens;           /* device int32 [B] N (gp_compress_hold writes (P-1) b,
                                    or (P-2) b on Shrink) */
  const int32_t* slot;           /* device int32 [B] query-state slot */
  const int32_t* position;       /* device int32 [B] absolute position of the current query */
  const int32_t* num_pages_host; /* host int32 [B], equal to num_pages at the call */
} gp_batch;

/* Outputs of gp_demand (device). */
typedef struct gp_demand_out {
  int32_t* k_short;  /* [B][L][Hkv] K^S = D_p of the short view over C_t (Eq. 7) */
  int32_t* k_long;   /* [B][L][Hkv] K^L */
  int64_t* k_diff;   /* [B] sum K^S - sum K^L (may be NULL) */
  double* delta;     /* [B] Delta_t = r^S - r^L (Eq. 8) (may be NULL) */
  int8_t* decision;  /* [B] GP_GROW iff Delta_t > tau, else GP_COMPRESS; with
                        GP_POLICY_SHRINK, GP_SHRINK iff Delta_t < shrink_tau,
                        P >= 3 and (P - 1) b >= min_tokens */
  float* abar;       /* optional [sum over rows of N][2]: the full-cache attention
                        distributions (short, long) per token, rows in (request,
                        layer, KV head) order; NULL skips the write */
} gp_demand_out;

typedef struct gp_counters {
  int64_t grown;     /* pages granted by gp_grow_page */
  int64_t compress;  /* Compress & Hold actions (decisions plus fallbacks) */
  int64_t fallback;  /* Grow decisions that fell back (§4.2, App. H.2) */
  int64_t shrunk;    /* pages returned to the pool by Shrink (App. H.1) */
  int64_t copied;    /* target pages allocated to replace shared pages (App. E.2) */
} gp_counters;

typedef struct gp_ctx gp_ctx;

/* Creates a context on the current HIP device.  Validates the config:
 * Hq % Hkv == 0, 0 <= recent_window < page_size, local_quota >= 0,
 * 0 < p_num <= p_den <= 2^20, 0 < alpha <= 1, max_slots >= 1, policy one of
 * GP_POLICY_*, shrink_tau <= tau, min_tokens >= 0. */
gp_status gp_create(const gp_config* cfg, gp_ctx** out);
void gp_destroy(gp_ctx* ctx);

/* Workspace bytes gp_demand and gp_compress_hold need for `batch` requests
 * holding `total_tokens` cached tokens in all (sum of N), the largest of them
 * `max_tokens` (max of N).  Returns 0 on invalid arguments. */
size_t gp_workspace_bytes(const gp_ctx* ctx, int32_t batch, int64_t total_tokens,
                          int64_t max_tokens);

/* A0: dual-timescale summaries (§3.2 Eq. 6; App. E.1 "Initialization and
 * online update").  For each request b and summary x in {short, long}:
 *   first_step[b] != 0:  qbar = q                   (slot (re)initialisation)
 *   otherwise:           qbar = qbar + alpha_x (q - qbar)   (= beta qbar + (1-beta) q)
 * qstate [L][M][2][Hq][d] is updated in place; q is [B][L][Hq][d];
 * slot, first_step are device [B]. */
gp_status gp_update_summaries(gp_ctx* ctx, float* qstate, const float* q,
                              const int32_t* slot, const uint8_t* first_step,
                              int32_t batch, void* stream);

/* A1-A5: online demand estimation (§3.2; App. E.1 "Demand estimation at
 * capacity boundaries").  Per request: calibrate each summary to the RMS of
 * the current query q_cur (Eq. 12), rotate it to the current position, score
 * it against every cached key of every (layer, KV head), form the attention
 * distributions over the historical candidates C_t (all slots but the newest
 * page) and over all slots, compute K^S, K^L (Eq. 7), Delta (Eq. 8) and the
 * decision.  Requires N = P * b; P comes from num_pages_host (checked against
 * the device copy).  A request with P = 1 has no candidates and is given
 * GP_GROW with Delta = 0.  The workspace keeps the per-token importance the
 * next gp_compress_hold on the same batch uses.
 * qstate [L][M][2][Hq][d]; q_cur [B][L][Hq][d]; rope [rope_rows][d]. */
gp_status gp_demand(gp_ctx* ctx, const gp_pool* pool, const gp_batch* batch,
                    const float* qstate, const float* q_cur, const float* rope,
                    int32_t rope_rows, void* workspace, size_t workspace_bytes,
                    const gp_demand_out* out, void* stream);

/* A6: Grow by One Page with fallback (§3.3; §4.2; App. H.2).  Requests are
 * served in index order: a request whose decision is GP_GROW takes the page on
 * top of the free stack while more than reserve_pages are free and its block
 * table has room; the page is appended to its block table and P += 1 (with
 * reference counts, the page gets one reference).
 * Otherwise it falls back to compression.  action[b] receives GP_GROW or
 * GP_COMPRESS, or GP_SHRINK for a GP_SHRINK decision (no page is taken);
 * decision may come from gp_demand or from the caller (policy variants).
 * Under GP_POLICY_GROWPAGE page counts never decrease (§3.3). */
gp_status gp_grow_page(gp_ctx* ctx, const gp_pool* pool, const gp_batch* batch,
                       const int8_t* decision, int8_t* action,
                       int32_t reserve_pages, void* stream);

/* A7-A9: Compress & Hold (§3.3 Eq. 9-10; §4.2; App. E.2) for every request
 * whose action is GP_COMPRESS (action == NULL: every request).  Per (layer,
 * KV head): importance s_i = max of the two full-cache distributions (Eq. 9);
 * the newest recent_window slots are kept; each logical page keeps its top
 * local_quota candidates; the rest of the budget (P-1) b - recent_window goes
 * to the globally most important remaining candidates (ties: newer slot
 * first); exactly b candidates are dropped and the kept K/V rows move, in
 * slot order, to slots 0 .. (P-1) b - 1 of the same pages.  num_tokens
 * becomes (P-1) b; block tables and P are unchanged.  A request whose action
 * is GP_SHRINK (App. H.1) drops 2b candidates instead (budget (P-2) b -
 * recent_window), its kept rows move to slots 0 .. (P-2) b - 1, then its last
 * page is pushed on the free stack (requests in index order), its block-table
 * entry set to -1, P -= 1 and num_tokens = (P-2) b with the old P; a Shrink
 * with fewer than 3 pages sets GP_DEVERR_SHORT and leaves the request as it
 * was; under GP_POLICY_GROWPAGE a GP_SHRINK action is ignored.  A request
 * longer than 65536 tokens is left as it was (GP_DEVERR_LONG) while the rest
 * of the batch is compressed.
 * Prefix sharing (App. E.2; pool->refcount != NULL): a page with more than
 * one reference is never written.  Before selection, each compressing
 * request gets a new target page for every shared page it keeps (its P
 * pages, or its first P-1 for Shrink), from the top of the free stack in
 * request and page order; a request whose pages cannot all be allocated, and
 * every later one that needs any, is left uncompressed (GP_DEVERR_NOPAGE).
 * The compaction writes the kept rows of a replaced page into its target
 * (copying rows before the first drop too); afterwards the block table
 * points at the targets, the old pages lose one reference each and the
 * targets have one; a page whose count reaches zero is left to the caller
 * (a prefix cache keeps it until eviction).  A Shrink whose last page is
 * shared drops its reference instead of returning the page, which goes back
 * to the pool with its last reference (requests in index order).  Counts
 * must be at least the number of block-table references to each page.
 * Must follow gp_demand on the same batch with the same workspace.
 * dropped_out (optional, device int32 [B][L][Hkv][b] under
 * GP_POLICY_GROWPAGE, [B][L][Hkv][2b] under GP_POLICY_SHRINK) receives the
 * dropped slots in ascending order; rows of requests that do not compress
 * are left unwritten. */
gp_status gp_compress_hold(gp_ctx* ctx, const gp_pool* pool, const gp_batch* batch,
                           const int8_t* action, void* workspace,
                           size_t workspace_bytes, int32_t* dropped_out,
                           void* stream);

/* Workspace bytes gp_decode_attention needs for `batch` requests holding
 * `total_pages` pages in all (sum of num_pages_host).  Returns 0 on invalid
 * arguments. */
size_t gp_decode_workspace_bytes(const gp_ctx* ctx, int32_t batch, int64_t total_pages);

/* Decode-step attention of one layer with the summary update fused (§4.1:
 * the regular decoding path's attention kernel also updates both summaries
 * from the normalised pre-RoPE query; App. E.1 "Initialization and online
 * update"; the output is §3.1 Eq. 3's full-cache o_t).  For each request r
 * and query head g of the layer `layer`:
 *   qhat = RoPE(q[r][g], position[r]) / sqrt(d)   (rotate-half pairs j, j+d/2)
 *   a_i  = softmax over the num_tokens[r] cached slots i of qhat . k_i, where
 *          logical slot i lives in page block_table[r][i / b] at offset i % b
 *          and query head g reads KV head g / (Hq / Hkv)
 *   out[r][g] = sum_i a_i v_i.
 * Any 1 <= num_tokens[r] <= num_pages[r] * b is allowed (mid-page decoding;
 * after Compress & Hold num_tokens = (P-1) b covers the compacted slots).
 * If qstate != NULL the layer's two summaries of slot[r] are updated from q
 * exactly as gp_update_summaries does (first_step may be NULL: no request is
 * on its first step), so calling this for every layer equals one
 * gp_update_summaries call bit for bit.
 *   q:     device fp32 [B][Hq][d], normalised, before RoPE (read only)
 *   out:   device fp32 [B][Hq][d] (written)
 *   rope:  device fp32 [rope_rows][d] (cos of the d/2 frequencies, then sin)
 *   workspace: gp_decode_workspace_bytes(ctx, B, sum of num_pages_host) bytes
 * Arithmetic is fp32 (hardware exp2): within 1e-3 of the largest |v| of the
 * row element-wise against the fp64 definition.  Device checks: counts
 * outside 1 <= N <= P b or P outside [1, max_pages] set GP_DEVERR_PAGES and
 * give a zero output (so does a device page total above the host mirror's,
 * which the workspace was sized for); a page id outside the pool sets
 * GP_DEVERR_PAGE and its slots are skipped; position and slot as in gp_demand and
 * gp_update_summaries.  Enqueued on `stream`; pool, batch, q, qstate, rope,
 * out and workspace are borrowed for the call. */
gp_status gp_decode_attention(gp_ctx* ctx, const gp_pool* pool, const gp_batch* batch,
                              int32_t layer, const float* q, float* qstate,
                              const uint8_t* first_step, const float* rope, int32_t rope_rows,
                              float* out, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Size of the library's static scratch buffer (one per GPU). */
#define GP_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * gp_decode_attention with its scratch (rotated queries, work list, per-run
 * partials) in a buffer the library holds instead of a caller workspace.
 * Same kernels and arguments as gp_decode_attention minus the workspace, and
 * the same outputs bit for bit.
 *  - The buffer is GP_STATIC_SCRATCH_BYTES (64 MiB) of device memory per GPU,
 *    set up by gp_create on its device and held until the process ends.
 *  - A batch whose gp_decode_workspace_bytes(ctx, B, sum of num_pages_host)
 *    exceeds GP_STATIC_SCRATCH_BYTES is refused with GP_ERR_WORKSPACE before
 *    anything is enqueued (with 8 KV heads: about 4000 cached pages, about a
 *    million tokens, per call).
 *  - All calls on one GPU share the buffer, which keeps the last call's
 *    contents (nothing in it needs clearing: every call writes what it
 *    reads).  Calls that overlap in time on one GPU (on different streams,
 *    or from several contexts or host threads) race on it: order them on one
 *    stream.
 *  - Allocates nothing and records no gp_profile events. */
gp_status gp_decode_attention_static(gp_ctx* ctx, const gp_pool* pool, const gp_batch* batch,
                                     int32_t layer, const float* q, float* qstate,
                                     const uint8_t* first_step, const float* rope,
                                     int32_t rope_rows, float* out, void* stream);

/* Kernels of the event, for gp_profile_read. */
enum gp_kernel_id {
  GP_K_EMA = 0,     /* A0 summary update */
  GP_K_PLAN = 1,    /* batch prefix sums, work order and validation: runs inside the
                       GP_K_QHAT launch, so it records no launches of its own */
  GP_K_QHAT = 2,    /* A1 calibrate + rotate, with the batch plan in the same launch */
  GP_K_DEMAND = 3,  /* A2-A4 paged key scoring, distributions, importance, D_p */
  GP_K_DECIDE = 4,  /* A5 trend and decision */
  GP_K_GROW = 5,    /* A6 page grant and fallback */
  GP_K_SELECT = 6,  /* A7-A8 window mask and Eq. 10 selection */
  GP_K_COMPACT = 7, /* A9 in-place compaction */
  GP_K_RETURN = 8,  /* page bookkeeping after compaction: shared-page release, Shrink's
                       page return (prefix sharing or GP_POLICY_SHRINK only) */
  GP_K_SHARE = 9,   /* target pages for shared pages (prefix sharing only) */
  GP_K_DECODE = 10, /* decode-step attention with the summary update (both kernels) */
  GP_NUM_KERNELS = 11
};

typedef struct gp_kernel_times {
  double ms[GP_NUM_KERNELS];        /* accumulated device time per kernel */
  int64_t launches[GP_NUM_KERNELS]; /* launches recorded per kernel */
} gp_kernel_times;

/* Kernel timing for measurement.  enable != 0 clears the accumulators and
 * from then on records a HIP event before and after every kernel the
 * context launches, on the launch stream; enable == 0 stops recording.
 * gp_profile_read synchronises on the recorded events, adds their elapsed
 * times to the accumulators and copies them to *out. */
gp_status gp_profile(gp_ctx* ctx, int enable);
gp_status gp_profile_read(gp_ctx* ctx, gp_kernel_times* out);

/* Copies the device counters to *out (synchronises the device). */
gp_status gp_get_counters(gp_ctx* ctx, gp_counters* out);

/* Returns the device error word (gp_err_bits) in *bits and clears it
 * (synchronises the device). */
gp_status gp_get_device_errors(gp_ctx* ctx, int32_t* bits);

const char* gp_status_str(gp_status status);

/* The last HIP error code seen by the context (0 = none). */
int gp_last_hip_error(const gp_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif /* GROWPAGE_H */
