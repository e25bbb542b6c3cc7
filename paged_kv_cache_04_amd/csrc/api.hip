// C ABI of the GrowPage boundary-event library: validation, workspace
// carving and launch sequencing.  Kernels live in the k_*.hip files.
// Citations are to "GrowPage: On-Demand KV Budgeting for Efficient LLM
// Reasoning Serving" (arXiv 2609.03494).
#include <mutex>
#include <new>
#include <tuple>
#include <vector>

#include "gp_internal.h"

// Scratch of gp_decode_attention_static: one copy per GPU the library runs
// on, held until the process ends.  In host code the name below stands for
// the array only symbolically; the device address of each GPU's copy comes
// from hipGetSymbolAddress (scratch_address) and only that address is used.
static __device__ __align__(256) unsigned char scratch[GP_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on `device`, which must be the current device;
// looked up once per device.
hipError_t scratch_address(int device, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  if (!g_scratch_dev[device]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_dev[device] = ptr;
  }
  *out = g_scratch_dev[device];
  return hipSuccess;
}

}  // namespace

struct gp_ctx {
  gp::Params p;
  int device = 0;
  int num_cus = 256;
  int64_t* d_counters = nullptr;  // [5]: granted, compress, fallback, returned, copied
  int32_t* d_err = nullptr;       // [1], right after the counters
  int last_hip = 0;
  void* scratch = nullptr;  // this device's copy of `scratch` (gp_decode_attention_static)
  // bookkeeping of the last gp_demand, checked by gp_compress_hold
  const void* ws = nullptr;
  size_t ws_bytes = 0;
  int batch = 0;
  int64_t total_tokens = 0;
  int64_t max_tokens = 0;
  std::vector<int32_t> pages;  // P per request at gp_demand time
  // kernel timing (gp_profile)
  bool profiling = false;
  std::vector<hipEvent_t> free_events;
  std::vector<std::tuple<int, hipEvent_t, hipEvent_t>> pending;
  double ms[GP_NUM_KERNELS] = {};
  int64_t launches[GP_NUM_KERNELS] = {};
};

namespace {

gp_status hip_fail(gp_ctx* c, hipError_t e) {
  if (e == hipSuccess) return GP_OK;
  c->last_hip = (int)e;
  return GP_ERR_HIP;
}

hipEvent_t take_event(gp_ctx* c) {
  if (!c->free_events.empty()) {
    hipEvent_t e = c->free_events.back();
    c->free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs one kernel launch; with profiling on, brackets it with events on s.
template <class F>
hipError_t timed(gp_ctx* c, int kid, hipStream_t s, F&& launch) {
  if (!c->profiling) return launch();
  hipEvent_t a = take_event(c), b = take_event(c);
  if (!a || !b) return launch();
  hipError_t e = hipEventRecord(a, s);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, s);
  c->pending.emplace_back(kid, a, b);
  return e;
}

bool shape_supported(const gp::Params& p) {
  return p.d == gp::kD && p.b == gp::kPage && p.Hq == gp::kGroup * p.Hkv;
}

gp_status check_batch(const gp_ctx* c, const gp_pool* pool, const gp_batch* bt,
                      int64_t* total_pages, int64_t* max_pages_used) {
  if (!pool || !bt) return GP_ERR_INVALID_ARG;
  if (!pool->k_pool || !pool->v_pool || pool->num_pages < 1) return GP_ERR_INVALID_ARG;
  if (bt->batch < 1 || bt->max_pages < 1 || !bt->block_table || !bt->num_pages ||
      !bt->num_tokens || !bt->slot || !bt->position || !bt->num_pages_host)
    return GP_ERR_INVALID_ARG;
  if (bt->batch > gp::kMaxBatch) return GP_ERR_UNSUPPORTED;
  int64_t tot = 0, mx = 0;
  for (int r = 0; r < bt->batch; ++r) {
    const int32_t P = bt->num_pages_host[r];
    if (P < 1 || P > bt->max_pages) return GP_ERR_INVALID_ARG;
    tot += P;
    mx = P > mx ? P : mx;
  }
  (void)c;
  *total_pages = tot;
  *max_pages_used = mx;
  return GP_OK;
}

// gp_decode_attention and its static-scratch variant: validation, then the
// three decode kernels on `ws` (at least ws_bytes long).  With profile
// false no HIP event is created or recorded.
gp_status decode_call(gp_ctx* c, const gp_pool* pool, const gp_batch* bt, int32_t layer,
                      const float* q, float* qstate, const uint8_t* first_step, const float* rope,
                      int32_t rope_rows, float* out, void* ws, size_t ws_bytes, void* stream,
                      bool profile) {
  if (!c || !q || !rope || rope_rows < 1 || !out || !ws) return GP_ERR_INVALID_ARG;
  if (!shape_supported(c->p)) return GP_ERR_UNSUPPORTED;
  if (layer < 0 || layer >= c->p.L) return GP_ERR_INVALID_ARG;
  int64_t total_pages = 0, max_pages_used = 0;
  gp_status st = check_batch(c, pool, bt, &total_pages, &max_pages_used);
  if (st != GP_OK) return st;
  const gp::DecodeWs w = gp::decode_ws_layout(c->p, bt->batch, total_pages);
  if (ws_bytes < w.total) return GP_ERR_WORKSPACE;
  if (w.unit_cap > INT32_MAX) return GP_ERR_UNSUPPORTED;
  const int unit_blocks = c->num_cus * GP_DECODE_BLOCKS_PER_CU;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto launch = [&] {
    return gp::launch_decode(c->p, w, bt->batch, layer, pool->k_pool, pool->v_pool,
                             pool->num_pages, bt->block_table, bt->max_pages, bt->num_pages,
                             bt->num_tokens, bt->slot, bt->position, q, qstate, first_step, rope,
                             rope_rows, unit_blocks, ws, out, c->d_err, s);
  };
  return hip_fail(c, profile ? timed(c, GP_K_DECODE, s, launch) : launch());
}

}  // namespace

extern "C" {

gp_status gp_create(const gp_config* cfg, gp_ctx** out) {
  if (!cfg || !out) return GP_ERR_INVALID_ARG;
  *out = nullptr;
  gp::Params p{};
  p.L = cfg->num_layers;
  p.Hq = cfg->num_q_heads;
  p.Hkv = cfg->num_kv_heads;
  p.d = cfg->head_dim;
  p.b = cfg->page_size;
  p.R = cfg->recent_window;
  p.kloc = cfg->local_quota;
  p.p_num = cfg->p_num;
  p.p_den = cfg->p_den;
  p.tau = cfg->tau;
  p.alpha_s = cfg->alpha_short;
  p.alpha_l = cfg->alpha_long;
  p.M = cfg->max_slots;
  p.policy = cfg->policy;
  p.shrink_tau = cfg->shrink_tau;
  p.min_tokens = cfg->min_tokens;
  p.compact_groups = cfg->compact_workgroups;
  if (p.compact_groups < 0) return GP_ERR_INVALID_ARG;
  if (p.policy != GP_POLICY_GROWPAGE && p.policy != GP_POLICY_SHRINK) return GP_ERR_INVALID_ARG;
  if (p.policy == GP_POLICY_SHRINK &&
      (!(p.shrink_tau <= p.tau) || p.min_tokens < 0))
    return GP_ERR_INVALID_ARG;
  if (p.L < 1 || p.Hq < 1 || p.Hkv < 1 || p.Hq % p.Hkv != 0 || p.d < 2 || p.d % 2 != 0 ||
      p.b < 1 || p.R < 0 || p.R >= p.b || p.kloc < 0 || p.p_num <= 0 || p.p_den < p.p_num ||
      p.p_den > (1 << 20) || !(p.alpha_s > 0.0f && p.alpha_s <= 1.0f) ||
      !(p.alpha_l > 0.0f && p.alpha_l <= 1.0f) || p.M < 1 || p.tau != p.tau)
    return GP_ERR_INVALID_ARG;
  gp_ctx* c = new (std::nothrow) gp_ctx();
  if (!c) return GP_ERR_INVALID_ARG;
  c->p = p;
  hipError_t e = hipGetDevice(&c->device);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&c->num_cus, hipDeviceAttributeMultiprocessorCount, c->device);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&c->d_counters), 64);
  if (e == hipSuccess) e = hipMemset(c->d_counters, 0, 64);
  if (e == hipSuccess) e = scratch_address(c->device, &c->scratch);
  if (e != hipSuccess) {
    if (c->d_counters) (void)hipFree(c->d_counters);
    delete c;
    return GP_ERR_HIP;
  }
  c->d_err = reinterpret_cast<int32_t*>(c->d_counters + 5);
  *out = c;
  return GP_OK;
}

void gp_destroy(gp_ctx* c) {
  if (!c) return;
  for (auto& t : c->pending) {
    (void)hipEventDestroy(std::get<1>(t));
    (void)hipEventDestroy(std::get<2>(t));
  }
  for (hipEvent_t e : c->free_events) (void)hipEventDestroy(e);
  if (c->d_counters) (void)hipFree(c->d_counters);
  delete c;
}

size_t gp_workspace_bytes(const gp_ctx* c, int32_t batch, int64_t total_tokens,
                          int64_t max_tokens) {
  if (!c || batch < 1 || total_tokens < 0 || max_tokens < 0) return 0;
  return gp::ws_layout(c->p, batch, total_tokens, max_tokens, c->num_cus * gp::kDemandBlocksPerCU).total;
}

gp_status gp_update_summaries(gp_ctx* c, float* qstate, const float* q, const int32_t* slot,
                              const uint8_t* first_step, int32_t batch, void* stream) {
  if (!c || !qstate || !q || !slot || !first_step || batch < 1) return GP_ERR_INVALID_ARG;
  if (c->p.d != gp::kD) return GP_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_fail(c, timed(c, GP_K_EMA, s, [&] {
    return gp::launch_ema(c->p, qstate, q, slot, first_step, batch, c->d_err, s);
  }));
}

gp_status gp_demand(gp_ctx* c, const gp_pool* pool, const gp_batch* bt, const float* qstate,
                    const float* q_cur, const float* rope, int32_t rope_rows, void* ws,
                    size_t ws_bytes, const gp_demand_out* out, void* stream) {
  if (!c || !qstate || !q_cur || !rope || rope_rows < 1 || !out || !out->k_short ||
      !out->k_long || !out->decision)
    return GP_ERR_INVALID_ARG;
  if (!shape_supported(c->p)) return GP_ERR_UNSUPPORTED;
  int64_t total_pages = 0, max_pages_used = 0;
  gp_status st = check_batch(c, pool, bt, &total_pages, &max_pages_used);
  if (st != GP_OK) return st;
  const int B = bt->batch;
  const int64_t total_tokens = total_pages * c->p.b;
  const int64_t max_tokens = max_pages_used * c->p.b;
  if (max_tokens > gp::kMaxRequestTokens) return GP_ERR_UNSUPPORTED;
  const gp::WsLayout w = gp::ws_layout(c->p, B, total_tokens, max_tokens, c->num_cus * gp::kDemandBlocksPerCU);
  if (!ws || ws_bytes < w.total) return GP_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the plan runs inside the summaries launch (its own block)
  hipError_t e = timed(c, GP_K_QHAT, s, [&] {
    return gp::launch_prep(c->p, w, qstate, q_cur, rope, rope_rows, bt->slot, bt->position,
                           bt->num_pages, B, bt->max_pages, total_pages, ws, c->d_err, s);
  });
  if (e == hipSuccess)
    e = timed(c, GP_K_DEMAND, s, [&] {
      return gp::launch_demand(c->p, w, pool->k_pool, pool->num_pages, bt->block_table,
                               bt->max_pages, B, ws, out->k_short, out->k_long, out->abar,
                               c->d_err, s);
    });
  if (e == hipSuccess)
    e = timed(c, GP_K_DECIDE, s, [&] {
      return gp::launch_decide(c->p, w, B, ws, out->k_short, out->k_long, out->k_diff,
                               out->delta, out->decision, s);
    });
  if (e != hipSuccess) {
    c->ws = nullptr;
    return hip_fail(c, e);
  }
  c->ws = ws;
  c->ws_bytes = ws_bytes;
  c->batch = B;
  c->total_tokens = total_tokens;
  c->max_tokens = max_tokens;
  c->pages.assign(bt->num_pages_host, bt->num_pages_host + B);
  return GP_OK;
}

gp_status gp_grow_page(gp_ctx* c, const gp_pool* pool, const gp_batch* bt,
                       const int8_t* decision, int8_t* action, int32_t reserve_pages,
                       void* stream) {
  if (!c || !decision || !action || reserve_pages < 0) return GP_ERR_INVALID_ARG;
  if (!pool || !pool->free_stack || !pool->free_count || pool->num_pages < 1)
    return GP_ERR_INVALID_ARG;
  if (!bt || bt->batch < 1 || !bt->block_table || !bt->num_pages || bt->max_pages < 1)
    return GP_ERR_INVALID_ARG;
  if (bt->batch > gp::kMaxBatch) return GP_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_fail(c, timed(c, GP_K_GROW, s, [&] {
    return gp::launch_grow(bt->batch, bt->max_pages, pool->num_pages, bt->block_table,
                           bt->num_pages, pool->free_stack, pool->free_count, reserve_pages,
                           decision, action, pool->refcount, c->d_counters, c->d_err, s);
  }));
}

gp_status gp_compress_hold(gp_ctx* c, const gp_pool* pool, const gp_batch* bt,
                           const int8_t* action, void* ws, size_t ws_bytes,
                           int32_t* dropped_out, void* stream) {
  if (!c || !pool || !bt || !pool->k_pool || !pool->v_pool || !bt->block_table ||
      !bt->num_tokens)
    return GP_ERR_INVALID_ARG;
  if (!shape_supported(c->p)) return GP_ERR_UNSUPPORTED;
  if (!ws || ws != c->ws || ws_bytes != c->ws_bytes || bt->batch != c->batch)
    return GP_ERR_WORKSPACE;
  const gp::Params& p = c->p;
  const bool shrink = p.policy == GP_POLICY_SHRINK && action;
  const bool shared = pool->refcount != nullptr;
  if ((shrink || shared) && (!pool->free_stack || !pool->free_count || !bt->num_pages))
    return GP_ERR_INVALID_ARG;
  // Eq. 10 needs the local quotas to fit the budget K_t = (P - m) b - R,
  // m = 1 for Compress & Hold, 2 for Shrink (any request with 3 or more pages
  // may shrink under GP_POLICY_SHRINK).  Requests too short or too long to
  // compress are flagged on the device if they are asked to, and skipped.
  for (int r = 0; r < c->batch; ++r) {
    const int64_t P = c->pages[r];
    if (P < 2 || P * p.b > gp::kMaxCompressTokens) continue;
    const int64_t kq = p.kloc;
    const int64_t loc = (P - 1) * (kq < p.b ? kq : p.b) + (kq < p.b - p.R ? kq : p.b - p.R);
    const int64_t m = (p.policy == GP_POLICY_SHRINK && P >= 3) ? 2 : 1;
    if (loc > (P - m) * p.b - p.R) return GP_ERR_UNSUPPORTED;
  }
  const gp::WsLayout w = gp::ws_layout(p, c->batch, c->total_tokens, c->max_tokens, c->num_cus * gp::kDemandBlocksPerCU);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the request flags start cleared (gp_demand's plan); only prefix sharing
  // needs the target-page step
  hipError_t e = hipSuccess;
  if (shared)
    e = timed(c, GP_K_SHARE, s, [&] {
      return gp::launch_share(p, w, c->batch, action, pool->num_pages, bt->block_table,
                              bt->max_pages, pool->refcount, pool->free_stack, pool->free_count,
                              ws, c->d_counters, c->d_err, s);
    });
  if (e == hipSuccess)
    e = timed(c, GP_K_SELECT, s, [&] {
      return gp::launch_select(p, w, c->batch, action, ws, dropped_out, c->d_err, c->num_cus,
                               s);
    });
  if (e == hipSuccess)
    e = timed(c, GP_K_COMPACT, s, [&] {
      return gp::launch_compact(p, w, c->batch, action, pool->k_pool, pool->v_pool,
                                pool->num_pages, bt->block_table, bt->max_pages, bt->num_tokens,
                                shared,
                                p.compact_groups > 0 ? p.compact_groups
                                                     : c->num_cus * GP_COMPACT_BLOCKS_PER_CU,
                                ws, c->d_err, s);
    });
  if (e == hipSuccess && (shrink || shared))
    e = timed(c, GP_K_RETURN, s, [&] {
      return gp::launch_return(w, c->batch, bt->max_pages, pool->num_pages, bt->block_table,
                               bt->num_pages, pool->free_stack, pool->free_count,
                               pool->refcount, action, ws, c->d_counters, c->d_err, s);
    });
  return hip_fail(c, e);
}

size_t gp_decode_workspace_bytes(const gp_ctx* c, int32_t batch, int64_t total_pages) {
  if (!c || batch < 1 || total_pages < 1) return 0;
  return gp::decode_ws_layout(c->p, batch, total_pages).total;
}

gp_status gp_decode_attention(gp_ctx* c, const gp_pool* pool, const gp_batch* bt, int32_t layer,
                              const float* q, float* qstate, const uint8_t* first_step,
                              const float* rope, int32_t rope_rows, float* out, void* ws,
                              size_t ws_bytes, void* stream) {
  return decode_call(c, pool, bt, layer, q, qstate, first_step, rope, rope_rows, out, ws,
                     ws_bytes, stream, true);
}

gp_status gp_decode_attention_static(gp_ctx* c, const gp_pool* pool, const gp_batch* bt,
                                     int32_t layer, const float* q, float* qstate,
                                     const uint8_t* first_step, const float* rope,
                                     int32_t rope_rows, float* out, void* stream) {
  if (!c || !c->scratch) return GP_ERR_INVALID_ARG;
  return decode_call(c, pool, bt, layer, q, qstate, first_step, rope, rope_rows, out,
                     c->scratch, GP_STATIC_SCRATCH_BYTES, stream, false);
}

gp_status gp_profile(gp_ctx* c, int enable) {
  if (!c) return GP_ERR_INVALID_ARG;
  if (enable) {
    for (auto& t : c->pending) {
      c->free_events.push_back(std::get<1>(t));
      c->free_events.push_back(std::get<2>(t));
    }
    c->pending.clear();
    for (int k = 0; k < GP_NUM_KERNELS; ++k) {
      c->ms[k] = 0.0;
      c->launches[k] = 0;
    }
  }
  c->profiling = enable != 0;
  return GP_OK;
}

gp_status gp_profile_read(gp_ctx* c, gp_kernel_times* out) {
  if (!c || !out) return GP_ERR_INVALID_ARG;
  hipError_t e = hipSuccess;
  for (auto& t : c->pending) {
    const int kid = std::get<0>(t);
    hipEvent_t a = std::get<1>(t), b = std::get<2>(t);
    if (e == hipSuccess) e = hipEventSynchronize(b);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    if (e == hipSuccess) {
      c->ms[kid] += ms;
      c->launches[kid] += 1;
    }
    c->free_events.push_back(a);
    c->free_events.push_back(b);
  }
  c->pending.clear();
  for (int k = 0; k < GP_NUM_KERNELS; ++k) {
    out->ms[k] = c->ms[k];
    out->launches[k] = c->launches[k];
  }
  return hip_fail(c, e);
}

gp_status gp_get_counters(gp_ctx* c, gp_counters* out) {
  if (!c || !out) return GP_ERR_INVALID_ARG;
  int64_t h[5];
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(h, c->d_counters, sizeof h, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(c, e);
  out->grown = h[0];
  out->compress = h[1];
  out->fallback = h[2];
  out->shrunk = h[3];
  out->copied = h[4];
  return GP_OK;
}

gp_status gp_get_device_errors(gp_ctx* c, int32_t* bits) {
  if (!c || !bits) return GP_ERR_INVALID_ARG;
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(bits, c->d_err, sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(c->d_err, 0, sizeof(int32_t));
  return hip_fail(c, e);
}

const char* gp_status_str(gp_status st) {
  switch (st) {
    case GP_OK: return "ok";
    case GP_ERR_INVALID_ARG: return "invalid argument";
    case GP_ERR_UNSUPPORTED: return "unsupported shape or size";
    case GP_ERR_WORKSPACE: return "workspace missing, too small or not prepared by gp_demand";
    case GP_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int gp_last_hip_error(const gp_ctx* c) { return c ? c->last_hip : 0; }

}  // extern "C"
