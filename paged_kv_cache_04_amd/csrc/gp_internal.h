// Internal definitions of the GrowPage boundary-event library (gfx950).
// Citations are to "GrowPage: On-Demand KV Budgeting for Efficient LLM
// Reasoning Serving" (arXiv 2609.03494).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/growpage.h"

namespace gp {

// Version-1 kernel shape: head_dim 128, page 256, 4 query heads per KV head,
// so each row is scored by 2 views x 4 heads = 8 summary queries.
constexpr int kD = 128;
constexpr int kPage = 256;
constexpr int kGroup = 4;
constexpr int kNQ = 2 * kGroup;
constexpr int kMaxBatch = 1024;
// Longest request gp_demand accepts: the demand kernel's per-lane fp64 sums
// of 2^-40 masses stay exact up to 2^13 terms per lane of a 1024-thread block.
constexpr int64_t kMaxRequestTokens = int64_t(1) << 23;
// Demand kernel: persistent workgroups per CU (each holds one row at a time).
#ifndef GP_DEMAND_BLOCKS_PER_CU
#define GP_DEMAND_BLOCKS_PER_CU 1
#endif
constexpr int kDemandBlocksPerCU = GP_DEMAND_BLOCKS_PER_CU;
// Compaction: persistent workgroups per CU when the context sets no count.
#ifndef GP_COMPACT_BLOCKS_PER_CU
#define GP_COMPACT_BLOCKS_PER_CU 2
#endif
// Decode attention: persistent workgroups per CU of the unit kernel.
#ifndef GP_DECODE_BLOCKS_PER_CU
#define GP_DECODE_BLOCKS_PER_CU 2
#endif
constexpr uint64_t kWsMagic = 0x4750574b53503031ull;  // "GPWKSP01"

// Fixed-point scale for exact, order-free sums of probabilities: values in
// [0, 1] are floored to multiples of 2^-40 and summed as uint64.
constexpr float kFix = 1099511627776.0f;       // 2^40
constexpr float kFixInv = 9.094947017729282e-13f;  // 2^-40

struct Params {
  int L, Hq, Hkv, d, b, R, kloc, p_num, p_den, M;
  double tau;
  float alpha_s, alpha_l;
  int policy;         // GP_POLICY_*
  double shrink_tau;  // Shrink threshold (GP_POLICY_SHRINK)
  int min_tokens;     // Shrink capacity floor
  int compact_groups; // workgroups of the compaction kernel
  // pages of slots one event can free per request: 2 with Shrink, else 1
  int max_freed() const { return policy == GP_POLICY_SHRINK ? 2 : 1; }
};

// Workspace layout, identical for gp_demand and gp_compress_hold.
struct WsHeader {
  uint64_t magic;
  int32_t batch;
  int32_t valid;         // 1 once the plan kernel accepted the batch
  int64_t total_tokens;  // sum of N over the batch
  int32_t row_counter;   // work queue of the demand kernel
  int32_t item_counter;  // work queue of the compaction kernel (cleared by the selection)
  int64_t pad[4];
};

// Per-request state of one gp_compress_hold call (req_flags).
constexpr int32_t kReqBlocked = 1;    // shared pages could not be replaced: not compressed
constexpr int32_t kReqCompacted = 2;  // K/V compacted (set by the compaction kernel)
constexpr int32_t kReqTooLong = 4;    // longer than the selection takes: not compressed
// Longest request the selection and compaction kernels take (their per-row
// page lists and block counts live in LDS).
constexpr int64_t kMaxCompressTokens = 65536;

// Workspace: batch plan, calibrated summaries, per-token importance (read by
// gp_compress_hold), dropped slots, per-request flags and target pages of the
// prefix-preserving compression, and per-workgroup rings that hold one row's
// logits and demand distributions at a time.
struct WsLayout {
  size_t header, page_off, req_order, qhat, ring_logits, ring_keys, imp, dropped, req_flags,
      target, total;
  int64_t rows, row_tokens, row_pages, ring_tokens, blocks;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WsLayout ws_layout(const Params& p, int B, int64_t total_tokens, int64_t max_tokens,
                          int blocks) {
  WsLayout w{};
  const int64_t lh = (int64_t)p.L * p.Hkv;
  w.rows = (int64_t)B * lh;
  w.row_tokens = lh * total_tokens;
  w.row_pages = lh * (total_tokens / p.b);
  w.ring_tokens = max_tokens;
  w.blocks = blocks;
  size_t o = 0;
  w.header = o;      o = align256(o + sizeof(WsHeader));
  w.page_off = o;    o = align256(o + sizeof(int64_t) * (B + 1));
  w.req_order = o;   o = align256(o + sizeof(int32_t) * B);
  w.qhat = o;        o = align256(o + sizeof(float) * (size_t)w.rows * kNQ * kD);
  w.ring_logits = o; o = align256(o + sizeof(float) * (size_t)blocks * max_tokens * kNQ);
  w.ring_keys = o;   o = align256(o + sizeof(float) * (size_t)blocks * max_tokens * 2);
  w.imp = o;         o = align256(o + sizeof(float) * (size_t)w.row_tokens);
  w.dropped = o;     o = align256(o + sizeof(int32_t) * (size_t)w.rows * p.b * p.max_freed());
  w.req_flags = o;   o = align256(o + sizeof(int32_t) * B);
  w.target = o;      o = align256(o + sizeof(int32_t) * (size_t)(total_tokens / p.b));
  w.total = o;
  return w;
}

// ---- device arithmetic -----------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// exp(x) for x <= 0: Cody & Waite reduction x = n ln2 + r (ln2 as a 16-bit
// head 0x1.62e4p-1 plus an fp32 tail), degree-6 Taylor polynomial of e^r in
// Horner form, scale by 2^n built in the exponent field; zero once n < -100
// so all later values stay normal fp32 numbers.
__device__ __forceinline__ float gp_exp(float x) {
  const float n = __builtin_rintf(x * 0x1.715476p+0f);
  float r = __builtin_fmaf(-n, 0x1.62e4p-1f, x);
  r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
  float p = 1.0f / 720.0f;
  p = __builtin_fmaf(p, r, 1.0f / 120.0f);
  p = __builtin_fmaf(p, r, 1.0f / 24.0f);
  p = __builtin_fmaf(p, r, 1.0f / 6.0f);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  // 2^n by the exponent field (n clamped so the conversion stays in range;
  // below n = -100 the select returns 0, branch-free).
  const float y = p * __uint_as_float((uint32_t)(127 + (int)fmaxf(n, -127.0f)) << 23);
  return n < -100.0f ? 0.0f : y;
}

// Cross-lane sums without LDS traffic: DPP rotations within each 16-lane
// row, and gfx950's permlane swaps, which exchange the odd 16-lane rows of
// one register with the even rows of another (permlane16) or the upper 32
// lanes of one with the lower 32 of another (permlane32).
__device__ __forceinline__ uint64_t pk64(uint32_t lo, uint32_t hi) {
  return ((uint64_t)hi << 32) | lo;
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, 0xf, 0xf, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return pk64(lo, hi);
}

// sum over the 16 lanes of each row, in every lane of the row (row_ror 8, 4, 2, 1)
__device__ __forceinline__ uint64_t row_sum_u64(uint64_t v) {
  v += dpp_u64<0x128>(v);
  v += dpp_u64<0x124>(v);
  v += dpp_u64<0x122>(v);
  v += dpp_u64<0x121>(v);
  return v;
}

// a + b after lanes 32..63 of a trade places with lanes 0..31 of b: lanes
// 0..31 get a's value there plus a's value 32 lanes up, lanes 32..63 b's
// value plus b's value 32 lanes down
__device__ __forceinline__ uint64_t swap32_add(uint64_t a, uint64_t b) {
  const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)a, (uint32_t)b, false, false);
  const auto hi =
      __builtin_amdgcn_permlane32_swap((uint32_t)(a >> 32), (uint32_t)(b >> 32), false, false);
  return pk64(lo[0], hi[0]) + pk64(lo[1], hi[1]);
}

// the same with the odd 16-lane rows of a and the even rows of b
__device__ __forceinline__ uint64_t swap16_add(uint64_t a, uint64_t b) {
  const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)a, (uint32_t)b, false, false);
  const auto hi =
      __builtin_amdgcn_permlane16_swap((uint32_t)(a >> 32), (uint32_t)(b >> 32), false, false);
  return pk64(lo[0], hi[0]) + pk64(lo[1], hi[1]);
}

// sum over the wave, in every lane
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  v = row_sum_u64(v);
  v = swap16_add(v, v);
  return swap32_add(v, v);
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x128, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0u, v, 0x124, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0u, v, 0x122, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0u, v, 0x121, 0xf, 0xf, false);
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = a[0] + a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return b[0] + b[1];
}

// Inclusive prefix sums over a wave: lane L gets the sum over lanes 0..L.
// DPP row shifts (lane i reads lane i - n of its 16-lane row, 0 before the
// row's start) give the sums within each row; each row then adds the totals
// of the rows below it, read from their last lanes.
__device__ __forceinline__ uint32_t wave_prefix_u32(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);
  const int row = (threadIdx.x & 63) >> 4;
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
                 r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (row > 0 ? r0 : 0u) + (row > 1 ? r1 : 0u) + (row > 2 ? r2 : 0u);
}

// Exclusive prefix sums over a block of nw waves (nw <= 16): returns the
// sum of v over the threads before this one and, through total, the sum over
// the block.  Ends with the block synchronised (s_w may be reused after).
__device__ __forceinline__ uint32_t block_prefix_excl_u32(uint32_t v, uint32_t* s_w, int nw,
                                                          uint32_t& total) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const uint32_t incl = wave_prefix_u32(v);
  if (lane == 63) s_w[wv] = incl;
  __syncthreads();
  uint32_t before = incl - v, all = 0;
  for (int u = 0; u < nw; ++u) {
    const uint32_t x = s_w[u];
    if (u < wv) before += x;
    all += x;
  }
  total = all;
  __syncthreads();
  return before;
}

// Mass of a probability in 2^-40 units (exact: v * 2^40 <= 2^40).
__device__ __forceinline__ uint64_t fix40(float v) { return (uint64_t)(v * kFix); }

// ---- launchers (each returns the hipError_t of its launch) -----------------

hipError_t launch_ema(const Params& p, float* qstate, const float* q, const int32_t* slot,
                      const uint8_t* first, int B, int32_t* err, hipStream_t s);

// Rotated summaries (A1) and the batch plan, one launch.
hipError_t launch_prep(const Params& p, const WsLayout& w, const float* qstate, const float* qcur,
                       const float* rope, int rope_rows, const int32_t* slot,
                       const int32_t* position, const int32_t* num_pages_dev, int B,
                       int max_pages, int64_t host_total_pages, void* ws, int32_t* err,
                       hipStream_t s);

hipError_t launch_demand(const Params& p, const WsLayout& w, const uint16_t* k_pool,
                         int pool_pages, const int32_t* block_table, int max_pages, int B,
                         void* ws, int32_t* k_short, int32_t* k_long, float* abar, int32_t* err,
                         hipStream_t s);

hipError_t launch_decide(const Params& p, const WsLayout& w, int B, const void* ws,
                         const int32_t* k_short,
                         const int32_t* k_long, int64_t* k_diff, double* delta,
                         int8_t* decision, hipStream_t s);

hipError_t launch_grow(int B, int max_pages, int pool_pages, int32_t* block_table,
                       int32_t* num_pages, const int32_t* free_stack, int32_t* free_count, int reserve,
                       const int8_t* decision, int8_t* action, int32_t* refcount,
                       int64_t* counters, int32_t* err, hipStream_t s);

hipError_t launch_share(const Params& p, const WsLayout& w, int B, const int8_t* action,
                        int pool_pages, const int32_t* block_table, int max_pages,
                        const int32_t* refcount, const int32_t* free_stack, int32_t* free_count,
                        void* ws, int64_t* counters, int32_t* err, hipStream_t s);

hipError_t launch_select(const Params& p, const WsLayout& w, int B, const int8_t* action,
                         void* ws, int32_t* dropped_out, int32_t* err, int num_cus,
                         hipStream_t s);

hipError_t launch_compact(const Params& p, const WsLayout& w, int B, const int8_t* action,
                          uint16_t* k_pool, uint16_t* v_pool, int pool_pages,
                          const int32_t* block_table, int max_pages, int32_t* num_tokens,
                          bool shared, int groups, void* ws, int32_t* err, hipStream_t s);

hipError_t launch_return(const WsLayout& w, int B, int max_pages, int pool_pages,
                         int32_t* block_table, int32_t* num_pages, int32_t* free_stack,
                         int32_t* free_count, int32_t* refcount, const int8_t* action,
                         const void* ws, int64_t* counters, int32_t* err, hipStream_t s);

// Decode-attention workspace: rotated queries, unit list, per-request page
// prefix, unit count, per-unit partials.
struct DecodeWs {
  size_t qhat, units, page_pre, n_units, part, total;
  int64_t unit_cap;
};

DecodeWs decode_ws_layout(const Params& p, int B, int64_t total_pages);

hipError_t launch_decode(const Params& p, const DecodeWs& w, int B, int layer,
                         const uint16_t* k_pool, const uint16_t* v_pool, int pool_pages,
                         const int32_t* block_table, int max_pages, const int32_t* num_pages,
                         const int32_t* num_tokens, const int32_t* slot, const int32_t* position,
                         const float* q, float* qstate, const uint8_t* first, const float* rope,
                         int rope_rows, int unit_blocks, void* ws, float* out, int32_t* err,
                         hipStream_t s);

}  // namespace gp
