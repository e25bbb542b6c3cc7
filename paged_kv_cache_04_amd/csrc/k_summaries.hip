// A0 (summary update), the batch plan, and A1 (calibrate + rotate).
// Citations are to "GrowPage: On-Demand KV Budgeting for Efficient LLM
// Reasoning Serving" (arXiv 2609.03494).
#include "gp_internal.h"

namespace gp {

// ---------------------------------------------------------------------------
// A0: dual-timescale EMA (§3.2 Eq. 6) with slot initialisation (App. E.1).
// One thread per 4 consecutive elements of one (request, layer, query head);
// both summaries are read and written as float4 (16 B per lane, coalesced
// along the head dimension).  Update: qbar + alpha * (q - qbar), the
// algebraically identical form of beta * qbar + (1 - beta) * q that keeps a
// constant stream exactly constant in fp32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ema(float* __restrict__ qstate, const float* __restrict__ q,
                                             const int32_t* __restrict__ slot,
                                             const uint8_t* __restrict__ first, int B, int L, int M,
                                             int Hq, float alpha_s, float alpha_l,
                                             int32_t* __restrict__ err) {
  constexpr int d4 = kD / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)B * L * Hq * d4;
  if (idx >= total) return;
  const int j4 = (int)(idx % d4);
  int64_t t = idx / d4;
  const int h = (int)(t % Hq);
  t /= Hq;
  const int l = (int)(t % L);
  const int b = (int)(t / L);
  const int s = slot[b];
  if (s < 0 || s >= M) {
    if (j4 == 0 && h == 0 && l == 0) atomicOr(err, GP_DEVERR_SLOT);
    return;
  }
  const float4 qv = reinterpret_cast<const float4*>(q)[(((int64_t)b * L + l) * Hq + h) * d4 + j4];
  float4* sp = reinterpret_cast<float4*>(qstate) + ((((int64_t)l * M + s) * 2 + 0) * Hq + h) * d4 + j4;
  float4* lp = sp + (int64_t)Hq * d4;
  if (first[b]) {
    *sp = qv;
    *lp = qv;
    return;
  }
  float4 a = *sp, c = *lp;
  a.x = __builtin_fmaf(alpha_s, qv.x - a.x, a.x);
  a.y = __builtin_fmaf(alpha_s, qv.y - a.y, a.y);
  a.z = __builtin_fmaf(alpha_s, qv.z - a.z, a.z);
  a.w = __builtin_fmaf(alpha_s, qv.w - a.w, a.w);
  c.x = __builtin_fmaf(alpha_l, qv.x - c.x, c.x);
  c.y = __builtin_fmaf(alpha_l, qv.y - c.y, c.y);
  c.z = __builtin_fmaf(alpha_l, qv.z - c.z, c.z);
  c.w = __builtin_fmaf(alpha_l, qv.w - c.w, c.w);
  *sp = a;
  *lp = c;
}

hipError_t launch_ema(const Params& p, float* qstate, const float* q, const int32_t* slot,
                      const uint8_t* first, int B, int32_t* err, hipStream_t s) {
  const int64_t total = (int64_t)B * p.L * p.Hq * (kD / 4);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(k_ema, dim3((unsigned)blocks), dim3(threads), 0, s, qstate, q, slot, first,
                     B, p.L, p.M, p.Hq, p.alpha_s, p.alpha_l, err);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Batch plan: prefix sums of the device page counts (page_off[r] = sum of P
// over requests before r), the demand kernel's work order (requests by page
// count, largest first, ties by index) and its queue counter, and resets the
// per-request flags of the compression that follows (a request longer than
// the compression takes is flagged kReqTooLong).  The batch is
// accepted (header.valid = 1) only if every count lies in [1, max_pages], no
// request is longer than the workspace's per-row rings and the total equals
// the host's; every later kernel of the event exits at once on a rejected
// batch, so a stale host mirror can never send a kernel outside the workspace.
// Runs as the last block of the summaries launch below.
// ---------------------------------------------------------------------------
constexpr int kPrepT = 256;                  // threads per block of the launch
constexpr int kPlanPer = kMaxBatch / kPrepT;  // requests per thread of the plan block

__device__ __forceinline__ void plan_block(const int32_t* __restrict__ num_pages, int B,
                                           int max_pages, int64_t host_total_pages, int b,
                                           int64_t ring_tokens, WsHeader* __restrict__ hdr,
                                           int64_t* __restrict__ page_off,
                                           int32_t* __restrict__ req_order,
                                           int32_t* __restrict__ req_flags,
                                           int32_t* __restrict__ err) {
  __shared__ int32_t pages[kMaxBatch];
  __shared__ uint32_t s_w[kPrepT / 64];
  const int t = threadIdx.x;
  // thread t takes requests kPlanPer t .. kPlanPer t + kPlanPer - 1
  int P[kPlanPer];
  bool any_bad = false;
  uint32_t v[kPlanPer], mine = 0;
#pragma unroll
  for (int k = 0; k < kPlanPer; ++k) {
    const int r = kPlanPer * t + k;
    P[k] = r < B ? num_pages[r] : 0;
    const bool ok_p = P[k] >= 1 && P[k] <= max_pages && (int64_t)P[k] * b <= ring_tokens;
    any_bad |= r < B && !ok_p;
    // counts outside [1, max_pages] reject the batch; they enter the sums as
    // 0 so the 32-bit prefix cannot wrap (valid counts sum to at most
    // 1024 * max_pages)
    v[k] = (r < B && ok_p) ? (uint32_t)P[k] : 0u;
    mine += v[k];
    if (r < B) pages[r] = P[k];
  }
  const int bad = __syncthreads_or(any_bad);
  uint32_t total_u = 0;
  uint32_t before = block_prefix_excl_u32(mine, s_w, kPrepT / 64, total_u);
#pragma unroll
  for (int k = 0; k < kPlanPer; ++k) {
    const int r = kPlanPer * t + k;
    before += v[k];
    if (r < B) {
      req_flags[r] = (int64_t)P[k] * b > kMaxCompressTokens ? kReqTooLong : 0;
      page_off[r + 1] = (int64_t)before;
      int rank = 0;
      for (int u = 0; u < B; ++u) rank += (pages[u] > P[k]) || (pages[u] == P[k] && u < r);
      req_order[rank] = r;
    }
  }
  if (t == 0) {
    page_off[0] = 0;
    const int64_t total = (int64_t)total_u;
    const int ok = (!bad) && total == host_total_pages;
    hdr->magic = kWsMagic;
    hdr->batch = B;
    hdr->total_tokens = total * b;
    hdr->row_counter = 0;
    hdr->valid = ok;
    if (!ok) atomicOr(err, GP_DEVERR_PAGES);
  }
}

// ---------------------------------------------------------------------------
// A1: calibrated, rotated summaries (App. E.1 Eq. 12 and the paragraph after
// it), one (request, layer) pair per block; thread x*Hq + hq handles
// summary x of query head hq:
//   gamma = sqrt(ss(q_t) / ss(qbar)) (serial fmaf sums of squares; 0 when
//   ss(qbar) = 0), qtilde = gamma * qbar, rotate-half rotary at the current
//   position with the caller's (cos, sin) row, times 1/sqrt(d).
// Output layout per row (request, layer, KV head): [32 quads][8 queries][4],
// query index x * 4 + g for the g-th query head of the KV head (GQA grouping
// of consecutive query heads); element j sits in quad j / 4 at j % 4, so the
// scoring kernel reads the 32 values of one 4-element key quad contiguously.
// It reads no page count, so it runs beside the plan in the same launch (a
// rejected batch stops at the demand kernel).  Loads that do not depend on
// each other are issued together: the current query with the slot and
// position, then the summaries with the rotary row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void qhat_slice(int pair, int tt, const float* __restrict__ qstate,
                                           const float* __restrict__ qcur,
                                           const float* __restrict__ rope, int rope_rows,
                                           const int32_t* __restrict__ slot,
                                           const int32_t* __restrict__ position, int L, int M,
                                           int Hq, int Hkv, float* __restrict__ qhat,
                                           int32_t* __restrict__ err) {
  const int r = pair / L, l = pair % L;
  const int x = tt / Hq, hq = tt % Hq;
  const int s_raw = slot[r], pos_raw = position[r];
  const float4* qt = reinterpret_cast<const float4*>(qcur + (((int64_t)r * L + l) * Hq + hq) * kD);
  float4 tv[kD / 4];
#pragma unroll
  for (int i = 0; i < kD / 4; ++i) tv[i] = qt[i];
  const bool zero = s_raw < 0 || s_raw >= M;
  if (zero && tt == 0) atomicOr(err, GP_DEVERR_SLOT);
  const int s = zero ? 0 : s_raw;
  const bool pos_bad = pos_raw < 0 || pos_raw >= rope_rows;
  if (pos_bad && tt == 0) atomicOr(err, GP_DEVERR_POSITION);
  const int pos = pos_raw < 0 ? 0 : (pos_raw >= rope_rows ? rope_rows - 1 : pos_raw);
  const float4* qb =
      reinterpret_cast<const float4*>(qstate + ((((int64_t)l * M + s) * 2 + x) * Hq + hq) * kD);
  const float4* cs = reinterpret_cast<const float4*>(rope + (int64_t)pos * kD);
  constexpr int hq4 = kD / 8;  // quads per half
  float4 bv[kD / 4], cv[kD / 4];
#pragma unroll
  for (int i = 0; i < kD / 4; ++i) {
    bv[i] = qb[i];
    cv[i] = cs[i];
  }
  float ssq = 0.0f, ssx = 0.0f;
#pragma unroll
  for (int i = 0; i < kD / 4; ++i) {
    ssq = __builtin_fmaf(tv[i].x, tv[i].x, ssq);
    ssq = __builtin_fmaf(tv[i].y, tv[i].y, ssq);
    ssq = __builtin_fmaf(tv[i].z, tv[i].z, ssq);
    ssq = __builtin_fmaf(tv[i].w, tv[i].w, ssq);
  }
#pragma unroll
  for (int i = 0; i < kD / 4; ++i) {
    ssx = __builtin_fmaf(bv[i].x, bv[i].x, ssx);
    ssx = __builtin_fmaf(bv[i].y, bv[i].y, ssx);
    ssx = __builtin_fmaf(bv[i].z, bv[i].z, ssx);
    ssx = __builtin_fmaf(bv[i].w, bv[i].w, ssx);
  }
  float gamma = ssx > 0.0f ? __builtin_sqrtf(ssq / ssx) : 0.0f;
  if (zero) gamma = 0.0f;
  const float scale = 1.0f / __builtin_sqrtf((float)kD);
  const int kvh = hq / kGroup, qi = x * kGroup + hq % kGroup;
  float* out = qhat + (((int64_t)r * L + l) * Hkv + kvh) * (kNQ * kD);
  // element j of the first half pairs with j + d/2; quad i holds j = 4i .. 4i+3
  auto rot = [&](float b1, float b2, float c, float sn, float& y1, float& y2) {
    const float a = gamma * b1, c2 = gamma * b2;
    y1 = __builtin_fmaf(a, c, -(c2 * sn)) * scale;
    y2 = __builtin_fmaf(c2, c, a * sn) * scale;
  };
#pragma unroll
  for (int i = 0; i < hq4; ++i) {
    const float4 c = cv[i], sn = cv[hq4 + i], b1 = bv[i], b2 = bv[hq4 + i];
    float4 y1, y2;
    rot(b1.x, b2.x, c.x, sn.x, y1.x, y2.x);
    rot(b1.y, b2.y, c.y, sn.y, y1.y, y2.y);
    rot(b1.z, b2.z, c.z, sn.z, y1.z, y2.z);
    rot(b1.w, b2.w, c.w, sn.w, y1.w, y2.w);
    *reinterpret_cast<float4*>(out + i * 32 + qi * 4) = y1;
    *reinterpret_cast<float4*>(out + (hq4 + i) * 32 + qi * 4) = y2;
  }
}

// The summaries launch: block p < B L computes the rotated summaries of
// (request, layer) pair p, block B L runs the plan.
__global__ __launch_bounds__(kPrepT) void k_prep(
    const float* __restrict__ qstate, const float* __restrict__ qcur,
    const float* __restrict__ rope, int rope_rows, const int32_t* __restrict__ slot,
    const int32_t* __restrict__ position, int L, int M, int Hq, int Hkv,
    float* __restrict__ qhat, const int32_t* __restrict__ num_pages, int B, int max_pages,
    int64_t host_total_pages, int b, int64_t ring_tokens, WsHeader* __restrict__ hdr,
    int64_t* __restrict__ page_off, int32_t* __restrict__ req_order,
    int32_t* __restrict__ req_flags, int32_t* __restrict__ err) {
  if ((int)blockIdx.x == B * L) {
    plan_block(num_pages, B, max_pages, host_total_pages, b, ring_tokens, hdr, page_off,
               req_order, req_flags, err);
    return;
  }
  const int t = threadIdx.x;
  if (t >= 2 * Hq) return;
  qhat_slice((int)blockIdx.x, t, qstate, qcur, rope, rope_rows, slot, position, L, M, Hq, Hkv,
             qhat, err);
}

hipError_t launch_prep(const Params& p, const WsLayout& w, const float* qstate, const float* qcur,
                       const float* rope, int rope_rows, const int32_t* slot,
                       const int32_t* position, const int32_t* num_pages_dev, int B,
                       int max_pages, int64_t host_total_pages, void* ws, int32_t* err,
                       hipStream_t s) {
  if (2 * p.Hq > kPrepT) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  hipLaunchKernelGGL(k_prep, dim3((unsigned)(B * p.L + 1)), dim3(kPrepT), 0, s, qstate, qcur,
                     rope, rope_rows, slot, position, p.L, p.M, p.Hq, p.Hkv,
                     reinterpret_cast<float*>(base + w.qhat), num_pages_dev, B, max_pages,
                     host_total_pages, p.b, w.ring_tokens,
                     reinterpret_cast<WsHeader*>(base + w.header),
                     reinterpret_cast<int64_t*>(base + w.page_off),
                     reinterpret_cast<int32_t*>(base + w.req_order),
                     reinterpret_cast<int32_t*>(base + w.req_flags), err);
  return hipGetLastError();
}

}  // namespace gp
