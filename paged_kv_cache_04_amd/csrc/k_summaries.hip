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
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_plan(const int32_t* __restrict__ num_pages, int B,
                                               int max_pages, int64_t host_total_pages, int b,
                                               int64_t ring_tokens, WsHeader* __restrict__ hdr,
                                               int64_t* __restrict__ page_off,
                                               int32_t* __restrict__ req_order,
                                               int32_t* __restrict__ req_flags,
                                               int32_t* __restrict__ err) {
  __shared__ int64_t buf[kMaxBatch];
  __shared__ int32_t pages[kMaxBatch];
  __shared__ int bad;
  const int t = threadIdx.x;
  if (t == 0) bad = 0;
  __syncthreads();
  int64_t v = 0;
  if (t < B) {
    const int P = num_pages[t];
    if (P < 1 || P > max_pages || (int64_t)P * b > ring_tokens) atomicOr(&bad, 1);
    v = P;
    pages[t] = P;
  }
  buf[t] = v;
  __syncthreads();
  for (int off = 1; off < kMaxBatch; off <<= 1) {
    const int64_t add = t >= off ? buf[t - off] : 0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  if (t < B) {
    req_flags[t] = (int64_t)pages[t] * b > kMaxCompressTokens ? kReqTooLong : 0;
    page_off[t + 1] = buf[t];
    const int32_t mine = pages[t];
    int rank = 0;
    for (int u = 0; u < B; ++u) rank += (pages[u] > mine) || (pages[u] == mine && u < t);
    req_order[rank] = t;
  }
  if (t == 0) {
    page_off[0] = 0;
    const int64_t total = buf[B - 1];
    const int ok = (!bad) && total == host_total_pages;
    hdr->magic = kWsMagic;
    hdr->batch = B;
    hdr->total_tokens = total * b;
    hdr->row_counter = 0;
    hdr->valid = ok;
    if (!ok) atomicOr(err, GP_DEVERR_PAGES);
  }
}

hipError_t launch_plan(const Params& p, const WsLayout& w, const int32_t* num_pages_dev, int B,
                       int max_pages, int64_t host_total_pages, void* ws, int32_t* err,
                       hipStream_t s) {
  char* base = static_cast<char*>(ws);
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kMaxBatch), 0, s, num_pages_dev, B, max_pages,
                     host_total_pages, p.b, w.ring_tokens,
                     reinterpret_cast<WsHeader*>(base + w.header),
                     reinterpret_cast<int64_t*>(base + w.page_off),
                     reinterpret_cast<int32_t*>(base + w.req_order),
                     reinterpret_cast<int32_t*>(base + w.req_flags), err);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// A1: calibrated, rotated summaries (App. E.1 Eq. 12 and the paragraph after
// it).  One block per (request, layer); thread x*Hq + hq handles summary x of
// query head hq:
//   gamma = sqrt(ss(q_t) / ss(qbar)) (serial fmaf sums of squares; 0 when
//   ss(qbar) = 0), qtilde = gamma * qbar, rotate-half rotary at the current
//   position with the caller's (cos, sin) row, times 1/sqrt(d).
// Output layout per row (request, layer, KV head): [32 quads][8 queries][4],
// query index x * 4 + g for the g-th query head of the KV head (GQA grouping
// of consecutive query heads); element j sits in quad j / 4 at j % 4, so the
// scoring kernel reads the 32 values of one 4-element key quad contiguously.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_qhat(const float* __restrict__ qstate,
                                              const float* __restrict__ qcur,
                                              const float* __restrict__ rope, int rope_rows,
                                              const int32_t* __restrict__ slot,
                                              const int32_t* __restrict__ position, int L, int M,
                                              int Hq, int Hkv, const WsHeader* __restrict__ hdr,
                                              float* __restrict__ qhat, int32_t* __restrict__ err) {
  if (!hdr->valid) return;
  const int r = blockIdx.x / L, l = blockIdx.x % L;
  const int t = threadIdx.x;
  if (t >= 2 * Hq) return;
  const int x = t / Hq, hq = t % Hq;
  int s = slot[r];
  bool zero = false;
  if (s < 0 || s >= M) {
    if (t == 0) atomicOr(err, GP_DEVERR_SLOT);
    zero = true;
    s = 0;
  }
  int pos = position[r];
  if (pos < 0 || pos >= rope_rows) {
    if (t == 0) atomicOr(err, GP_DEVERR_POSITION);
    pos = pos < 0 ? 0 : rope_rows - 1;
  }
  // both vectors are read with 16-byte loads, all issued before the serial
  // sums of squares run over them in index order
  const float4* qt = reinterpret_cast<const float4*>(qcur + (((int64_t)r * L + l) * Hq + hq) * kD);
  const float4* qb =
      reinterpret_cast<const float4*>(qstate + ((((int64_t)l * M + s) * 2 + x) * Hq + hq) * kD);
  float4 tv[kD / 4], bv[kD / 4];
#pragma unroll
  for (int i = 0; i < kD / 4; ++i) {
    tv[i] = qt[i];
    bv[i] = qb[i];
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
  const float4* cs = reinterpret_cast<const float4*>(rope + (int64_t)pos * kD);
  const int kvh = hq / kGroup, qi = x * kGroup + hq % kGroup;
  float* out = qhat + (((int64_t)r * L + l) * Hkv + kvh) * (kNQ * kD);
  // element j of the first half pairs with j + d/2; quad i holds j = 4i .. 4i+3
  constexpr int hq4 = kD / 8;  // quads per half
  auto rot = [&](float b1, float b2, float c, float sn, float& y1, float& y2) {
    const float a = gamma * b1, c2 = gamma * b2;
    y1 = __builtin_fmaf(a, c, -(c2 * sn)) * scale;
    y2 = __builtin_fmaf(c2, c, a * sn) * scale;
  };
#pragma unroll
  for (int i = 0; i < hq4; ++i) {
    const float4 c = cs[i], sn = cs[hq4 + i], b1 = bv[i], b2 = bv[hq4 + i];
    float4 y1, y2;
    rot(b1.x, b2.x, c.x, sn.x, y1.x, y2.x);
    rot(b1.y, b2.y, c.y, sn.y, y1.y, y2.y);
    rot(b1.z, b2.z, c.z, sn.z, y1.z, y2.z);
    rot(b1.w, b2.w, c.w, sn.w, y1.w, y2.w);
    *reinterpret_cast<float4*>(out + i * 32 + qi * 4) = y1;
    *reinterpret_cast<float4*>(out + (hq4 + i) * 32 + qi * 4) = y2;
  }
}

hipError_t launch_qhat(const Params& p, const WsLayout& w, const float* qstate, const float* qcur,
                       const float* rope, int rope_rows, const int32_t* slot,
                       const int32_t* position, int B, void* ws, int32_t* err, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  hipLaunchKernelGGL(k_qhat, dim3((unsigned)(B * p.L)), dim3(256), 0, s, qstate, qcur, rope,
                     rope_rows, slot, position, p.L, p.M, p.Hq, p.Hkv,
                     reinterpret_cast<const WsHeader*>(base + w.header),
                     reinterpret_cast<float*>(base + w.qhat), err);
  return hipGetLastError();
}

}  // namespace gp
