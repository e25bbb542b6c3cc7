// A5: request-level trend and decision; A6: Grow by One Page with fallback.
// Citations are to "GrowPage: On-Demand KV Budgeting for Efficient LLM
// Reasoning Serving" (arXiv 2609.03494).
#include "gp_internal.h"

namespace gp {

// ---------------------------------------------------------------------------
// A5 (§3.2 Eq. 8 and the threshold rule).  r^x is the mean over the L*Hkv
// (layer, KV head) pairs of K^x / |C_t|, so Delta = (sum K^S - sum K^L) /
// (L * Hkv * |C_t|), evaluated in fp64 from the exact integer difference.
// Grow iff Delta > tau.  A request of one page has no candidates: Delta = 0
// and it grows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_decide(int LH, int b, double tau, int policy,
                                                double shrink_tau, int min_tokens,
                                                const WsHeader* __restrict__ hdr,
                                                const int64_t* __restrict__ page_off,
                                                const int32_t* __restrict__ k_short,
                                                const int32_t* __restrict__ k_long,
                                                int64_t* __restrict__ k_diff,
                                                double* __restrict__ delta,
                                                int8_t* __restrict__ decision) {
  __shared__ int64_t red[4];
  const int r = blockIdx.x, t = threadIdx.x;
  // every load is issued before the batch's validity is looked at (all of
  // them lie inside the outputs of a valid launch; a rejected batch returns
  // before any value is used)
  const int valid = hdr->valid;
  const int64_t off0 = page_off[r], off1 = page_off[r + 1];
  int64_t s = 0;
  for (int i = t; i < LH; i += 256)
    s += (int64_t)k_short[(int64_t)r * LH + i] - (int64_t)k_long[(int64_t)r * LH + i];
  if (!valid) return;
  s = (int64_t)wave_sum_u64((uint64_t)s);  // two's complement: the wrap-around sum is exact
  if ((t & 63) == 0) red[t >> 6] = s;
  __syncthreads();
  if (t == 0) {
    const int64_t diff = red[0] + red[1] + red[2] + red[3];
    const int64_t P = off1 - off0;
    const int64_t card = (P - 1) * b;
    double dl = 0.0;
    int grow = 1;
    if (card > 0) {
      dl = (double)diff / ((double)LH * (double)card);
      grow = dl > tau;
    }
    if (k_diff) k_diff[r] = diff;
    if (delta) delta[r] = dl;
    int8_t dec = grow ? GP_GROW : GP_COMPRESS;
    // GrowPage-Shrink (App. H.1 Eq. 13): below shrink_tau, and only while
    // (P - 1) b tokens of capacity, at least min_tokens, would remain; a
    // Shrink drops two pages of slots and keeps the recent window, so Eq. 10's
    // budget (P - 2) b - R needs P >= 3 (a shorter request compresses)
    if (policy == GP_POLICY_SHRINK && !grow && dl < shrink_tau && P >= 3 &&
        (P - 1) * b >= min_tokens)
      dec = GP_SHRINK;
    decision[r] = dec;
  }
}

hipError_t launch_decide(const Params& p, const WsLayout& w, int B, const void* ws,
                         const int32_t* k_short, const int32_t* k_long, int64_t* k_diff,
                         double* delta, int8_t* decision, hipStream_t s) {
  const char* base = static_cast<const char*>(ws);
  hipLaunchKernelGGL(k_decide, dim3(B), dim3(256), 0, s, p.L * p.Hkv, p.b, p.tau, p.policy,
                     p.shrink_tau, p.min_tokens,
                     reinterpret_cast<const WsHeader*>(base + w.header),
                     reinterpret_cast<const int64_t*>(base + w.page_off), k_short, k_long,
                     k_diff, delta, decision);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// A6 (§3.3 "Grow by One Page"; §4.2; App. H.2 defines a fallback).  Requests
// are served in index order: the k-th request (0-based, counting only those
// that want a page and have block-table room) is granted iff
// k < free_count - reserve, and takes free_stack[free_count - 1 - k], i.e.
// pages leave the top of the stack in request order.  That is the serial
// rule computed with one block-wide prefix count.  Everyone else, including
// growing requests that were refused, is marked for compression.
// A Shrink decision (GrowPage-Shrink policy) passes through as action
// GP_SHRINK and takes no page.  With reference counts (prefix sharing,
// App. E.2) a granted page gets one reference.
// counters: [0] pages granted, [1] compress actions, [2] fallbacks.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kMaxBatch) void k_grow(int B, int max_pages, int pool_pages,
                                                    int32_t* __restrict__ block_table,
                                                    int32_t* __restrict__ num_pages,
                                                    const int32_t* __restrict__ free_stack,
                                                    int32_t* __restrict__ free_count,
                                                    int reserve,
                                                    const int8_t* __restrict__ decision,
                                                    int8_t* __restrict__ action,
                                                    int32_t* __restrict__ refcount,
                                                    int64_t* __restrict__ counters,
                                                    int32_t* __restrict__ err) {
  __shared__ uint32_t s_w[kMaxBatch / 64];
  __shared__ int n_fallback, n_shrink;
  const int t = threadIdx.x;
  if (t == 0) n_fallback = n_shrink = 0;
  int fc = *free_count;
  if (fc < 0 || fc > pool_pages) {
    if (t == 0) atomicOr(err, GP_DEVERR_PAGES);
    fc = 0;
  }
  const int avail = fc - reserve > 0 ? fc - reserve : 0;
  bool dec_grow = false, want = false;
  int P = 0;
  if (t < B) {
    dec_grow = decision[t] == GP_GROW;
    P = num_pages[t];
    want = dec_grow && P >= 1 && P < max_pages;
  }
  uint32_t total_u = 0;
  const int rank = (int)block_prefix_excl_u32(want ? 1u : 0u, s_w, kMaxBatch / 64, total_u);
  const int total_want = (int)total_u;
  const bool granted = want && rank < avail;
  if (t < B) {
    if (granted) {
      const int page = free_stack[fc - 1 - rank];
      block_table[(int64_t)t * max_pages + P] = page;
      num_pages[t] = P + 1;
      if (refcount && page >= 0 && page < pool_pages) refcount[page] = 1;
      action[t] = GP_GROW;
    } else if (decision[t] == GP_SHRINK) {
      action[t] = GP_SHRINK;  // needs no page; gp_compress_hold returns one
      atomicAdd(&n_shrink, 1);
    } else {
      action[t] = GP_COMPRESS;
      if (dec_grow) atomicAdd(&n_fallback, 1);
    }
  }
  __syncthreads();
  if (t == 0) {
    const int n_grant = total_want < avail ? total_want : avail;
    *free_count = fc - n_grant;
    counters[0] += n_grant;
    counters[1] += B - n_grant - n_shrink;
    counters[2] += n_fallback;
  }
}

hipError_t launch_grow(int B, int max_pages, int pool_pages, int32_t* block_table,
                       int32_t* num_pages, const int32_t* free_stack, int32_t* free_count,
                       int reserve, const int8_t* decision, int8_t* action, int32_t* refcount,
                       int64_t* counters, int32_t* err, hipStream_t s) {
  hipLaunchKernelGGL(k_grow, dim3(1), dim3(kMaxBatch), 0, s, B, max_pages, pool_pages,
                     block_table, num_pages, free_stack, free_count, reserve, decision, action,
                     refcount, counters, err);
  return hipGetLastError();
}

}  // namespace gp
