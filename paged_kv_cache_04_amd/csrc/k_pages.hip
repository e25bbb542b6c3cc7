// Page bookkeeping around the compaction of Compress & Hold and Shrink:
// prefix-preserving compression (App. E.2) and Shrink's page return
// (App. H.1).  Citations are to "GrowPage: On-Demand KV Budgeting for
// Efficient LLM Reasoning Serving" (arXiv 2609.03494).
//
// Both kernels are one 1024-thread workgroup (the batch limit).  Per-request
// page scans use one wave per request with lanes over its pages; decisions
// that depend on request order use a block-wide prefix sum in LDS.
#include "gp_internal.h"

namespace gp {

namespace {

constexpr int kWaves = kMaxBatch / 64;

// Inclusive prefix sum of v[0 .. kMaxBatch) in place (every thread calls).
__device__ void block_scan(int* v) {
  const int t = threadIdx.x;
  for (int off = 1; off < kMaxBatch; off <<= 1) {
    const int add = t >= off ? v[t - off] : 0;
    __syncthreads();
    v[t] += add;
    __syncthreads();
  }
}

// Pages of a compressing request that stay in its block table and may be
// written by the compaction or by later decoding: all P for Compress & Hold,
// the first P - 1 for Shrink (its last page is released); 0 for a request
// that does not compress.  Mirrors the action checks of the select and
// compaction kernels (a Shrink counts only when the dropped-slot stride has
// room for 2b slots, i.e. under the GrowPage-Shrink policy).
__device__ int kept_pages(const int8_t* action, int r, int64_t P, int b, int stride,
                          int32_t flags) {
  const int8_t act = action ? action[r] : (int8_t)GP_COMPRESS;
  if (flags & kReqTooLong) return 0;  // the selection skips it
  int m = 0;
  if (act == GP_COMPRESS) m = 1;
  if (act == GP_SHRINK && stride >= 2 * b) m = 2;
  if (m == 0 || P < m + 1) return 0;
  return (int)(m == 1 ? P : P - 1);
}

__device__ __forceinline__ int load_agent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// ---------------------------------------------------------------------------
// Before selection (App. E.2): a page referenced more than once is never
// written by a request's compression, so each compressing request needs a
// new target page for every shared page it keeps.  Requests are served in
// index order from the top of the free stack: with need_r the request's
// shared kept pages and S_r their inclusive prefix sum over the batch,
// request r is served iff need_r = 0 or S_r <= free_count, and its k-th
// shared page (page order) gets free_stack[free_count - 1 - (S_r - need_r + k)].
// Since S_r only grows, the first request that cannot be served blocks every
// later one that needs a page, as in a serial walk that stops allocating at
// the first failure.  target[page_off[r] + i] = new page or -1;
// req_flags[r] = kReqBlocked for a request left uncompressed.  A request the
// batch plan flagged kReqTooLong is not compressed: it needs no target and
// keeps its flag.
// counters[4] counts the pages allocated.  Launched only with reference
// counts (the batch plan clears req_flags); on a rejected batch it clears
// req_flags and returns.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kMaxBatch) void k_share(int B, int b, int stride, int pool_pages,
                                                     const WsHeader* __restrict__ hdr,
                                                     const int64_t* __restrict__ page_off,
                                                     const int8_t* __restrict__ action,
                                                     const int32_t* __restrict__ block_table,
                                                     int max_pages,
                                                     const int32_t* __restrict__ refcount,
                                                     const int32_t* __restrict__ free_stack,
                                                     int32_t* __restrict__ free_count,
                                                     int32_t* __restrict__ target,
                                                     int32_t* __restrict__ req_flags,
                                                     int64_t* __restrict__ counters,
                                                     int32_t* __restrict__ err) {
  __shared__ int cum[kMaxBatch];
  __shared__ int s_used, s_blocked;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  if (!refcount || !hdr->valid) {
    if (t < B) req_flags[t] = 0;
    return;
  }
  if (t == 0) s_used = s_blocked = 0;
  cum[t] = 0;
  __syncthreads();
  for (int r = wv; r < B; r += kWaves) {
    const int64_t P = page_off[r + 1] - page_off[r];
    const int keep = kept_pages(action, r, P, b, stride, req_flags[r]);
    const int32_t* bt = block_table + (int64_t)r * max_pages;
    int cnt = 0;
    for (int i0 = 0; i0 < keep; i0 += 64) {
      const int i = i0 + lane;
      bool sh = false;
      if (i < keep) {
        const int page = bt[i];
        sh = page >= 0 && page < pool_pages && refcount[page] > 1;
      }
      cnt += __popcll(__ballot(sh));
    }
    if (lane == 0) cum[r] = cnt;
  }
  __syncthreads();
  block_scan(cum);
  const int fc0 = *free_count;
  const bool fc_ok = fc0 >= 0 && fc0 <= pool_pages;
  const int fc = fc_ok ? fc0 : 0;
  if (t < B && cum[t] <= fc) atomicMax(&s_used, cum[t]);
  for (int r = wv; r < B; r += kWaves) {
    const int incl = cum[r];
    const int own = incl - (r > 0 ? cum[r - 1] : 0);
    const bool served = own == 0 || incl <= fc;
    const int32_t flags = __builtin_amdgcn_readfirstlane(req_flags[r]);
    if (lane == 0) {
      req_flags[r] = (flags & kReqTooLong) | (served ? 0 : kReqBlocked);
      if (!served) s_blocked = 1;
    }
    const int64_t P = page_off[r + 1] - page_off[r];
    const int keep = served ? kept_pages(action, r, P, b, stride, flags) : 0;
    const int32_t* bt = block_table + (int64_t)r * max_pages;
    int32_t* tg = target + page_off[r];
    int taken = incl - own;
    for (int i0 = 0; i0 < (int)P; i0 += 64) {
      const int i = i0 + lane;
      bool sh = false;
      if (i < keep) {
        const int page = bt[i];
        sh = page >= 0 && page < pool_pages && refcount[page] > 1;
      }
      const uint64_t mask = __ballot(sh);
      const int rank = __popcll(mask & ((1ull << lane) - 1ull));
      if (i < (int)P) tg[i] = sh ? free_stack[fc - 1 - (taken + rank)] : -1;
      taken += __popcll(mask);
    }
  }
  __syncthreads();
  if (t == 0) {
    if (fc_ok) *free_count = fc - s_used;
    else atomicOr(err, GP_DEVERR_PAGES);
    counters[4] += s_used;
    if (s_blocked) atomicOr(err, GP_DEVERR_NOPAGE);
  }
}

hipError_t launch_share(const Params& p, const WsLayout& w, int B, const int8_t* action,
                        int pool_pages, const int32_t* block_table, int max_pages,
                        const int32_t* refcount, const int32_t* free_stack, int32_t* free_count,
                        void* ws, int64_t* counters, int32_t* err, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  hipLaunchKernelGGL(k_share, dim3(1), dim3(kMaxBatch), 0, s, B, p.b, p.b * p.max_freed(),
                     pool_pages, reinterpret_cast<const WsHeader*>(base + w.header),
                     reinterpret_cast<const int64_t*>(base + w.page_off), action, block_table,
                     max_pages, refcount, free_stack, free_count,
                     reinterpret_cast<int32_t*>(base + w.target),
                     reinterpret_cast<int32_t*>(base + w.req_flags), counters, err);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// After the compaction of the event.
// (1) Prefix sharing (App. E.2): every replaced page of a compacted request
//     is swapped in its block table for its target; the old page loses the
//     request's reference, the target has one.  A page whose count reaches
//     zero stays with the caller (a prefix cache keeps such pages until it
//     evicts them).
// (2) Shrink (App. H.1): a compacted Shrink request releases its last page:
//     its block-table entry becomes -1 and P -= 1.  Without reference counts
//     the page goes back on the free stack.  With them the request drops its
//     reference, and the page goes back only when no reference is left; a
//     page shared by several shrinking requests goes back with the one of
//     highest index (a serial walk in index order decrements until the last
//     reference).  Pages go back in request order: the k-th to free_stack[
//     free_count + k].  counters[3] counts them.
// A free count outside [0, pool_pages], or a push beyond the stack, flags
// GP_DEVERR_PAGES.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kMaxBatch) void k_return(int B, int max_pages, int pool_pages,
                                                      const int64_t* __restrict__ page_off,
                                                      const int32_t* __restrict__ req_flags,
                                                      const int32_t* __restrict__ target,
                                                      int32_t* __restrict__ block_table,
                                                      int32_t* __restrict__ num_pages,
                                                      int32_t* __restrict__ free_stack,
                                                      int32_t* __restrict__ free_count,
                                                      int32_t* __restrict__ refcount,
                                                      const int8_t* __restrict__ action,
                                                      int64_t* __restrict__ counters,
                                                      int32_t* __restrict__ err) {
  __shared__ int scan[kMaxBatch];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int fc = *free_count;
  if (fc < 0 || fc > pool_pages) {
    if (t == 0) atomicOr(err, GP_DEVERR_PAGES);
    return;
  }
  if (refcount) {
    for (int r = wv; r < B; r += kWaves) {
      if (!(req_flags[r] & kReqCompacted)) continue;
      const int P = (int)(page_off[r + 1] - page_off[r]);
      const int32_t* tg = target + page_off[r];
      int32_t* bt = block_table + (int64_t)r * max_pages;
      for (int i = lane; i < P; i += 64) {
        const int32_t page = tg[i];
        if (page < 0) continue;
        atomicSub(&refcount[bt[i]], 1);
        refcount[page] = 1;
        bt[i] = page;
      }
    }
  }
  __syncthreads();
  int P = 0;
  int32_t last = -1;
  bool want = false;
  if (t < B && action && action[t] == GP_SHRINK && (req_flags[t] & kReqCompacted)) {
    P = (int)(page_off[t + 1] - page_off[t]);
    want = true;  // compacted as a Shrink: P >= 3 and its pages were checked
    last = block_table[(int64_t)t * max_pages + (P - 1)];
  }
  bool push = want;
  if (refcount) {
    if (want) atomicSub(&refcount[last], 1);
    __syncthreads();
    const bool freed = want && load_agent(&refcount[last]) <= 0;
    __syncthreads();
    if (freed) atomicMin(&refcount[last], -(t + 1));
    __syncthreads();
    push = freed && load_agent(&refcount[last]) == -(t + 1);
    __syncthreads();
    if (push) atomicExch(&refcount[last], 0);
  }
  scan[t] = push ? 1 : 0;
  __syncthreads();
  block_scan(scan);
  const int total = scan[kMaxBatch - 1];
  if (fc + total > pool_pages) {
    if (t == 0) atomicOr(err, GP_DEVERR_PAGES);
    return;
  }
  if (push) free_stack[fc + scan[t] - 1] = last;
  if (want) {
    block_table[(int64_t)t * max_pages + (P - 1)] = -1;
    num_pages[t] = P - 1;
  }
  if (t == 0) {
    *free_count = fc + total;
    counters[3] += total;
  }
}

hipError_t launch_return(const WsLayout& w, int B, int max_pages, int pool_pages,
                         int32_t* block_table, int32_t* num_pages, int32_t* free_stack,
                         int32_t* free_count, int32_t* refcount, const int8_t* action,
                         const void* ws, int64_t* counters, int32_t* err, hipStream_t s) {
  const char* base = static_cast<const char*>(ws);
  hipLaunchKernelGGL(k_return, dim3(1), dim3(kMaxBatch), 0, s, B, max_pages, pool_pages,
                     reinterpret_cast<const int64_t*>(base + w.page_off),
                     reinterpret_cast<const int32_t*>(base + w.req_flags),
                     reinterpret_cast<const int32_t*>(base + w.target), block_table, num_pages,
                     free_stack, free_count, refcount, action, counters, err);
  return hipGetLastError();
}

}  // namespace gp
