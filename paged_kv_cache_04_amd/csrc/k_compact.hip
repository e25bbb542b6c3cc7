// A9: in-place compaction of one row's K or V chain (§3.3 "compacted within
// the existing physical-page allocation"; §4.2; App. E.2: at most (P - 1) b
// occupied slots).  Citations are to "GrowPage: On-Demand KV Budgeting for
// Efficient LLM Reasoning Serving" (arXiv 2609.03494).
//
// Kept slots keep their order and move to destination j = slot - #(dropped
// before slot); for destination j the source is j + #{k : d_k - k <= j},
// found by binary search over the sorted dropped slots d_k (b of them, 2b for
// a Shrink row of the GrowPage-Shrink policy, App. H.1) (one search
// per destination row, kept with both addresses in a per-chunk table).
// Slots before the first dropped one stay where they are.  Each source lies
// at most 2b slots after its destination, so the workgroup (1024 threads)
// walks destinations in 1024-row chunks (256 KiB, 16 pieces of 16 bytes per
// thread): it loads a whole chunk into registers, waits for the loads and
// barriers, then stores.
// Loads and stores are non-temporal: each byte is touched once, and keeping
// it out of the caches leaves them to the next event's demand pass.  A
// chunk's stores land below every later chunk's sources, and every earlier
// chunk has finished reading, so the in-place move needs no copy of the row.
// K and V rows, and different rows, are disjoint items.  A persistent grid
// takes the items of the requests that compress, in the plan's request
// order (longest first), from a queue (one atomic per item, a few µs against
// an item's hundreds), so the rows whose first drop comes late and leave less
// to move do not leave compute units idle at the end; its size is a context
// setting, so that compression on a second stream can leave CUs to decoding
// (App. E.3).
// Prefix-preserving compression (App. E.2): a shared page i of the request
// has a target page, and destinations in page i are written there instead.
// Sources stay in the old pages, which are only read, so the move is still
// in place for every other page; rows from the first replaced page on are
// copied even before the first dropped slot (their destination page is new).
#include "gp_internal.h"

namespace gp {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCT = 1024;                     // threads
constexpr int kPer = 16;                      // 16-byte pieces per thread per chunk
constexpr int kRowsC = kCT * kPer / 16;       // destination rows per chunk (1024)
constexpr int kMaxPages = 65536 / kPage;      // pages per row held in LDS
static_assert(kRowsC <= kCT, "one chunk-table row per thread");
static_assert(kMaxBatch <= kCT, "one request of the batch per thread");

__global__ __launch_bounds__(kCT) void k_compact(int L, int Hkv, int b, int stride,
                                                 int pool_pages,
                                                 const WsHeader* __restrict__ hdr,
                                                 int32_t* __restrict__ item_counter,
                                                 const int64_t* __restrict__ page_off,
                                                 const int32_t* __restrict__ req_order,
                                                 int B,
                                                 const int8_t* __restrict__ action,
                                                 uint16_t* __restrict__ k_pool,
                                                 uint16_t* __restrict__ v_pool,
                                                 const int32_t* __restrict__ block_table,
                                                 int max_pages, int32_t* __restrict__ num_tokens,
                                                 const int32_t* __restrict__ dropped,
                                                 const int32_t* __restrict__ target,
                                                 int32_t* __restrict__ req_flags,
                                                 int32_t* __restrict__ err) {
  __shared__ int32_t gap[2 * kPage];
  __shared__ int32_t pg[kMaxPages];   // source pages
  __shared__ int32_t pgd[kMaxPages];  // destination pages
  __shared__ int64_t s_src[2][kRowsC];
  __shared__ int64_t s_dst[2][kRowsC];
  __shared__ int32_t creq[kMaxBatch];  // requests that compress, in the plan's order
  __shared__ uint32_t s_w[kCT / 64];
  __shared__ int bad, first_new, s_it;
  if (!hdr->valid) return;
  const int LH = L * Hkv;
  const int t = threadIdx.x;
  // whether request r has rows to move (the item below checks the same)
  auto compresses = [&](int r) -> bool {
    const int8_t act = action ? action[r] : (int8_t)GP_COMPRESS;
    const int64_t P = page_off[r + 1] - page_off[r];
    const int32_t flags = req_flags[r];
    if (act != GP_COMPRESS && (act != GP_SHRINK || stride < 2 * b)) return false;
    const int m = act == GP_SHRINK ? 2 : 1;
    return P >= m + 1 && !(flags & (kReqBlocked | kReqTooLong));
  };
  // one item: the K (which 0) or V (which 1) chain of row (r, lh); every
  // value that steers a branch is workgroup-uniform and read into a scalar
  auto item = [&](int r, int lh, int which) {
    const int row = r * LH + lh;
    // the request's metadata in one round of loads
    const int8_t act = action ? action[r] : (int8_t)GP_COMPRESS;
    const int P = __builtin_amdgcn_readfirstlane((int)(page_off[r + 1] - page_off[r]));
    const int32_t flags = __builtin_amdgcn_readfirstlane(req_flags[r]);
    if (act != GP_COMPRESS && act != GP_SHRINK) return;
    if (act == GP_SHRINK && stride < 2 * b) return;  // Shrink outside its policy: ignored
    const int m = act == GP_SHRINK ? 2 : 1;  // pages of slots freed
    const int nd = m * b;                    // dropped slots
    if (P < m + 1) return;
    // pages short (App. E.2), or longer than the selection takes
    if (flags & (kReqBlocked | kReqTooLong)) return;
    const int l = lh / Hkv, h = lh % Hkv;
    if (t == 0) {
      bad = 0;
      first_new = P;
    }
    __syncthreads();
    for (int k = t; k < nd; k += kCT) gap[k] = dropped[(int64_t)row * stride + k] - k;
    for (int i = t; i < P; i += kCT) {
      const int page = block_table[(int64_t)r * max_pages + i];
      int dst = page;
      if (target) {
        const int tg = target[page_off[r] + i];
        if (tg >= 0) {
          dst = tg;
          atomicMin(&first_new, i);
        }
      }
      if (page < 0 || page >= pool_pages || dst < 0 || dst >= pool_pages) bad = 1;
      pg[i] = page;
      pgd[i] = dst;
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(bad)) {
      if (t == 0) atomicOr(err, GP_DEVERR_PAGE);
      return;
    }
    uint16_t* pool = which ? v_pool : k_pool;
    // element offset of slot i of this row in physical page `page`
    auto slot_base = [&](int page, int i) -> int64_t {
      return (((int64_t)l * pool_pages + page) * Hkv + h) * (int64_t)(kPage * kD) +
             (int64_t)(i & (kPage - 1)) * kD;
    };
    const int end = (P - m) * b;
    const int g0 = __builtin_amdgcn_readfirstlane(gap[0]);
    const int fn = __builtin_amdgcn_readfirstlane(first_new);
    const int d0 = g0 > 0 ? g0 : 0;
    const int start = fn * b < d0 ? fn * b : d0;
    int par = 0;
    for (int c0 = start; c0 < end; c0 += kRowsC, par ^= 1) {
      // source and destination offsets of the chunk's destination rows,
      // one binary search per thread (tables alternate between two buffers
      // so the next chunk's tables never overwrite ones still being read)
      {
        const int drow = c0 + t;
        if (t < kRowsC && drow < end) {
          int lo = 0, hi = nd;
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (gap[mid] <= drow) lo = mid + 1; else hi = mid;
          }
          const int srow = drow + lo;
          s_src[par][t] = slot_base(pg[srow >> 8], srow);
          s_dst[par][t] = slot_base(pgd[drow >> 8], drow);
        }
      }
      __syncthreads();
      const int nrows = end - c0 < kRowsC ? end - c0 : kRowsC;
      u32x4 v[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int piece = u * kCT + t;
        const int ri = piece >> 4, part = piece & 15;
        if (ri < nrows)
          v[u] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(pool + s_src[par][ri] + part * 8));
      }
      // every source of this chunk must be read before any of its stores
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int piece = u * kCT + t;
        const int ri = piece >> 4, part = piece & 15;
        if (ri < nrows)
          __builtin_nontemporal_store(v[u],
                                      reinterpret_cast<u32x4*>(pool + s_dst[par][ri] + part * 8));
      }
    }
    if (lh == 0 && which == 0 && t == 0) {
      num_tokens[r] = end;
      req_flags[r] = kReqCompacted;
    }
  };
  // the compressing requests in the plan's order (longest first), 2 LH
  // items each, handed out one at a time by the queue
  int r_t = -1;
  if (t < B) {
    r_t = req_order[t];
    if (!compresses(r_t)) r_t = -1;
  }
  uint32_t n_c;
  const uint32_t pos = block_prefix_excl_u32(r_t >= 0 ? 1u : 0u, s_w, kCT / 64, n_c);
  if (r_t >= 0) creq[pos] = r_t;
  __syncthreads();
  const int n_items = 2 * LH * (int)n_c;
  if (n_items == 0) return;
  for (;;) {
    if (t == 0) s_it = atomicAdd(item_counter, 1);
    __syncthreads();
    const int it = s_it;
    __syncthreads();  // every thread has the item before the next one is fetched
    if (it >= n_items) break;
    const int r = creq[it / (2 * LH)];
    const int rem = it % (2 * LH);
    item(r, rem >> 1, rem & 1);
    __syncthreads();  // the next item rewrites the LDS tables
  }
}

hipError_t launch_compact(const Params& p, const WsLayout& w, int B, const int8_t* action,
                          uint16_t* k_pool, uint16_t* v_pool, int pool_pages,
                          const int32_t* block_table, int max_pages, int32_t* num_tokens,
                          bool shared, int groups, void* ws, int32_t* err, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  const int64_t n_items = w.rows * 2;
  const int64_t grid = groups < n_items ? groups : n_items;
  hipLaunchKernelGGL(k_compact, dim3((unsigned)grid), dim3(kCT), 0, s, p.L, p.Hkv, p.b,
                     p.b * p.max_freed(), pool_pages,
                     reinterpret_cast<const WsHeader*>(base + w.header),
                     &reinterpret_cast<WsHeader*>(base + w.header)->item_counter,
                     reinterpret_cast<const int64_t*>(base + w.page_off),
                     reinterpret_cast<const int32_t*>(base + w.req_order), B, action,
                     k_pool, v_pool,
                     block_table, max_pages, num_tokens,
                     reinterpret_cast<const int32_t*>(base + w.dropped),
                     shared ? reinterpret_cast<const int32_t*>(base + w.target) : nullptr,
                     reinterpret_cast<int32_t*>(base + w.req_flags), err);
  return hipGetLastError();
}

}  // namespace gp
