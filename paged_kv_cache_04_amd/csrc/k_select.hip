// A7 + A8: Compress & Hold selection per (layer, KV head) row.
// Citations are to "GrowPage: On-Demand KV Budgeting for Efficient LLM
// Reasoning Serving" (arXiv 2609.03494): §3.3 Eq. 9 (importance), Eq. 10
// (block-local plus global selection), window mask (§3.3, §5.1).
//
// Candidates C = [0, N - R): the R newest slots are always kept.  Order:
// larger importance first, equal importance the newer slot first.  With
// exactly b candidates to drop per row, the selection is computed from the
// bottom:
//   step 1: each logical page (block) protects its top-min(k_loc, |B_j|)
//           candidates (one wave per block, 4 keys per lane, bit-serial
//           threshold search with ballots; ties broken by slot);
//   step 2: among the unprotected candidates, a 4-pass 8-bit radix select
//           finds the importance value v of the b-th smallest;
//   step 3: candidates below v are dropped, and of those equal to v the
//           oldest ones until exactly b are dropped (block-wide prefix count
//           in slot order); the dropped slots are written in ascending order.
// Importance values are non-negative fp32, so their bit patterns order like
// the values.
#include "gp_internal.h"

namespace gp {

constexpr int kSel = 1024;
constexpr int kMaxRowTokens = 65536;

// Exclusive prefix sum over the block (1024 threads); total in *total.
__device__ __forceinline__ int block_excl_scan(int v, int* buf, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) buf[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int w = lane < kSel / 64 ? buf[lane] : 0;
#pragma unroll
    for (int off = 1; off < kSel / 64; off <<= 1) {
      const int y = __shfl_up(w, off);
      if (lane >= off) w += y;
    }
    if (lane < kSel / 64) buf[lane] = w;
  }
  __syncthreads();
  const int base = wv > 0 ? buf[wv - 1] : 0;
  *total = buf[kSel / 64 - 1];
  __syncthreads();
  return base + x - v;
}

__global__ __launch_bounds__(kSel) void k_select(int L, int Hkv, int b, int R, int kloc,
                                                 const WsHeader* __restrict__ hdr,
                                                 const int64_t* __restrict__ page_off,
                                                 const int8_t* __restrict__ action,
                                                 const float* __restrict__ imp,
                                                 int32_t* __restrict__ dropped,
                                                 int32_t* __restrict__ dropped_out,
                                                 int32_t* __restrict__ err) {
  __shared__ uint32_t sloc[kMaxRowTokens / 32];
  __shared__ uint32_t hcnt[256];
  __shared__ int scanbuf[kSel / 64];
  __shared__ uint32_t s_prefix, s_below;
  if (!hdr->valid) return;
  const int LH = L * Hkv;
  const int row = blockIdx.x;
  const int r = row / LH, lh = row % LH;
  if (action && action[r] != GP_COMPRESS) return;
  const int64_t P = page_off[r + 1] - page_off[r];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  if (P < 2) {
    if (t == 0) atomicOr(err, GP_DEVERR_SHORT);
    return;
  }
  const int N = (int)(P * b), nc = N - R;
  const int64_t row_tok = (int64_t)LH * page_off[r] * b + (int64_t)lh * N;
  const float* __restrict__ s = imp + row_tok;

  // step 1: per-block quota S_loc as a bitmap
  for (int j = wv; j < P; j += kSel / 64) {
    const int blk = j * kPage;
    uint32_t key[4];
    bool valid[4], sel[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = blk + u * 64 + lane;
      valid[u] = i < nc;
      key[u] = valid[u] ? __float_as_uint(s[i]) : 0u;
      sel[u] = false;
    }
    const int nvalid = nc - blk < kPage ? nc - blk : kPage;
    const int k = kloc < nvalid ? kloc : nvalid;
    if (k > 0) {
      uint32_t th = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = th | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) cnt += __popcll(__ballot(valid[u] && key[u] >= cand));
        if (cnt >= k) th = cand;
      }
      int gt = 0;
      unsigned long long eqm[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        gt += __popcll(__ballot(valid[u] && key[u] > th));
        eqm[u] = __ballot(valid[u] && key[u] == th);
      }
      const int need = k - gt;
      const unsigned long long above_lane = lane == 63 ? 0ull : (~0ull << (lane + 1));
      int higher = 0;  // ties in rounds above u (newer slots)
#pragma unroll
      for (int u = 3; u >= 0; --u) {
        const int rank = higher + __popcll(eqm[u] & above_lane);
        sel[u] = valid[u] && (key[u] > th || (key[u] == th && rank < need));
        higher += __popcll(eqm[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const unsigned long long m = __ballot(sel[u]);
      if (lane == 0) {
        sloc[(blk + u * 64) >> 5] = (uint32_t)m;
        sloc[((blk + u * 64) >> 5) + 1] = (uint32_t)(m >> 32);
      }
    }
  }
  __syncthreads();

  // step 2: value of the b-th smallest unprotected candidate
  uint32_t prefix = 0, mask = 0, below = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int k = t; k < 256; k += kSel) hcnt[k] = 0;
    __syncthreads();
    for (int i = t; i < nc; i += kSel) {
      if ((sloc[i >> 5] >> (i & 31)) & 1u) continue;
      const uint32_t key = __float_as_uint(s[i]);
      if ((key & mask) == prefix) atomicAdd(&hcnt[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wv == 0) {
      uint32_t c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) c[u] = hcnt[4 * lane + u];
      const uint32_t lc = c[0] + c[1] + c[2] + c[3];
      uint32_t incl = lc;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      uint32_t cum = below + incl - lc;
      int best = -1;
      uint32_t best_below = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t before = cum;
        cum += c[u];
        if (best < 0 && cum >= (uint32_t)b) {
          best = 4 * lane + u;
          best_below = before;
        }
      }
      const unsigned long long ok = __ballot(best >= 0);
      const int ll = __ffsll((long long)ok) - 1;
      if (lane == ll) {
        s_prefix = prefix | ((uint32_t)best << shift);
        s_below = best_below;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    below = s_below;
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t v = prefix;
  const int need = b - (int)below;

  // step 3: ties at v go oldest first; write dropped slots in ascending order
  const int q = (nc + kSel - 1) / kSel;
  const int lo = t * q < nc ? t * q : nc;
  const int hi = lo + q < nc ? lo + q : nc;
  int ties = 0;
  for (int i = lo; i < hi; ++i)
    if (!((sloc[i >> 5] >> (i & 31)) & 1u) && __float_as_uint(s[i]) == v) ++ties;
  int total;
  const int tie0 = block_excl_scan(ties, scanbuf, &total);
  int nd = 0;
  {
    int tr = tie0;
    for (int i = lo; i < hi; ++i) {
      if ((sloc[i >> 5] >> (i & 31)) & 1u) continue;
      const uint32_t key = __float_as_uint(s[i]);
      if (key < v) ++nd;
      else if (key == v) nd += (tr++ < need);
    }
  }
  const int pos0 = block_excl_scan(nd, scanbuf, &total);
  int32_t* dst = dropped + (int64_t)row * b;
  int32_t* dst2 = dropped_out ? dropped_out + (int64_t)row * b : nullptr;
  {
    int tr = tie0, pos = pos0;
    for (int i = lo; i < hi; ++i) {
      if ((sloc[i >> 5] >> (i & 31)) & 1u) continue;
      const uint32_t key = __float_as_uint(s[i]);
      bool drop = key < v;
      if (key == v) drop = tr++ < need;
      if (drop) {
        if (pos < b) {
          dst[pos] = i;
          if (dst2) dst2[pos] = i;
        }
        ++pos;
      }
    }
  }
  if (t == 0 && total != b) atomicOr(err, GP_DEVERR_SHORT);
}

hipError_t launch_select(const Params& p, const WsLayout& w, int B, const int8_t* action,
                         void* ws, int32_t* dropped_out, int32_t* err, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  hipLaunchKernelGGL(k_select, dim3((unsigned)w.rows), dim3(kSel), 0, s, p.L, p.Hkv, p.b, p.R,
                     p.kloc, reinterpret_cast<const WsHeader*>(base + w.header),
                     reinterpret_cast<const int64_t*>(base + w.page_off), action,
                     reinterpret_cast<const float*>(base + w.imp),
                     reinterpret_cast<int32_t*>(base + w.dropped), dropped_out, err);
  (void)B;
  return hipGetLastError();
}

}  // namespace gp
