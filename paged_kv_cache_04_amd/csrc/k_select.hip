// A7 + A8: Compress & Hold selection per (layer, KV head) row.
// Citations are to "GrowPage: On-Demand KV Budgeting for Efficient LLM
// Reasoning Serving" (arXiv 2609.03494): §3.3 Eq. 9 (importance), Eq. 10
// (block-local plus global selection), window mask (§3.3, §5.1).
//
// A Shrink row (GrowPage-Shrink, App. H.1) drops 2b candidates instead of b
// (budget (P - 2) b - R); everything below holds with that drop count.
// Candidates C = [0, N - R): the R newest slots are always kept.  Order:
// larger importance first, equal importance the newer slot first.  With
// exactly b candidates to drop per row, the selection is computed from the
// bottom:
//   1. the b smallest candidates of C: a 3-digit radix select (11 + 10 + 10
//      bits) finds the value v of the b-th smallest; candidates below v are
//      dropped and of those equal to v the oldest until exactly b; dropped
//      slots written in ascending order.  A row of up to 32768 candidates
//      is read from HBM once into the workgroup's registers and its first
//      digit counted as it arrives; when the boundary bucket and the
//      buckets below hold few candidates those are listed once (slot and
//      key) and the later digits, the drops and the ties are taken from the
//      list (slot order from bitmaps).  Otherwise, and for longer rows, each
//      digit is a pass over the row's importance array in HBM and ranks in
//      slot order come from ballots over per-wave slot ranges;
//   2. if no block loses more than |B_j| - min(k_loc, |B_j|) candidates, no
//      protected (block top-k_loc) candidate was dropped and this is Eq. 10's
//      answer; otherwise each block's top-min(k_loc, |B_j|) is marked (one
//      wave per block, bit-serial threshold search with ballots, ties by
//      slot) and step 1 is repeated over the unmarked candidates.
// Importance values are non-negative fp32, so their bit patterns order like
// the values.
#include "gp_internal.h"

namespace gp {

constexpr int kSel = 512;
constexpr int kMaxRowTokens = 65536;
constexpr int kSelRegTokens = 32768;  // candidates a workgroup holds in registers
constexpr int kSelH1 = 2048;          // first radix digit: bits 30..20
constexpr int kSelH2 = 1024;          // second and third digits: 10 bits each
constexpr int kLoadU = 16;            // float4 row loads per thread, all in flight at once
constexpr int kSelList = 2048;        // candidates the list path keeps (slot and key)
constexpr int kBitWords = kSelRegTokens / 32;  // words of each list-path bitmap
static_assert(kSelRegTokens == 4 * kLoadU * kSel, "a register row is one round of float4 loads");
static_assert(kBitWords % kSel == 0, "whole bitmap words per thread");
static_assert(kSelH1 % kSel == 0 && kSelH2 % kSel == 0, "whole buckets per thread");

// One radix pass's search over the whole block: thread t holds buckets
// PER t .. PER t + PER - 1 of hcnt.  The digit is the smallest bucket whose
// count of smaller values (below, plus the buckets up to and including it)
// reaches nd; counts grow with the bucket, so one bucket has the crossing and
// the thread holding it writes the extended prefix and the count below it.
// (If no bucket reaches nd, the row has fewer than nd candidates; the top
// bucket is taken and the caller reports the short row.)  The bucket's own
// count goes to s_count.  Wave prefix sums by DPP, one barrier for the
// totals of the lower waves.
template <int PER>
__device__ __forceinline__ void block_select_digit(const uint32_t* hcnt, uint32_t below, int nd,
                                                   uint32_t prefix, int shift, uint32_t* s_wc,
                                                   uint32_t& s_prefix, uint32_t& s_below,
                                                   uint32_t& s_count) {
  constexpr int nb = PER * kSel;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  uint32_t c[PER], own = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    c[u] = hcnt[PER * t + u];
    own += c[u];
  }
  const uint32_t incl = wave_prefix_u32(own);
  if (lane == 63) s_wc[wv] = incl;
  __syncthreads();
  uint32_t cum = below + (incl - own);
  for (int u = 0; u < wv; ++u) cum += s_wc[u];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const uint32_t before = cum;
    cum += c[u];
    const int bkt = PER * t + u;
    if ((cum >= (uint32_t)nd && before < (uint32_t)nd) || (bkt == nb - 1 && cum < (uint32_t)nd)) {
      s_prefix = prefix | ((uint32_t)bkt << shift);
      s_below = before;
      s_count = c[u];
    }
  }
}

// Block-wide scalars of a row's selection (in LDS).
struct SelShared {
  uint32_t prefix, below, count;  // a digit search's result
  int listn;                      // boundary-bucket members collected so far
};

// Steps 2-3: the nd smallest candidates of [0, nc) (skipping those marked in
// the S_loc bitmap when PROT), written ascending to dst (and dst2); without
// PROT each dropped slot is also counted in blkcnt[its block].  Returns the
// number of candidates the threshold selects (nd unless the row is too short).
template <bool PROT>
__device__ __forceinline__ int drop_smallest(const float* __restrict__ s, int nc, int nd,
                                             const uint32_t* sloc, uint32_t* hcnt, int* scanbuf,
                                             SelShared& sh, int32_t* dst, int32_t* dst2,
                                             int* blkcnt) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  // step 2: value of the nd-th smallest unprotected candidate.  Three radix
  // digits: bits 30..20 (the exponent and three mantissa bits, so that the
  // buckets spread the values and the counting atomics rarely collide), then
  // bits 19..10 and 9..0.  The sign bit is 0 for every importance value.
  uint32_t prefix = 0, mask = 0, below = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
    const int nb = pass == 0 ? kSelH1 : kSelH2;
    for (int k = t; k < nb; k += kSel) hcnt[k] = 0;
    __syncthreads();
    for (int i = t; i < nc; i += kSel) {
      if (PROT && ((sloc[i >> 5] >> (i & 31)) & 1u)) continue;
      const uint32_t key = __float_as_uint(s[i]);
      if ((key & mask) == prefix) atomicAdd(&hcnt[(key >> shift) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    // the bucket where the count of smaller values reaches nd
    uint32_t* s_wc = reinterpret_cast<uint32_t*>(scanbuf);
    if (pass == 0)
      block_select_digit<kSelH1 / kSel>(hcnt, below, nd, prefix, shift, s_wc, sh.prefix,
                                        sh.below, sh.count);
    else
      block_select_digit<kSelH2 / kSel>(hcnt, below, nd, prefix, shift, s_wc, sh.prefix,
                                        sh.below, sh.count);
    __syncthreads();
    prefix = sh.prefix;
    below = sh.below;
    mask |= (uint32_t)(nb - 1) << shift;
    __syncthreads();
  }
  const uint32_t v = prefix;
  const int need = nd - (int)below;

  // step 3: ties at v go oldest first; dropped slots are written in
  // ascending order.  Each wave walks one contiguous range of slots, 64 at a
  // time (one per lane, so the row is read in whole 256-byte lines); ranks in
  // slot order come from ballots within a wave and, across waves, from the
  // counts of the waves before it.
  constexpr int kW = kSel / 64;
  const int span = (nc + kW * 64 - 1) / (kW * 64) * 64;  // slots per wave
  const int w0 = wv * span;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;  // lanes below this one
  auto cand = [&](int i, uint32_t& key) -> bool {
    if (i >= nc || (PROT && ((sloc[i >> 5] >> (i & 31)) & 1u))) return false;
    key = __float_as_uint(s[i]);
    return true;
  };
  {
    int nt = 0, nl = 0;
    for (int j = 0; j < span; j += 64) {
      uint32_t key = 0;
      const bool ok = cand(w0 + j + lane, key);
      nt += __popcll(__ballot(ok && key == v));
      nl += __popcll(__ballot(ok && key < v));
    }
    if (lane == 0) {
      scanbuf[wv] = nt;
      scanbuf[kW + wv] = nl;
    }
  }
  __syncthreads();
  // ties and drops of the waves before this one; the row's total drops
  int tr = 0, pos = 0, tb = 0, db = 0;
  for (int u = 0; u < kW; ++u) {
    if (u == wv) {
      tr = tb;
      pos = db;
    }
    const int tu = scanbuf[u];
    int take = need - tb;
    take = take < 0 ? 0 : (take > tu ? tu : take);
    db += scanbuf[kW + u] + take;
    tb += tu;
  }
  for (int j = 0; j < span; j += 64) {
    const int i = w0 + j + lane;
    uint32_t key = 0;
    const bool ok = cand(i, key);
    const bool tie = ok && key == v;
    const uint64_t tm = __ballot(tie);
    const bool drop = (ok && key < v) || (tie && tr + __popcll(tm & lt) < need);
    const uint64_t dm = __ballot(drop);
    const int p = pos + __popcll(dm & lt);
    if (drop && p < nd) {
      dst[p] = i;
      if (dst2) dst2[p] = i;
    }
    // a 64-slot step lies in one page: one count per step and wave
    if (!PROT && lane == 0 && dm != 0) {
      const int room = nd - pos;  // drops of this step that are written
      const int cnt = __popcll(dm);
      if (room > 0) atomicAdd(&blkcnt[(w0 + j) >> 8], cnt < room ? cnt : room);
    }
    tr += __popcll(tm);
    pos += __popcll(dm);
  }
  return db;
}

// Step 1: S_loc of every block as a bitmap.
__device__ __forceinline__ void protect_blocks(const float* __restrict__ s, int P, int nc,
                                               int kloc, uint32_t* sloc) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  (void)t;
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

}

// Steps 2-3 for a row held in registers (vr: thread t holds candidates
// 4 q .. 4 q + 3 for q = t + kSel u in vr[u]) whose first-digit histogram
// (hcnt: min(key >> 20, 2047), bits 30..20 of every finite candidate) was
// counted as the row arrived, when the boundary bucket d1 < 2047 and the
// buckets below it hold at most kSelList candidates together.  Instead of
// further passes over the whole row: one pass over the registers (each wave
// takes every kSel/64-th 256-slot group, 4 slots per lane) lists the slots
// and keys of the candidates below the top of the boundary bucket (the sure
// drops below it and the bucket's members), counting the members' second
// digit; the second and third digits are resolved on the list alone; the
// listed candidates below the final value v are marked in the drop bitmap
// dbits, those equal to v in the tie bitmap tbits (bit i & 31 of word i >> 5
// for slot i).  The drops are then the bits of dbits plus the `need` lowest
// bits of tbits (ties oldest first), numbered in slot order by one
// block-wide prefix sum over the words (kBitWords / kSel consecutive words
// per thread) and written ascending.  Returns the number of candidates
// selected.  Expects dbits, tbits (kBitWords words each), hist2 and sh.listn
// zeroed.
__device__ __forceinline__ int drop_smallest_reg(const float4* vr, int nc, int nd,
                                                 uint32_t* hcnt, uint32_t* hist2, int* lslot,
                                                 uint32_t* lkey, uint32_t* dbits,
                                                 uint32_t* tbits, int* scanbuf, SelShared& sh,
                                                 uint32_t d1, uint32_t below1, int nl,
                                                 int32_t* dst, int32_t* dst2, int* blkcnt) {
  const int t = threadIdx.x, lane = t & 63;
  // the wave index in a scalar register, so that the group bounds below are
  // wave-uniform branches
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  uint32_t* s_wc = reinterpret_cast<uint32_t*>(scanbuf);
  constexpr int kW = kSel / 64;
  // first digit below d1: keys below a1; the bucket's members: [a1, a2)
  const uint32_t a1 = d1 << 20, a2 = a1 + (1u << 20);
  for (int k = t; k < kSelH2; k += kSel) hcnt[k] = 0;  // the third digit's histogram
  // the keys of group u (slots g0 .. g0 + 255, g0 = 4 kSel u + 256 wv, lane
  // l at 4 l within it); slots past the row get a key above every bucket
  auto group_keys = [&](int u, int g0, uint32_t (&key)[4]) {
    key[0] = __float_as_uint(vr[u].x);
    key[1] = __float_as_uint(vr[u].y);
    key[2] = __float_as_uint(vr[u].z);
    key[3] = __float_as_uint(vr[u].w);
    if (g0 + 256 > nc) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (g0 + 4 * lane + c >= nc) key[c] = 0xffffffffu;
    }
  };
  // this wave's list entries, then its place in the list by one atomic
  int nw = 0;
#pragma unroll
  for (int u = 0; u < kLoadU; ++u) {
    const int g0 = 4 * kSel * u + 256 * wv;
    if (g0 >= nc) break;
    uint32_t key[4];
    group_keys(u, g0, key);
#pragma unroll
    for (int c = 0; c < 4; ++c) nw += __popcll(__ballot(key[c] < a2));
  }
  int base = 0;
  if (nw != 0) {
    if (lane == 0) base = atomicAdd(&sh.listn, nw);
    base = __builtin_amdgcn_readfirstlane(base);
  }
#pragma unroll
  for (int u = 0; u < kLoadU; ++u) {
    const int g0 = 4 * kSel * u + 256 * wv;
    if (g0 >= nc) break;
    uint32_t key[4];
    group_keys(u, g0, key);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint64_t le = __ballot(key[c] < a2);
      if (le != 0) {
        if (key[c] < a2) {
          const int k = base + (int)__builtin_amdgcn_mbcnt_hi(
                                   (uint32_t)(le >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)le, 0u));
          lslot[k] = g0 + 4 * lane + c;
          lkey[k] = key[c];
          if (key[c] >= a1) atomicAdd(&hist2[(key[c] >> 10) & (uint32_t)(kSelH2 - 1)], 1u);
        }
        base += __popcll(le);
      }
    }
  }
  __syncthreads();
  block_select_digit<kSelH2 / kSel>(hist2, below1, nd, a1, 10, s_wc, sh.prefix, sh.below,
                                    sh.count);
  __syncthreads();
  const uint32_t p2 = sh.prefix, below2 = sh.below;
  const uint32_t d2 = (p2 >> 10) & (uint32_t)(kSelH2 - 1);
  for (int k = t; k < nl; k += kSel) {
    const int i = lslot[k];
    const uint32_t key = lkey[k];
    const uint32_t dg = (key >> 10) & (uint32_t)(kSelH2 - 1);
    if (key < a1 || dg < d2)
      atomicOr(&dbits[i >> 5], 1u << (i & 31));
    else if (dg == d2)
      atomicAdd(&hcnt[key & (uint32_t)(kSelH2 - 1)], 1u);
  }
  __syncthreads();
  block_select_digit<kSelH2 / kSel>(hcnt, below2, nd, p2, 0, s_wc, sh.prefix, sh.below, sh.count);
  __syncthreads();
  const uint32_t v = sh.prefix;
  const int need = nd - (int)sh.below;
  for (int k = t; k < nl; k += kSel) {
    const int i = lslot[k];
    const uint32_t key = lkey[k];
    if ((key >> 10) == (v >> 10) && key <= v)
      atomicOr(key < v ? &dbits[i >> 5] : &tbits[i >> 5], 1u << (i & 31));
  }
  __syncthreads();
  // words kWp t .. kWp t + kWp - 1 (slots 32 kWp t onwards, in slot order);
  // one packed prefix sum gives the ties (high half) and the drops below v
  // (low half, <= nd) of the words before this thread's
  constexpr int kWp = kBitWords / kSel;
  uint32_t dw[kWp], tw[kWp];
  uint32_t nt_all = 0, nl_all = 0;
#pragma unroll
  for (int j = 0; j < kWp; ++j) {
    dw[j] = dbits[kWp * t + j];
    tw[j] = tbits[kWp * t + j];
    nt_all += __popc(tw[j]);
    nl_all += __popc(dw[j]);
  }
  uint32_t tot;
  const uint32_t ex = block_prefix_excl_u32((nt_all << 16) | nl_all, s_wc, kW, tot);
  int ties_before = (int)(ex >> 16);
  int pos = (int)(ex & 0xffffu) + (ties_before < need ? ties_before : (need > 0 ? need : 0));
#pragma unroll
  for (int j = 0; j < kWp; ++j) {
    const int nt = __popc(tw[j]);
    int take = need - ties_before;
    take = take < 0 ? 0 : (take > nt ? nt : take);
    uint32_t d = dw[j];
    for (uint32_t x = tw[j]; take > 0; --take) {  // the oldest ties of this word
      d |= x & (0u - x);
      x &= x - 1;
    }
    ties_before += nt;
    const int w = kWp * t + j;
    if (d != 0) {
      const int cnt = __popc(d), room = nd - pos;
      if (room > 0) atomicAdd(&blkcnt[w >> 3], cnt < room ? cnt : room);  // 8 words per page
      for (uint32_t x = d; x != 0; x &= x - 1, ++pos) {
        if (pos >= nd) continue;
        const int i = 32 * w + __builtin_ctz(x);
        dst[pos] = i;
        if (dst2) dst2[pos] = i;
      }
    }
  }
  const int all_ties = (int)(tot >> 16);
  return (int)(tot & 0xffffu) + (all_ties < need ? all_ties : (need > 0 ? need : 0));
}

// One row whose importance values are at s (global memory).  The
// b smallest candidates are found first without the block quotas; they are
// the answer unless some block would lose more than |B_j| - min(k_loc,
// |B_j|) of its candidates (then one of them is in that block's protected
// top), in which case the quotas are computed and the selection repeated
// over the unprotected candidates.  (The nd smallest of C avoid S_loc, so
// they are also the nd smallest of C minus S_loc.)  With vr the row is
// also in registers with its first-digit histogram counted and the bitmaps,
// hist2 and sh.listn zeroed: the first selection then takes the list path
// when the boundary bucket allows it.
__device__ __forceinline__ void select_row(const float* __restrict__ s, const float4* vr, int P,
                                           int nc, int nd, int kloc, uint32_t* sloc,
                                           uint32_t* hcnt, uint32_t* hist2, int* lslot,
                                           uint32_t* lkey, int* scanbuf, int* blkcnt,
                                           SelShared& sh, int32_t* dst, int32_t* dst2,
                                           int32_t* err) {
  const int t = threadIdx.x;
  for (int j = t; j < P; j += kSel) blkcnt[j] = 0;
  bool listed = false;
  if (vr) {
    block_select_digit<kSelH1 / kSel>(hcnt, 0, nd, 0, 20, reinterpret_cast<uint32_t*>(scanbuf),
                                      sh.prefix, sh.below, sh.count);
    __syncthreads();
    listed = sh.below + sh.count <= (uint32_t)kSelList &&
             (sh.prefix >> 20) < (uint32_t)(kSelH1 - 1);
  } else {
    __syncthreads();
  }
  int total;
  if (listed) {
    // the drop and tie bitmaps share the S_loc area (nc <= kSelRegTokens:
    // kBitWords words each)
    total = drop_smallest_reg(vr, nc, nd, hcnt, hist2, lslot, lkey, sloc, sloc + kBitWords,
                              scanbuf, sh, sh.prefix >> 20, sh.below,
                              (int)(sh.below + sh.count), dst, dst2, blkcnt);
  } else {
    total = drop_smallest<false>(s, nc, nd, sloc, hcnt, scanbuf, sh, dst, dst2, blkcnt);
  }
  __syncthreads();
  int over = 0;
  if (kloc > 0)
    for (int j = t; j < P; j += kSel) {
      const int nb = nc - j * kPage < kPage ? nc - j * kPage : kPage;
      const int keep_min = kloc < nb ? kloc : nb;
      over |= blkcnt[j] > nb - keep_min;
    }
  if (__syncthreads_or(over)) {
    protect_blocks(s, P, nc, kloc, sloc);
    __syncthreads();
    total = drop_smallest<true>(s, nc, nd, sloc, hcnt, scanbuf, sh, dst, dst2, nullptr);
  }
  if (t == 0 && total != nd) atomicOr(err, GP_DEVERR_SHORT);
}

// One 512-thread workgroup per row; two fit per CU (registers), so one
// row's load is in flight while the other row is selected.
__global__ __launch_bounds__(kSel, 2) void k_select(int L, int Hkv, int b, int R, int kloc,
                                                    int stride,
                                                    const WsHeader* __restrict__ hdr,
                                                    const int64_t* __restrict__ page_off,
                                                    const int8_t* __restrict__ action,
                                                    const float* __restrict__ imp,
                                                    int32_t* __restrict__ dropped,
                                                    int32_t* __restrict__ dropped_out,
                                                    const int32_t* __restrict__ req_flags,
                                                    int32_t* __restrict__ item_counter,
                                                    int32_t* __restrict__ err) {
  __shared__ uint32_t sloc[kMaxRowTokens / 32];
  __shared__ uint32_t hcnt[kSelH1];
  __shared__ uint32_t hist2[kSelH2];
  __shared__ int lslot[kSelList];
  __shared__ uint32_t lkey[kSelList];
  __shared__ int scanbuf[2 * (kSel / 64)];
  __shared__ int blkcnt[kMaxRowTokens / kPage];
  __shared__ SelShared sh;
  const int LH = L * Hkv;
  const int row = blockIdx.x;
  const int r = row / LH, lh = row % LH;
  // the compaction that follows takes its items from this counter
  if (row == 0 && threadIdx.x == 0) item_counter[0] = 0;
  // the row's metadata in one round of loads (all inside the workspace and
  // the caller's arrays whatever the batch), looked at after validity
  const int valid = hdr->valid;
  const int8_t act = action ? action[r] : (int8_t)GP_COMPRESS;
  const int64_t off0 = page_off[r], off1 = page_off[r + 1];
  const int32_t flags = req_flags[r];
  if (!valid) return;
  if (act != GP_COMPRESS && act != GP_SHRINK) return;
  if (act == GP_SHRINK && stride < 2 * b) return;  // Shrink outside its policy: ignored
  const int m = act == GP_SHRINK ? 2 : 1;  // pages of slots to free
  const int64_t P = off1 - off0;
  const int t = threadIdx.x;
  if (flags & kReqTooLong) {  // longer than the selection takes: left as it is
    if (t == 0 && lh == 0) atomicOr(err, GP_DEVERR_LONG);
    return;
  }
  if (P < m + 1) {
    if (t == 0) atomicOr(err, GP_DEVERR_SHORT);
    return;
  }
  if (flags & kReqBlocked) return;  // left uncompressed (App. E.2 page shortage)
  const int N = (int)(P * b), nc = N - R;
  const float* __restrict__ s = imp + (int64_t)LH * off0 * b + (int64_t)lh * N;
  int32_t* dst = dropped + (int64_t)row * stride;
  int32_t* dst2 = dropped_out ? dropped_out + (int64_t)row * stride : nullptr;
  const int nd = m * b;  // candidates to drop
  if (nc <= kSelRegTokens) {
    // the row's candidates are read from HBM once, all loads in flight
    // before any is used (thread t: candidates 4 q .. 4 q + 3, q = t + kSel
    // u, in v[u]), the first radix digit (min(key >> 20, 2047)) counted as
    // they arrive
    const int n4 = (nc + 3) / 4;  // rows start 1 KiB aligned; N is a multiple of 256
    const float4* s4 = reinterpret_cast<const float4*>(s);
    float4 v[kLoadU];
#pragma unroll
    for (int u = 0; u < kLoadU; ++u) {  // quads past the row read its first one (n4 >= 1)
      const int q = t + u * kSel;
      v[u] = s4[q < n4 ? q : 0];
    }
    for (int k = t; k < kSelH1; k += kSel) hcnt[k] = 0;
    for (int k = t; k < kSelH2; k += kSel) hist2[k] = 0;
    for (int k = t; k < 2 * kBitWords; k += kSel) sloc[k] = 0;
    if (t == 0) sh.listn = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kLoadU; ++u) {
      const int q = t + u * kSel;
      if (q < n4) {
        const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (4 * q + c < nc) atomicAdd(&hcnt[min(__float_as_uint(e[c]) >> 20, kSelH1 - 1u)], 1u);
      }
    }
    __syncthreads();
    select_row(s, v, (int)P, nc, nd, kloc, sloc, hcnt, hist2, lslot, lkey, scanbuf, blkcnt, sh,
               dst, dst2, err);
  } else {
    select_row(s, nullptr, (int)P, nc, nd, kloc, sloc, hcnt, hist2, lslot, lkey, scanbuf, blkcnt,
               sh, dst, dst2, err);
  }
}

hipError_t launch_select(const Params& p, const WsLayout& w, int B, const int8_t* action,
                         void* ws, int32_t* dropped_out, int32_t* err, int num_cus,
                         hipStream_t s) {
  char* base = static_cast<char*>(ws);
  (void)num_cus;
  hipLaunchKernelGGL(k_select, dim3((unsigned)w.rows), dim3(kSel), 0, s, p.L, p.Hkv, p.b, p.R,
                     p.kloc, p.b * p.max_freed(),
                     reinterpret_cast<const WsHeader*>(base + w.header),
                     reinterpret_cast<const int64_t*>(base + w.page_off), action,
                     reinterpret_cast<const float*>(base + w.imp),
                     reinterpret_cast<int32_t*>(base + w.dropped), dropped_out,
                     reinterpret_cast<const int32_t*>(base + w.req_flags),
                     &reinterpret_cast<WsHeader*>(base + w.header)->item_counter, err);
  (void)B;
  return hipGetLastError();
}

}  // namespace gp
