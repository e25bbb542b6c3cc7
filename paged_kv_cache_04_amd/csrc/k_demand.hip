// A2-A4 fused per row: score every cached key of a (layer, KV head) row
// against its 8 calibrated summary queries, form the attention distributions,
// the per-token importance and the p-coverage demand of both views.
// Citations are to "GrowPage: On-Demand KV Budgeting for Efficient LLM
// Reasoning Serving" (arXiv 2609.03494): §3.1 Eq. 2, §3.2 Eq. 7, §3.3 Eq. 9,
// App. E.1 ("Demand estimation at capacity boundaries").
//
// Persistent kernel, kDemandBlocksPerCU workgroups of 16 / kDemandBlocksPerCU
// waves per CU (one 16-wave workgroup by default: two 8-wave workgroups, one
// streaming keys while the other works on its row's distributions, measured
// no faster).  Workgroups pull rows from a queue ordered longest request
// first.  Per row:
//  1. score: each wave takes every 16th 64-key tile of the row and pipelines
//     it in two halves (key elements 0-63, then 64-127): while it multiplies
//     one half from its private LDS stage (half rows padded to 144 B so the
//     lanes' 16-byte row reads hit distinct banks), the 8 coalesced 16-byte
//     loads of the next half are in flight into registers.  Each lane scores
//     one key with 8 serial fmaf chains over j = 0..127 in index order (the
//     fp32 contract shared with the CPU reference); the summary values come
//     by scalar loads, one quad of 4 elements x 8 queries at a time, requested
//     a quad ahead.  The 8 logits per key go to the workgroup's own logits
//     ring, which it overwrites row after row, so they are read back from
//     cache instead of making a round trip through HBM;
//  2. maxima over C_t = [0, N - b) and over all slots; exact normalisers
//     Z = sum floor(exp(l - m) * 2^40) (uint64, order-free);
//  3. a = exp(l - m) * (1 / Z), GQA mean of the 4 heads of each view, for C_t
//     and for all slots; s = max of the full-cache means (Eq. 9) to the
//     importance array; demand means to the key ring; first radix digit
//     (bits 30..20 of the fp32 pattern: exponent and 3 mantissa bits) of each
//     view histogrammed in LDS with counts and masses floor(abar * 2^40);
//  4. D_p per view: the bucket where the descending prefix mass reaches p,
//     then the remaining 20 bits resolved on that bucket's members only
//     (collected into LDS, or scanned in the key ring when too many; both
//     views in the same two passes), then
//     D_p = (count above) + ceil(remaining mass / member mass).  Each digit
//     is found by one block-wide suffix-sum search over its buckets.
#include "gp_internal.h"

namespace gp {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDW = 16 / kDemandBlocksPerCU;  // waves per workgroup
constexpr int kDT = kDW * 64;                 // threads
constexpr int kHalfPad = 144;                 // bytes per staged half row
constexpr int kWaveStage = 64 * kHalfPad;     // bytes per wave
constexpr int kLdsBytes = kDW * kWaveStage;   // 147456, reused after scoring
constexpr int kH1 = 2048;                     // first-digit buckets
constexpr int kH2 = 1024;                     // second/third-digit buckets
constexpr int kListCap = (kLdsBytes - 2 * kH1 * 8 - 2 * kH2 * 12) / 4;  // boundary members in LDS
constexpr int kRingU = 8;  // demand-key ring loads in flight per thread in phase 4
constexpr int kListHalf = kListCap / 2;                            // per view

// acc[qi] += q[qi][e] * k[e] for e = 0..3 in order (4 bf16 keys in k).
__device__ __forceinline__ void fma_quad(float* acc, const float* q, u32x2 k) {
  const float k0 = bf16_lo(k.x), k1 = bf16_hi(k.x), k2 = bf16_lo(k.y), k3 = bf16_hi(k.y);
#pragma unroll
  for (int qi = 0; qi < kNQ; ++qi) acc[qi] = __builtin_fmaf(q[qi * 4 + 0], k0, acc[qi]);
#pragma unroll
  for (int qi = 0; qi < kNQ; ++qi) acc[qi] = __builtin_fmaf(q[qi * 4 + 1], k1, acc[qi]);
#pragma unroll
  for (int qi = 0; qi < kNQ; ++qi) acc[qi] = __builtin_fmaf(q[qi * 4 + 2], k2, acc[qi]);
#pragma unroll
  for (int qi = 0; qi < kNQ; ++qi) acc[qi] = __builtin_fmaf(q[qi * 4 + 3], k3, acc[qi]);
}

__device__ __forceinline__ void wave_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t shfl_down_u64(uint64_t v, int off) {
  const unsigned lo = __shfl_down((unsigned)v, off);
  const unsigned hi = __shfl_down((unsigned)(v >> 32), off);
  return ((uint64_t)hi << 32) | lo;
}

// 16 values per lane summed over the wave, transposed: each exchange halves
// the values a lane carries.  Lane L ends with the totals of values
// 8 b5 + 4 b4 + j (j = 0..3) in out[j], b5 and b4 being bits 5 and 4 of L.
__device__ __forceinline__ void wave_sum16_u64(const uint64_t (&v)[16], uint64_t (&out)[4]) {
  uint64_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = swap32_add(v[i], v[i + 8]);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = row_sum_u64(swap16_add(h[i], h[i + 4]));
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  return pk64(__builtin_amdgcn_readlane((uint32_t)v, lane),
              __builtin_amdgcn_readlane((uint32_t)(v >> 32), lane));
}

// Inclusive suffix sums over a wave: lane L gets the sum over lanes L..63.
// DPP row shifts (lane i reads lane i + n of its 16-lane row, 0 past the
// row's end) give the sums within each row; then each row adds the totals of
// the rows above it, read from their first lanes.
__device__ __forceinline__ uint64_t wave_suffix_u64(uint64_t v) {
  v += dpp_u64<0x101>(v);
  v += dpp_u64<0x102>(v);
  v += dpp_u64<0x104>(v);
  v += dpp_u64<0x108>(v);
  const int row = (threadIdx.x & 63) >> 4;
  const uint64_t r1 = readlane_u64(v, 16), r2 = readlane_u64(v, 32), r3 = readlane_u64(v, 48);
  return v + (row < 1 ? r1 : 0) + (row < 2 ? r2 : 0) + (row < 3 ? r3 : 0);
}

__device__ __forceinline__ uint32_t wave_suffix_u32(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x101, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0u, v, 0x102, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0u, v, 0x104, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0u, v, 0x108, 0xf, 0xf, false);
  const int row = (threadIdx.x & 63) >> 4;
  const uint32_t r1 = __builtin_amdgcn_readlane(v, 16), r2 = __builtin_amdgcn_readlane(v, 32),
                 r3 = __builtin_amdgcn_readlane(v, 48);
  return v + (row < 1 ? r1 : 0u) + (row < 2 ? r2 : 0u) + (row < 3 ? r3 : 0u);
}

// Radix-digit searches of phase 4, both views at once over the whole block:
// threads 512 x .. 512 x + 511 (waves 8 x .. 8 x + 7) take view x, each a run
// of consecutive buckets.  A view's digit is the largest bucket d with
// p_den * (mass above the bucket's prefix + mass of buckets >= d) >= target;
// the mass is non-increasing in d, so exactly one bucket satisfies that and
// has the next bucket up failing it (or is the top bucket), and the thread
// holding it writes the digit and the mass (and count) above it.  Wave
// suffix sums by DPP, one barrier to add the totals of the higher waves.
static_assert(kDT == 1024, "the digit searches split the block into two views of 512 threads");

// First digit: 2048 fp64 bucket masses per view (integer-valued), 4 per thread.
__device__ __forceinline__ void block_first_digit(const double* h1m, const uint64_t* s_W,
                                                  uint32_t p_num, uint32_t p_den,
                                                  uint64_t* s_wm, int* s_dig, uint64_t* s_mab) {
  static_assert(kH1 == 4 * 512, "4 buckets per thread");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, x = t >> 9, j = t & 511;
  const double* hm = h1m + x * kH1 + 4 * j;
  uint64_t m[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) m[u] = (uint64_t)hm[u];
  const uint64_t own = m[0] + m[1] + m[2] + m[3];
  const uint64_t suf = wave_suffix_u64(own);
  if (lane == 0) s_wm[w] = suf;
  __syncthreads();
  uint64_t cum = suf - own;  // mass of the buckets above this thread's run
  // the totals of the view's higher waves: all 8 read at once, summed by rank
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint64_t v = s_wm[8 * x + k];
    cum += 8 * x + k > w ? v : 0;
  }
  const uint64_t target = s_W[x] * (uint64_t)p_num;
#pragma unroll
  for (int u = 3; u >= 0; --u) {
    const uint64_t above = cum;
    cum += m[u];
    const int b = 4 * j + u;
    if (cum * p_den >= target && (b == kH1 - 1 || above * p_den < target)) {
      s_dig[x] = b;
      s_mab[x] = above;
    }
  }
}

// Later digits: 1024 buckets of (count, mass) per view, 2 per thread; the
// mass and count above the bucket's prefix come in s_mab / s_cab and leave
// updated to the new digit.
__device__ __forceinline__ void block_next_digit(const uint32_t* h2c, const uint64_t* h2m,
                                                 const uint64_t* s_W, uint32_t p_num,
                                                 uint32_t p_den, uint64_t* s_wm, uint32_t* s_wc,
                                                 int* s_dig, uint64_t* s_mab, uint32_t* s_cab) {
  static_assert(kH2 == 2 * 512, "2 buckets per thread");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, x = t >> 9, j = t & 511;
  const uint64_t mab0 = s_mab[x];
  const uint32_t cab0 = s_cab[x];
  uint64_t m[2];
  uint32_t c[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    m[u] = h2m[x * kH2 + 2 * j + u];
    c[u] = h2c[x * kH2 + 2 * j + u];
  }
  const uint64_t own_m = m[0] + m[1];
  const uint32_t own_c = c[0] + c[1];
  const uint64_t suf_m = wave_suffix_u64(own_m);
  const uint32_t suf_c = wave_suffix_u32(own_c);
  if (lane == 0) {
    s_wm[w] = suf_m;
    s_wc[w] = suf_c;
  }
  __syncthreads();
  uint64_t cm = mab0 + (suf_m - own_m);
  uint32_t cc = cab0 + (suf_c - own_c);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint64_t vm = s_wm[8 * x + k];
    const uint32_t vc = s_wc[8 * x + k];
    const bool higher = 8 * x + k > w;
    cm += higher ? vm : 0;
    cc += higher ? vc : 0u;
  }
  const uint64_t target = s_W[x] * (uint64_t)p_num;
#pragma unroll
  for (int u = 1; u >= 0; --u) {
    const uint64_t am = cm;
    const uint32_t ac = cc;
    cm += m[u];
    cc += c[u];
    const int b = 2 * j + u;
    if (cm * p_den >= target && (b == kH2 - 1 || am * p_den < target)) {
      s_dig[x] = b;
      s_mab[x] = am;
      s_cab[x] = ac;
    }
  }
}

__device__ __forceinline__ float uniform_f(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// floor(v * 2^40) as an integer-valued float: exact, since below 2^23 floorf
// is exact and from 2^23 on every fp32 value is an integer (v <= 1).
__device__ __forceinline__ float mass40(float v) { return __builtin_floorf(v * kFix); }


// The logits ring holds, per 64-key tile, the first four logits of its keys
// and then the last four ([tile][2][64][4] floats), so that each store
// instruction of the scoring loop writes 1 KiB contiguously.
__device__ __forceinline__ void load_logits8(const float* lg, int64_t i, float (&lv)[kNQ]) {
  const float4* lp = reinterpret_cast<const float4*>(lg + (i >> 6) * (64 * kNQ)) + (i & 63);
  const float4 x0 = lp[0], x1 = lp[64];
  lv[0] = x0.x; lv[1] = x0.y; lv[2] = x0.z; lv[3] = x0.w;
  lv[4] = x1.x; lv[5] = x1.y; lv[6] = x1.z; lv[7] = x1.w;
}


// Compile-time tags for the token loops of phases 2 and 3: when every
// query's maximum over C_t equals its maximum over all slots (the usual
// case) the demand and full-cache exponentials coincide and the loop body is
// one block of 8 independent exponentials, with no per-query branch.
struct AllSame {
  static constexpr bool value = true;
};
struct SomeDiffer {
  static constexpr bool value = false;
};

struct DemandArgs {
  const uint16_t* k_pool;
  int pool_pages;
  const int32_t* block_table;
  int max_pages;
  int L, Hkv, B, b, p_num, p_den;
  const WsHeader* hdr;
  const int64_t* page_off;
  const int32_t* req_order;
  int32_t* row_counter;
  const float* qhat;
  float* ring_logits;   // [blocks][ring_tokens / 64][2][64][4]
  float* ring_keys;     // [blocks][ring_tokens][2]
  int64_t ring_tokens;
  float* imp;
  int32_t* k_short;
  int32_t* k_long;
  float* abar;
  int32_t* err;
};

__global__ __launch_bounds__(kDT) void k_demand(DemandArgs a, const float* __restrict__ qhat,
                                               const uint16_t* __restrict__ k_pool,
                                               const int32_t* __restrict__ block_table) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  __shared__ float s_wmax[kDW][2][kNQ];
  __shared__ float s_m[2][kNQ];
  __shared__ float s_rho[2][kNQ];
  __shared__ uint64_t s_red[kDW][2 * kNQ];
  __shared__ uint64_t s_W[2];
  __shared__ int s_item;
  __shared__ int s_list_n[2];
  __shared__ int s_dig[2];
  __shared__ uint64_t s_mab[2];
  __shared__ uint32_t s_cab[2];  // slots above the boundary so far, per view
  __shared__ uint64_t s_wm[kDW];  // per-wave suffix totals of the digit searches
  __shared__ uint32_t s_wc[kDW];
  if (!a.hdr->valid) return;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int LH = a.L * a.Hkv;
  const int n_items = a.B * LH;  // <= 1024 requests x (L * Hkv) rows
  float* lg = a.ring_logits + (int64_t)blockIdx.x * a.ring_tokens * kNQ;
  float* rk = a.ring_keys + (int64_t)blockIdx.x * a.ring_tokens * 2;
  unsigned char* my = lds + w * kWaveStage;
  // LDS views used after scoring
  double* h1m = reinterpret_cast<double*>(lds);                              // [2][kH1]
  uint32_t* h2c = reinterpret_cast<uint32_t*>(lds + 2 * kH1 * 8);                // [2][kH2]
  uint64_t* h2m = reinterpret_cast<uint64_t*>(lds + 2 * kH1 * 8 + 2 * kH2 * 4);  // [2][kH2]
  uint32_t* list = reinterpret_cast<uint32_t*>(lds + 2 * kH1 * 8 + 2 * kH2 * 12);  // [kListCap]

  while (true) {
    if (t == 0) s_item = atomicAdd(a.row_counter, 1);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    if (item >= n_items) break;
    const int r = __builtin_amdgcn_readfirstlane(a.req_order[item / LH]);
    const int lh = __builtin_amdgcn_readfirstlane(item % LH);
    const int row = __builtin_amdgcn_readfirstlane(r * LH + lh);
    const int l = __builtin_amdgcn_readfirstlane(lh / a.Hkv);
    const int h = __builtin_amdgcn_readfirstlane(lh % a.Hkv);
    // row sizes are block-uniform; read them into scalar registers so every
    // branch and loop bound around the barriers below is a scalar branch
    const int64_t P = __builtin_amdgcn_readfirstlane((int)(a.page_off[r + 1] - a.page_off[r]));
    const int64_t N = P * kPage, ndem = N - kPage;
    const int64_t row_tok = (int64_t)LH * a.page_off[r] * kPage + (int64_t)lh * N;
    const float* __restrict__ qv = qhat + (int64_t)row * (kNQ * kD);

    // ---- 1. score -------------------------------------------------------------
    // A tile's 8 logits per key are stored one tile late, right after the
    // loads of the next half are issued, so that no wait for key loads ever
    // covers a ring store (vector loads and stores share one in-order
    // counter).  A key of the newest page belongs to a wave's last tile, so
    // the maxima over C_t run over the earlier tiles and the last one is
    // sorted after the loop.
    float md[kNQ], ml[kNQ];
#pragma unroll
    for (int q = 0; q < kNQ; ++q) md[q] = ml[q] = -INFINITY;
    const int n_tiles = (int)(4 * P);
    if (w < n_tiles) {
      const int32_t* __restrict__ bt_row = block_table + (int64_t)r * a.max_pages;
      // lane part of a key load: key lane >> 3 of each group of 8, 16 bytes
      // (lane & 7) of its half row
      const uint32_t lane_off = (uint32_t)((lane >> 3) * 256 + (lane & 7) * 16);
      auto tile_base = [&](int tt, int page, bool& bad) -> const unsigned char* {
        bad = page < 0 || page >= a.pool_pages;
        return reinterpret_cast<const unsigned char*>(
            k_pool + ((((int64_t)l * a.pool_pages + (bad ? 0 : page)) * a.Hkv + h) * kPage +
                        (tt & 3) * 64) * kD);
      };
      auto issue = [&](const unsigned char* base, int half, u32x4* v) {
        const unsigned char* p = base + lane_off + half * 128;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + i * 2048));
      };
      int tt = w;
      bool bad;
      const unsigned char* src = tile_base(tt, bt_row[tt >> 2], bad);
      u32x4 v[8];
      issue(src, 0, v);
      float pacc[kNQ];  // logits of the previous tile, stored during this one
#pragma unroll
      for (int qi = 0; qi < kNQ; ++qi) pacc[qi] = 0.0f;
      int ptile = tt;  // the first round stores zeros into its own tile's slot
      while (true) {
        const int tcur = tt;
        const bool cur_bad = bad;
        const unsigned char* cur_src = src;
        const bool has_next = tt + kDW < n_tiles;
        const int next_page = has_next ? bt_row[(tt + kDW) >> 2] : 0;
        float acc[kNQ];
#pragma unroll
        for (int qi = 0; qi < kNQ; ++qi) acc[qi] = 0.0f;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int key = i * 8 + (lane >> 3);
            *reinterpret_cast<u32x4*>(my + key * kHalfPad + (lane & 7) * 16) = v[i];
          }
          wave_order();
          if (half == 0) {
            issue(cur_src, 1, v);
            float4* out = reinterpret_cast<float4*>(lg + (int64_t)ptile * (64 * kNQ)) + lane;
            out[0] = make_float4(pacc[0], pacc[1], pacc[2], pacc[3]);
            out[64] = make_float4(pacc[4], pacc[5], pacc[6], pacc[7]);
          } else if (has_next) {
            tt += kDW;
            src = tile_base(tt, next_page, bad);
            issue(src, 0, v);
          }
          if (!cur_bad) {
            const unsigned char* rowp = my + lane * kHalfPad;
            const float* qh = qv + half * 16 * 32;
            float qa[32], qb[32];
            u32x4 kc, kn;
#pragma unroll
            for (int i = 0; i < 32; ++i) qa[i] = qh[i];
            kc = *reinterpret_cast<const u32x4*>(rowp);
#pragma unroll
            for (int ch = 0; ch < 8; ++ch) {
              __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): quad 2ch and chunk ch ready
#pragma unroll
              for (int i = 0; i < 32; ++i) qb[i] = qh[(2 * ch + 1) * 32 + i];
              fma_quad(acc, qa, kc.xy);
              __builtin_amdgcn_s_waitcnt(0xc07f);  // quad 2ch+1 ready
              if (ch + 1 < 8) {
#pragma unroll
                for (int i = 0; i < 32; ++i) qa[i] = qh[(2 * ch + 2) * 32 + i];
                kn = *reinterpret_cast<const u32x4*>(rowp + (ch + 1) * 16);
              }
              fma_quad(acc, qb, kc.zw);
              kc = kn;
            }
          }
          wave_order();
        }
        if (cur_bad && lane == 0) atomicOr(a.err, GP_DEVERR_PAGE);
        if (ptile != tcur) {  // the previous tile lies in C_t (it is not a wave's last)
#pragma unroll
          for (int q = 0; q < kNQ; ++q) md[q] = fmaxf(md[q], pacc[q]);
        }
#pragma unroll
        for (int qi = 0; qi < kNQ; ++qi) pacc[qi] = acc[qi];
        ptile = tcur;
        if (!has_next) break;
      }
      float4* out = reinterpret_cast<float4*>(lg + (int64_t)ptile * (64 * kNQ)) + lane;
      out[0] = make_float4(pacc[0], pacc[1], pacc[2], pacc[3]);
      out[64] = make_float4(pacc[4], pacc[5], pacc[6], pacc[7]);
      if ((ptile >> 2) < P - 1) {
#pragma unroll
        for (int q = 0; q < kNQ; ++q) md[q] = fmaxf(md[q], pacc[q]);
      } else {
#pragma unroll
        for (int q = 0; q < kNQ; ++q) ml[q] = pacc[q];
      }
    }
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        md[q] = fmaxf(md[q], __shfl_xor(md[q], off));
        ml[q] = fmaxf(ml[q], __shfl_xor(ml[q], off));
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < kNQ; ++q) {
        s_wmax[w][0][q] = md[q];
        s_wmax[w][1][q] = ml[q];
      }
    }
    __syncthreads();  // logits visible to the block, maxima gathered
    if (t < kNQ) {
      float d = -INFINITY, e = -INFINITY;
      for (int ww = 0; ww < kDW; ++ww) {
        d = fmaxf(d, s_wmax[ww][0][t]);
        e = fmaxf(e, s_wmax[ww][1][t]);
      }
      s_m[0][t] = d;
      s_m[1][t] = fmaxf(d, e);
    }
    // clear the first-digit histograms (the stage is free now)
    for (int k = t; k < 2 * kH1; k += kDT) h1m[k] = 0.0;
    __syncthreads();
    float mdem[kNQ], mall[kNQ];
    bool same[kNQ];
    bool all_same = true;
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {  // block-uniform: held in scalar registers
      mdem[q] = uniform_f(s_m[0][q]);
      mall[q] = uniform_f(s_m[1][q]);
      same[q] = mdem[q] == mall[q];
      all_same = all_same && same[q];
    }

    // ---- 2. exact fixed-point normalisers ----------------------------------------
    // Z = sum over the set of floor(e * 2^40).  Each term is an integer-valued
    // float (mass40); a lane sums its ceil(N / kDT) terms in fp64, exactly
    // while that is below 2^13 terms; lanes and waves combine in uint64.
    // Z over all slots = (sum over C_t) + (sum over the newest page); when the
    // two maxima agree the C_t part is also Z over C_t.
    {
      double zc[kNQ], zd[kNQ];
#pragma unroll
      for (int q = 0; q < kNQ; ++q) zc[q] = zd[q] = 0.0;
      auto ct_terms = [&](auto tag) {
        for (int64_t i = t; i < ndem; i += kDT) {
          float lv[kNQ];
          load_logits8(lg, i, lv);
#pragma unroll
          for (int q = 0; q < kNQ; ++q) {
            zc[q] += (double)mass40(gp_exp(lv[q] - mall[q]));
            if (!decltype(tag)::value && !same[q])
              zd[q] += (double)mass40(gp_exp(lv[q] - mdem[q]));
          }
        }
      };
      if (all_same)
        ct_terms(AllSame{});
      else
        ct_terms(SomeDiffer{});
#pragma unroll
      for (int q = 0; q < kNQ; ++q)
        if (same[q]) zd[q] = zc[q];
      for (int64_t i = ndem + t; i < N; i += kDT) {
        float lv[kNQ];
        load_logits8(lg, i, lv);
#pragma unroll
        for (int q = 0; q < kNQ; ++q) zc[q] += (double)mass40(gp_exp(lv[q] - mall[q]));
      }
      static_assert(2 * kNQ == 16, "one transposed reduction of 16 sums");
      uint64_t zv[2 * kNQ], zs[4];
#pragma unroll
      for (int v = 0; v < 2 * kNQ; ++v) zv[v] = (uint64_t)(v < kNQ ? zd[v] : zc[v - kNQ]);
      wave_sum16_u64(zv, zs);
      if ((lane & 15) == 0) {
        const int v0 = (lane >> 5) * 8 + ((lane >> 4) & 1) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) s_red[w][v0 + j] = zs[j];
      }
      __syncthreads();
      if (t < 2 * kNQ) {
        uint64_t z = 0;
        for (int ww = 0; ww < kDW; ++ww) z += s_red[ww][t];
        const float zf = (float)z * kFixInv;
        if (t < kNQ) s_rho[0][t] = ndem > 0 ? 1.0f / zf : 0.0f;
        else s_rho[1][t - kNQ] = 1.0f / zf;
      }
      __syncthreads();
    }

    // ---- 3. distributions, importance, demand keys, first-digit histograms -----
    {
      float rd[kNQ], ra[kNQ];
#pragma unroll
      for (int q = 0; q < kNQ; ++q) {
        rd[q] = uniform_f(s_rho[0][q]);
        ra[q] = uniform_f(s_rho[1][q]);
      }
      double w0 = 0.0, w1 = 0.0;
      auto ct_tokens = [&](auto tag) {
      for (int64_t i = t; i < ndem; i += kDT) {
        float lv[kNQ];
        load_logits8(lg, i, lv);
        float aa[2], ad[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          float sa = 0.0f, sd = 0.0f;
#pragma unroll
          for (int g = 0; g < kGroup; ++g) {
            const int q = x * kGroup + g;
            const float ea = gp_exp(lv[q] - mall[q]);
            sa = sa + ea * ra[q];
            const float ed = (decltype(tag)::value || same[q]) ? ea : gp_exp(lv[q] - mdem[q]);
            sd = sd + ed * rd[q];
          }
          aa[x] = sa * (1.0f / (float)kGroup);
          ad[x] = sd * (1.0f / (float)kGroup);
        }
        a.imp[row_tok + i] = fmaxf(aa[0], aa[1]);
        if (a.abar) reinterpret_cast<float2*>(a.abar)[row_tok + i] = make_float2(aa[0], aa[1]);
        reinterpret_cast<float2*>(rk)[i] = make_float2(ad[0], ad[1]);
        const float f0 = mass40(ad[0]), f1 = mass40(ad[1]);
        atomicAdd(&h1m[__float_as_uint(ad[0]) >> 20], (double)f0);
        atomicAdd(&h1m[kH1 + (__float_as_uint(ad[1]) >> 20)], (double)f1);
        w0 += (double)f0;
        w1 += (double)f1;
      }
      };
      if (all_same)
        ct_tokens(AllSame{});
      else
        ct_tokens(SomeDiffer{});
      for (int64_t i = ndem + t; i < N; i += kDT) {
        float lv[kNQ];
        load_logits8(lg, i, lv);
        float aa[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          float sa = 0.0f;
#pragma unroll
          for (int g = 0; g < kGroup; ++g) {
            const int q = x * kGroup + g;
            sa = sa + gp_exp(lv[q] - mall[q]) * ra[q];
          }
          aa[x] = sa * (1.0f / (float)kGroup);
        }
        a.imp[row_tok + i] = fmaxf(aa[0], aa[1]);
        if (a.abar) reinterpret_cast<float2*>(a.abar)[row_tok + i] = make_float2(aa[0], aa[1]);
      }
      const uint64_t ws0 = wave_sum_u64((uint64_t)w0), ws1 = wave_sum_u64((uint64_t)w1);
      if (lane == 0) {
        s_red[w][0] = ws0;
        s_red[w][1] = ws1;
      }
      __syncthreads();
      if (t < 2) {
        uint64_t sw = 0;
        for (int ww = 0; ww < kDW; ++ww) sw += s_red[ww][t];
        s_W[t] = sw;
      }
      __syncthreads();
    }

    // ---- 4. D_p of each view ------------------------------------------------------
    // Runs for every row, including a single-page one (no candidates: its
    // loops are empty and its outputs are forced to 0 at the end); no branch
    // around this phase's barriers, so the row loop keeps one plain structure.
    {
    // first digit of both views (the whole block searches), then one pass
    // over the key ring collects each view's boundary-bucket members into its
    // half of the LDS list and counts the slots in buckets above it
    if (t < 2) {
      s_cab[t] = 0;
      s_list_n[t] = 0;
    }
    block_first_digit(h1m, s_W, (uint32_t)a.p_num, (uint32_t)a.p_den, s_wm, s_dig, s_mab);
    __syncthreads();
    {
      const uint32_t d0 = (uint32_t)s_dig[0], d1 = (uint32_t)s_dig[1];
      uint32_t above0 = 0, above1 = 0;
      // two tokens per 16-byte load (ndem is a multiple of the page size),
      // kRingU loads in flight per thread before any is used
      const float4* rk4 = reinterpret_cast<const float4*>(rk);
      const int64_t npair = ndem >> 1;
      auto visit = [&](uint32_t k0, uint32_t k1) {
        above0 += (k0 >> 20) > d0;
        above1 += (k1 >> 20) > d1;
        if ((k0 >> 20) == d0) {
          const int idx = atomicAdd(&s_list_n[0], 1);
          if (idx < kListHalf) list[idx] = k0;
        }
        if ((k1 >> 20) == d1) {
          const int idx = atomicAdd(&s_list_n[1], 1);
          if (idx < kListHalf) list[kListHalf + idx] = k1;
        }
      };
      for (int64_t p0 = t; p0 < npair; p0 += (int64_t)kRingU * kDT) {
        float4 kk[kRingU];
#pragma unroll
        for (int u = 0; u < kRingU; ++u) {
          const int64_t pi = p0 + (int64_t)u * kDT;
          kk[u] = rk4[pi < npair ? pi : p0];
        }
#pragma unroll
        for (int u = 0; u < kRingU; ++u) {
          if (p0 + (int64_t)u * kDT < npair) {
            visit(__float_as_uint(kk[u].x), __float_as_uint(kk[u].y));
            visit(__float_as_uint(kk[u].z), __float_as_uint(kk[u].w));
          }
        }
      }
      above0 = wave_sum_u32(above0);
      above1 = wave_sum_u32(above1);
      if (lane == 0) {
        atomicAdd(&s_cab[0], above0);
        atomicAdd(&s_cab[1], above1);
      }
    }
    __syncthreads();
    // digits 2 (bits 19..10) and 3 (bits 9..0) over each view's boundary
    // members, both views in the same passes (each into its own counts and
    // masses, then one block-wide search for both)
    {
      const bool in_lds0 = s_list_n[0] <= kListHalf, in_lds1 = s_list_n[1] <= kListHalf;
      uint32_t prefix0 = (uint32_t)s_dig[0] << 20, prefix1 = (uint32_t)s_dig[1] << 20;
      for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 10 : 0;
        const uint32_t mask = pass == 0 ? 0xfff00000u : 0xfffffc00u;
        for (int k = t; k < 2 * kH2; k += kDT) {
          h2c[k] = 0;
          h2m[k] = 0;
        }
        __syncthreads();
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const uint32_t prefix = x == 0 ? prefix0 : prefix1;
          uint32_t* hc = h2c + x * kH2;
          uint64_t* hm = h2m + x * kH2;
          if (x == 0 ? in_lds0 : in_lds1) {
            const uint32_t* lst = list + x * kListHalf;
            const int n = s_list_n[x];
            for (int k = t; k < n; k += kDT) {
              const uint32_t key = lst[k];
              if ((key & mask) == prefix) {
                const uint32_t dig = (key >> shift) & (kH2 - 1);
                atomicAdd(&hc[dig], 1u);
                atomicAdd((unsigned long long*)&hm[dig],
                          (unsigned long long)fix40(__uint_as_float(key)));
              }
            }
          } else {
            for (int64_t i = t; i < ndem; i += kDT) {
              const uint32_t key = __float_as_uint(rk[i * 2 + x]);
              if ((key & mask) == prefix) {
                const uint32_t dig = (key >> shift) & (kH2 - 1);
                atomicAdd(&hc[dig], 1u);
                atomicAdd((unsigned long long*)&hm[dig],
                          (unsigned long long)fix40(__uint_as_float(key)));
              }
            }
          }
        }
        __syncthreads();
        block_next_digit(h2c, h2m, s_W, (uint32_t)a.p_num, (uint32_t)a.p_den, s_wm, s_wc, s_dig,
                         s_mab, s_cab);
        __syncthreads();
        prefix0 |= (uint32_t)s_dig[0] << shift;
        prefix1 |= (uint32_t)s_dig[1] << shift;
      }
      if (t < 2) {
        int32_t* outp = t == 0 ? a.k_short : a.k_long;
        const uint32_t prefix = t == 0 ? prefix0 : prefix1;
        const uint64_t target = s_W[t] * (uint64_t)a.p_num;
        const bool has = ndem > 0;
        const uint64_t wt = fix40(__uint_as_float(has ? prefix : 0u));
        const uint64_t need = target - s_mab[t] * (uint64_t)a.p_den;
        const uint64_t den = wt * (uint64_t)a.p_den;
        const uint64_t rest = den != 0 ? (need + den - 1) / den : 0;
        outp[row] = has ? (int32_t)(s_cab[t] + rest) : 0;
      }
      __syncthreads();
    }
    }
  }
}

hipError_t launch_demand(const Params& p, const WsLayout& w, const uint16_t* k_pool,
                         int pool_pages, const int32_t* block_table, int max_pages, int B,
                         void* ws, int32_t* k_short, int32_t* k_long, float* abar, int32_t* err,
                         hipStream_t s) {
  char* base = static_cast<char*>(ws);
  DemandArgs a;
  a.k_pool = k_pool;
  a.pool_pages = pool_pages;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.L = p.L;
  a.Hkv = p.Hkv;
  a.B = B;
  a.b = p.b;
  a.p_num = p.p_num;
  a.p_den = p.p_den;
  a.hdr = reinterpret_cast<const WsHeader*>(base + w.header);
  a.page_off = reinterpret_cast<const int64_t*>(base + w.page_off);
  a.req_order = reinterpret_cast<const int32_t*>(base + w.req_order);
  a.row_counter = &reinterpret_cast<WsHeader*>(base + w.header)->row_counter;
  a.qhat = reinterpret_cast<const float*>(base + w.qhat);
  a.ring_logits = reinterpret_cast<float*>(base + w.ring_logits);
  a.ring_keys = reinterpret_cast<float*>(base + w.ring_keys);
  a.ring_tokens = w.ring_tokens;
  a.imp = reinterpret_cast<float*>(base + w.imp);
  a.k_short = k_short;
  a.k_long = k_long;
  a.abar = abar;
  a.err = err;
  hipLaunchKernelGGL(k_demand, dim3((unsigned)w.blocks), dim3(kDT), 0, s, a, a.qhat, a.k_pool,
                     a.block_table);
  return hipGetLastError();
}

}  // namespace gp
