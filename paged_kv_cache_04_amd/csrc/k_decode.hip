// Decode-step paged attention for one layer with the dual-timescale summary
// update fused into it (§4.1: the attention kernel of the regular decoding
// path also updates both summaries from the normalised pre-RoPE query;
// App. E.1 "Initialization and online update"; §3.1 Eq. 3 defines the
// full-cache output o_t).  Citations are to "GrowPage: On-Demand KV
// Budgeting for Efficient LLM Reasoning Serving" (arXiv 2609.03494).
//
// Three kernels:
//  1. prep, a workgroup per request: the summary update, the rotated and
//     scaled queries of all heads (to the workspace), and the request's work
//     units, one per (cached page, KV head), at its offset in the batch list;
//  2. units, persistent: every wave walks the unit list with a stride of all
//     waves of the grid and computes, for the 4 query heads of the unit's KV
//     head, the page's maximum logit, its sum of exp(l - max) and the
//     unnormalised sum of exp(l - max) v.  A wave reads its page's 64 KiB of
//     K and 64 KiB of V as one sequential stream of 16-byte loads; this
//     one-stream-per-wave order reads HBM markedly faster than workgroups
//     whose waves share the pages of one token range;
//  3. merge, a workgroup per (request, KV head): combines the pages.
// Work units never straddle requests, so each wave's running sums need no
// cross-wave synchronisation; the partials cost 2 KiB per page and head.
// Inside a unit, lanes own slices of the head dimension: 16 lanes hold one
// token's 128 elements (8 each, one 16-byte load of K and one of V), so a
// load instruction reads 4 whole consecutive rows, and the query's slice of
// all 4 heads (32 values) stays in registers.  Pass 1 streams the page's
// keys, 32 tokens per step (8 loads per lane, the next step's loads issued as
// soon as the current ones are consumed), reduces the 32 partial dot products
// of a step's 8 tokens x 4 heads across the row's 16 lanes by a transposed
// DPP reduction (each lane ends with 2 complete logits) and stores the
// logits in the wave's LDS stage; the page maximum is known at its end, so
// each weight exp(l - max) is taken once, in place, with no rescaling; pass 2
// streams the values and accumulates them with the weights read from LDS.  The path reads K
// and V once: 512 bytes per cached token and KV head, HBM-bound.  Arithmetic
// is fp32 with the hardware exp2; results are compared with the fp64
// definition within a stated tolerance.
#include "gp_internal.h"

namespace gp {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kDecT = 256;                             // threads per workgroup (4 waves)
constexpr int kDecWaves = kDecT / 64;
constexpr int kStep = 32;                              // tokens per wave step
constexpr int kPartStride = kGroup * kD + 2 * kGroup;  // floats per unit partial
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// value of another lane of the same 16-lane row, by a DPP lane pattern
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

// orders a wave's LDS accesses (all lanes) before the following ones
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct DecodeArgs {
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  int pool_pages;
  const int32_t* block_table;
  int max_pages;
  const int32_t* num_pages;
  const int32_t* num_tokens;
  const int32_t* slot;
  const int32_t* position;
  int B, layer, Hkv, Hq, M, rope_rows, unit_cap;
  float alpha_s, alpha_l;
  const float* q;        // [B][Hq][d]
  float* qstate;         // [L][M][2][Hq][d] or null
  const uint8_t* first;  // [B] or null
  const float* rope;     // [rope_rows][d]
  float* qhat;           // [B][Hq][d]  rotated, scaled queries
  int2* units;           // [unit_cap]  (request * Hkv + KV head, page index)
  int32_t* page_pre;     // [B + 1]     pages before each request (valid requests only)
  int32_t* n_units;      // [1]
  float* part;           // [unit_cap][kPartStride]
  float* out;            // [B][Hq][d]
  int32_t* err;
};

// Tokens of request r that attention covers, or -1 when the counts are
// inconsistent (then the request's output is zero and PAGES is flagged).
__device__ __forceinline__ int decode_tokens(const DecodeArgs& a, int r) {
  const int P = a.num_pages[r], N = a.num_tokens[r];
  if (P < 1 || P > a.max_pages || N < 1 || N > P * kPage) return -1;
  return N;
}

// ---- 1. prep ------------------------------------------------------------------
__global__ __launch_bounds__(kDecT) void k_decode_prep(DecodeArgs a) {
  const int t = threadIdx.x, r = blockIdx.x;
  const int Hq = a.Hq;
  int pos = a.position[r];
  if (pos < 0 || pos >= a.rope_rows) {
    if (t == 0) atomicOr(a.err, GP_DEVERR_POSITION);
    pos = pos < 0 ? 0 : a.rope_rows - 1;
  }
  const int sl = a.slot[r];
  const bool upd = a.qstate && sl >= 0 && sl < a.M;
  if (a.qstate && !upd && t == 0) atomicOr(a.err, GP_DEVERR_SLOT);
  const bool init = a.first && a.first[r];
  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
  for (int it = t; it < Hq * (kD / 2); it += kDecT) {
    const int g = it / (kD / 2), j = it % (kD / 2);
    const float* qr = a.q + ((int64_t)r * Hq + g) * kD;
    const float x1 = qr[j], x2 = qr[j + kD / 2];
    // summary update, bit for bit the gp_update_summaries arithmetic:
    // qbar + alpha (q - qbar), or q itself on a slot's first step
    if (upd) {
      float* sp = a.qstate + (((int64_t)a.layer * a.M + sl) * 2 * Hq + g) * kD;
      float* lp = sp + (int64_t)Hq * kD;
      if (init) {
        sp[j] = x1; sp[j + kD / 2] = x2;
        lp[j] = x1; lp[j + kD / 2] = x2;
      } else {
        sp[j] = __builtin_fmaf(a.alpha_s, x1 - sp[j], sp[j]);
        sp[j + kD / 2] = __builtin_fmaf(a.alpha_s, x2 - sp[j + kD / 2], sp[j + kD / 2]);
        lp[j] = __builtin_fmaf(a.alpha_l, x1 - lp[j], lp[j]);
        lp[j + kD / 2] = __builtin_fmaf(a.alpha_l, x2 - lp[j + kD / 2], lp[j + kD / 2]);
      }
    }
    // rotate to the query's position (pairs j, j + d/2), scale by 1/sqrt(d)
    const float c = a.rope[(int64_t)pos * kD + j], sn = a.rope[(int64_t)pos * kD + kD / 2 + j];
    float* qh = a.qhat + ((int64_t)r * Hq + g) * kD;
    qh[j] = __builtin_fmaf(x1, c, -(x2 * sn)) * scale;
    qh[j + kD / 2] = __builtin_fmaf(x2, c, x1 * sn) * scale;
  }
  // pages of the requests before this one and of the whole batch (0 for a
  // request with inconsistent counts), then this request's units, in
  // (request, page, KV head) order
  __shared__ int red[2][kDecWaves];
  int before = 0, all = 0;
  for (int i = t; i < a.B; i += kDecT) {
    const int N = decode_tokens(a, i);
    if (N < 0 && r == 0) atomicOr(a.err, GP_DEVERR_PAGES);
    const int n = N < 0 ? 0 : (N + kPage - 1) / kPage;
    all += n;
    if (i < r) before += n;
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    before += __shfl_xor(before, m);
    all += __shfl_xor(all, m);
  }
  if ((t & 63) == 0) {
    red[0][t >> 6] = before;
    red[1][t >> 6] = all;
  }
  __syncthreads();
  before = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  all = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const bool fits = (int64_t)all * a.Hkv <= a.unit_cap;
  if (t == 0) {
    a.page_pre[r] = before;
    if (r == 0) {
      a.page_pre[a.B] = all;
      *a.n_units = fits ? all * a.Hkv : 0;
      if (!fits) atomicOr(a.err, GP_DEVERR_PAGES);  // device pages beyond the workspace's size
    }
  }
  const int N = decode_tokens(a, r);
  const int own = N < 0 ? 0 : (N + kPage - 1) / kPage;
  if (fits)
    for (int k = t; k < own * a.Hkv; k += kDecT)
      a.units[(int64_t)before * a.Hkv + k] = make_int2(r * a.Hkv + k % a.Hkv, k / a.Hkv);
}

// ---- 2. units -----------------------------------------------------------------
// Per unit, two passes over the page: the keys (logits to the wave's LDS
// stage, the page maximum per head), then the weights exp(l - max) in place
// with their sums, then the values.  The wave's memory stream is the K tile
// followed by the V tile, and no running sum is ever rescaled.
__global__ __launch_bounds__(kDecT) void k_decode_units(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) float lgs[kDecWaves][kPage][kGroup];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_units = __builtin_amdgcn_readfirstlane(*a.n_units);
  const int sub = lane & 15, grp = lane >> 4;  // slice of d, token within a group of 4
  // lane bits within its row of 16, used by the transposed reduction
  const bool b3 = sub & 8, b2 = sub & 4, b1 = sub & 2, b0 = sub & 1;
  const int my_i = sub >> 1;  // token group whose logits of heads 2 b0, 2 b0 + 1 this lane ends with
  float(*lw)[kGroup] = lgs[w];
  const int64_t head_stride = (int64_t)kPage * kD;  // elements per (page, KV head)
  for (int u = blockIdx.x * kDecWaves + w; u < n_units; u += gridDim.x * kDecWaves) {
    const int2 e = a.units[u];
    const int rh = __builtin_amdgcn_readfirstlane(e.x), pg = __builtin_amdgcn_readfirstlane(e.y);
    const int r = rh / a.Hkv, h = rh % a.Hkv;
    const int begin = pg * kPage;
    const int end = min(__builtin_amdgcn_readfirstlane(a.num_tokens[r]), begin + kPage);
    const int n_tok = end - begin;                           // 1 .. 256
    const int n_pad = (n_tok + kStep - 1) / kStep * kStep;  // slots the steps cover
    const int page = a.block_table[(int64_t)r * a.max_pages + pg];
    const bool ok = page >= 0 && page < a.pool_pages;
    if (!ok && lane == 0) atomicOr(a.err, GP_DEVERR_PAGE);
    const int64_t base =
        (((int64_t)a.layer * a.pool_pages + (ok ? page : 0)) * a.Hkv + h) * head_stride;
    const uint16_t* kp = a.k_pool + base;
    const uint16_t* vp = a.v_pool + base;
    // element offset of token group i of the step at slot c (clamped to the
    // step's first slot past the end, so every load stays inside the tile)
    auto row_off = [&](int c, int i) -> int64_t {
      const int tok = c + 4 * i + grp;
      return (int64_t)(tok < n_tok ? tok : c) * kD + sub * 8;
    };
    u32x4 kv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      kv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + row_off(0, i)));
    // the query slices of the 4 heads
    float qs[kGroup][8];
#pragma unroll
    for (int gg = 0; gg < kGroup; ++gg) {
      const float4* qp = reinterpret_cast<const float4*>(
          a.qhat + ((int64_t)r * a.Hq + h * kGroup + gg) * kD + sub * 8);
      const float4 x = qp[0], y = qp[1];
      qs[gg][0] = x.x; qs[gg][1] = x.y; qs[gg][2] = x.z; qs[gg][3] = x.w;
      qs[gg][4] = y.x; qs[gg][5] = y.y; qs[gg][6] = y.z; qs[gg][7] = y.w;
    }
    // -- pass 1: logits ---------------------------------------------------------
    float mx0 = -INFINITY, mx1 = -INFINITY;  // this lane's heads 2 b0, 2 b0 + 1
    for (int c0 = 0; c0 < n_tok; c0 += kStep) {
      // partial dot products over this lane's 8 elements: v[i * 4 + g]
      float v[8 * kGroup];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float k0 = bf16_lo(kv[i].x), k1 = bf16_hi(kv[i].x), k2 = bf16_lo(kv[i].y),
                    k3 = bf16_hi(kv[i].y), k4 = bf16_lo(kv[i].z), k5 = bf16_hi(kv[i].z),
                    k6 = bf16_lo(kv[i].w), k7 = bf16_hi(kv[i].w);
#pragma unroll
        for (int gg = 0; gg < kGroup; ++gg) {
          float d = qs[gg][0] * k0;
          d = __builtin_fmaf(qs[gg][1], k1, d);
          d = __builtin_fmaf(qs[gg][2], k2, d);
          d = __builtin_fmaf(qs[gg][3], k3, d);
          d = __builtin_fmaf(qs[gg][4], k4, d);
          d = __builtin_fmaf(qs[gg][5], k5, d);
          d = __builtin_fmaf(qs[gg][6], k6, d);
          d = __builtin_fmaf(qs[gg][7], k7, d);
          v[i * kGroup + gg] = d;
        }
      }
      // the next step's keys (or the first values) go into the registers just
      // consumed
      const int cn = c0 + kStep;
      if (cn < n_tok) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          kv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + row_off(cn, i)));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          kv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + row_off(0, i)));
      }
      // transposed reduction over the 16 lanes of the row: at each step a
      // lane keeps the half of its values selected by one lane bit and adds
      // the partner's copy of that half (partners sub^8, sub^7, sub^2, sub^1
      // have the opposite bit and the same higher bits), so after 4 steps
      // lane sub holds the full dot products v[2 sub] and v[2 sub + 1]
      float a16[16], a8[8], a4[4], x[2];
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const float keep = b3 ? v[m + 16] : v[m], send = b3 ? v[m] : v[m + 16];
        a16[m] = keep + dpp_f<0x128>(send);  // row_ror:8 = lane sub ^ 8
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float keep = b2 ? a16[m + 8] : a16[m], send = b2 ? a16[m] : a16[m + 8];
        a8[m] = keep + dpp_f<0x141>(send);  // row_half_mirror = lane sub ^ 7
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float keep = b1 ? a8[m + 4] : a8[m], send = b1 ? a8[m] : a8[m + 4];
        a4[m] = keep + dpp_f<0x4E>(send);  // quad_perm 2,3,0,1 = lane sub ^ 2
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float keep = b0 ? a4[m + 2] : a4[m], send = b0 ? a4[m] : a4[m + 2];
        x[m] = keep + dpp_f<0xB1>(send);  // quad_perm 1,0,3,2 = lane sub ^ 1
      }
      const int tl = c0 + 4 * my_i + grp;
      const bool live = ok && tl < n_tok;
      const float l0 = live ? x[0] : -INFINITY, l1 = live ? x[1] : -INFINITY;
      mx0 = fmaxf(mx0, l0);
      mx1 = fmaxf(mx1, l1);
      *reinterpret_cast<float2*>(&lw[tl][b0 ? 2 : 0]) = make_float2(l0, l1);
    }
    // page maximum per head: lanes with the same bit 0 hold the same heads
    float mh[kGroup];
    {
      float y[2] = {mx0, mx1};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        y[q] = fmaxf(y[q], dpp_f<0x4E>(y[q]));
        y[q] = fmaxf(y[q], dpp_f<0x124>(y[q]));  // row_ror:4
        y[q] = fmaxf(y[q], dpp_f<0x128>(y[q]));  // row_ror:8
        y[q] = fmaxf(y[q], __shfl_xor(y[q], 16));
        y[q] = fmaxf(y[q], __shfl_xor(y[q], 32));
      }
      const float o0 = dpp_f<0xB1>(y[0]), o1 = dpp_f<0xB1>(y[1]);  // the other two heads
      mh[0] = b0 ? o0 : y[0];
      mh[1] = b0 ? o1 : y[1];
      mh[2] = b0 ? y[0] : o0;
      mh[3] = b0 ? y[1] : o1;
    }
    wave_sync();
    // -- weights in place: entry idx = 4 token + head; a lane's entries all
    // have head lane & 3 -------------------------------------------------------
    const int hl = lane & 3;
    const float m_l = hl == 0 ? mh[0] : hl == 1 ? mh[1] : hl == 2 ? mh[2] : mh[3];
    float s_l = 0.0f;
    float* flat = &lw[0][0];
    for (int idx = lane; idx < n_pad * kGroup; idx += 64) {
      const float l = flat[idx];
      const float pv = l == -INFINITY ? 0.0f : exp_fast(l - m_l);
      flat[idx] = pv;
      s_l += pv;
    }
    // sum over the lanes of one head (same lane & 3): row_ror 4 and 8, then rows
    s_l += dpp_f<0x124>(s_l);
    s_l += dpp_f<0x128>(s_l);
    s_l += __shfl_xor(s_l, 16);
    s_l += __shfl_xor(s_l, 32);
    wave_sync();
    // -- pass 2: values ----------------------------------------------------------
    float acc[kGroup][8];
#pragma unroll
    for (int gg = 0; gg < kGroup; ++gg)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[gg][k] = 0.0f;
    for (int c0 = 0; c0 < n_tok; c0 += kStep) {
      float4 pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pr[i] = *reinterpret_cast<const float4*>(&lw[c0 + 4 * i + grp][0]);
      u32x4 vv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) vv[i] = kv[i];
      const int cn = c0 + kStep;
      if (cn < n_tok) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          kv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + row_off(cn, i)));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float vf[8] = {bf16_lo(vv[i].x), bf16_hi(vv[i].x), bf16_lo(vv[i].y),
                             bf16_hi(vv[i].y), bf16_lo(vv[i].z), bf16_hi(vv[i].z),
                             bf16_lo(vv[i].w), bf16_hi(vv[i].w)};
        const float pg4[kGroup] = {pr[i].x, pr[i].y, pr[i].z, pr[i].w};
#pragma unroll
        for (int gg = 0; gg < kGroup; ++gg)
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[gg][k] = __builtin_fmaf(pg4[gg], vf[k], acc[gg][k]);
      }
    }
    wave_sync();
    // merge the wave's 4 token rows (lanes l, l^16, l^32, l^48)
#pragma unroll
    for (int gg = 0; gg < kGroup; ++gg) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        acc[gg][k] += __shfl_xor(acc[gg][k], 16);
        acc[gg][k] += __shfl_xor(acc[gg][k], 32);
      }
    }
    float* pp = a.part + (int64_t)u * kPartStride;
    if (lane < 16) {
#pragma unroll
      for (int gg = 0; gg < kGroup; ++gg) {
        float4* o = reinterpret_cast<float4*>(pp + gg * kD + sub * 8);
        o[0] = make_float4(acc[gg][0], acc[gg][1], acc[gg][2], acc[gg][3]);
        o[1] = make_float4(acc[gg][4], acc[gg][5], acc[gg][6], acc[gg][7]);
      }
    }
    if (lane < kGroup) {
      pp[kGroup * kD + lane] = m_l;
      pp[kGroup * kD + kGroup + lane] = s_l;
    }
  }
}

// ---- 3. merge -------------------------------------------------------------------
// o = sum_p e^(m_p - m) o_p / sum_p e^(m_p - m) S_p over the request's pages,
// m the largest page maximum.  1024 threads: the maxima over all threads,
// then 4 groups of pages summed side by side and added in LDS.
constexpr int kMergeT = 1024;

__global__ __launch_bounds__(kMergeT) void k_decode_merge(DecodeArgs a) {
  __shared__ float s_m[kMergeT / 64][kGroup];
  __shared__ float s_o[4][kGroup][kD];
  __shared__ float s_s[4][kGroup];
  const int t = threadIdx.x;
  const int rh = blockIdx.x;
  const int r = rh / a.Hkv, h = rh % a.Hkv;
  const int N = decode_tokens(a, r);
  const bool empty = N < 0 || *a.n_units == 0;
  const int np = empty ? 0 : (N + kPage - 1) / kPage;
  const float* base = a.part + ((int64_t)a.page_pre[r] * a.Hkv + h) * kPartStride;
  const int64_t stride = (int64_t)a.Hkv * kPartStride;  // next page, same KV head
  // maxima: thread t reads head t & 3 of pages t >> 2, (t >> 2) + 256, ...
  float mloc = -INFINITY;
  for (int idx = t; idx < np * kGroup; idx += kMergeT)
    mloc = fmaxf(mloc, base[(idx >> 2) * stride + kGroup * kD + (idx & 3)]);
#pragma unroll
  for (int m = 4; m < 64; m <<= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, m));
  if ((t & 63) < kGroup) s_m[t >> 6][t & 63] = mloc;
  __syncthreads();
  const int grp = t >> 8, g = (t >> 6) & 3, j = t & 63;
  float m = -INFINITY;
#pragma unroll
  for (int w = 0; w < kMergeT / 64; ++w) m = fmaxf(m, s_m[w][g]);
  float o1 = 0.0f, o2 = 0.0f, ssum = 0.0f;
#pragma unroll 4
  for (int p = grp; p < np; p += 4) {
    const float* ps = base + p * stride;
    const float mp = ps[kGroup * kD + g];
    const float f = mp == -INFINITY ? 0.0f : exp_fast(mp - m);
    o1 = __builtin_fmaf(f, ps[g * kD + j], o1);
    o2 = __builtin_fmaf(f, ps[g * kD + j + kD / 2], o2);
    ssum = __builtin_fmaf(f, ps[kGroup * kD + kGroup + g], ssum);
  }
  s_o[grp][g][j] = o1;
  s_o[grp][g][j + kD / 2] = o2;
  if (j == 0) s_s[grp][g] = ssum;
  __syncthreads();
  if (grp == 0) {
    float x1 = 0.0f, x2 = 0.0f, sv = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x1 += s_o[q][g][j];
      x2 += s_o[q][g][j + kD / 2];
      sv += s_s[q][g];
    }
    const float inv = sv > 0.0f ? 1.0f / sv : 0.0f;
    float* orow = a.out + ((int64_t)r * a.Hq + h * kGroup + g) * kD;
    orow[j] = x1 * inv;
    orow[j + kD / 2] = x2 * inv;
  }
}

DecodeWs decode_ws_layout(const Params& p, int B, int64_t total_pages) {
  DecodeWs w{};
  const int64_t cap = total_pages * p.Hkv;
  size_t o = 0;
  w.qhat = o;     o = align256(o + sizeof(float) * (size_t)B * p.Hq * kD);
  w.units = o;    o = align256(o + sizeof(int2) * (size_t)cap);
  w.page_pre = o; o = align256(o + sizeof(int32_t) * (size_t)(B + 1));
  w.n_units = o;  o = align256(o + sizeof(int32_t));
  w.part = o;     o = align256(o + sizeof(float) * (size_t)cap * kPartStride);
  w.total = o;
  w.unit_cap = cap;
  return w;
}

hipError_t launch_decode(const Params& p, const DecodeWs& w, int B, int layer,
                         const uint16_t* k_pool, const uint16_t* v_pool, int pool_pages,
                         const int32_t* block_table, int max_pages, const int32_t* num_pages,
                         const int32_t* num_tokens, const int32_t* slot, const int32_t* position,
                         const float* q, float* qstate, const uint8_t* first, const float* rope,
                         int rope_rows, int unit_blocks, void* ws, float* out, int32_t* err,
                         hipStream_t s) {
  char* base = static_cast<char*>(ws);
  DecodeArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.pool_pages = pool_pages;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.num_tokens = num_tokens;
  a.slot = slot;
  a.position = position;
  a.B = B;
  a.layer = layer;
  a.Hkv = p.Hkv;
  a.Hq = p.Hq;
  a.M = p.M;
  a.rope_rows = rope_rows;
  a.unit_cap = (int)w.unit_cap;
  a.alpha_s = p.alpha_s;
  a.alpha_l = p.alpha_l;
  a.q = q;
  a.qstate = qstate;
  a.first = first;
  a.rope = rope;
  a.qhat = reinterpret_cast<float*>(base + w.qhat);
  a.units = reinterpret_cast<int2*>(base + w.units);
  a.page_pre = reinterpret_cast<int32_t*>(base + w.page_pre);
  a.n_units = reinterpret_cast<int32_t*>(base + w.n_units);
  a.part = reinterpret_cast<float*>(base + w.part);
  a.out = out;
  a.err = err;
  hipLaunchKernelGGL(k_decode_prep, dim3((unsigned)B), dim3(kDecT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_units, dim3((unsigned)unit_blocks), dim3(kDecT), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_merge, dim3((unsigned)B * p.Hkv), dim3(kMergeT), 0, s, a);
  return hipGetLastError();
}

}  // namespace gp
