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
//     units, one per (KV head, cached page), at its offset in the batch list;
//  2. units, persistent: the unit list is cut into equal contiguous ranges,
//     one per wave, so the work is balanced to a page.  For the 4 query
//     heads of a unit's KV head a wave computes the running maximum logit,
//     sum of exp(l - max) and unnormalised sum of exp(l - max) v over runs of
//     pages of one (request, KV head), writing one partial per run.  A wave
//     reads its pages' 64 KiB of K and 64 KiB of V as one sequential stream
//     of 16-byte loads: one stream per wave reads HBM markedly faster than
//     workgroups whose waves share one token range;
//  3. merge, a workgroup per (request, KV head): combines its runs.
// Inside a page, lanes own slices of the head dimension: 16 lanes hold one
// token's 128 elements (8 each, one 16-byte load of K and one of V), so a
// load instruction reads 4 whole consecutive rows, and the query's slice of
// all 4 heads (32 values) stays in registers.  Pass 1 streams the page's
// keys, 32 tokens per step (8 loads per lane; two register buffers hold
// alternate steps, so the next step's loads are always in flight), reduces
// the 32 partial dot products of a step's 8 tokens x 4 heads across the
// row's 16 lanes by a transposed DPP reduction (each lane ends with 2
// complete logits) and stores the logits in the wave's LDS stage; with the
// page maximum known, each weight exp(l - max) is taken once, in place;
// pass 2 streams the values and accumulates them with the weights read from
// LDS.  The path reads K and V once: 512 bytes per cached token and KV head,
// HBM-bound.  Arithmetic is fp32 with the hardware exp2; results are
// compared with the fp64 definition within a stated tolerance.
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
  // (request, KV head, page) order
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
      a.units[(int64_t)before * a.Hkv + k] = make_int2(r * a.Hkv + k / own, k % own);
}

// ---- 2. units -----------------------------------------------------------------
// The unit list is cut into equal contiguous ranges, one per wave.  Units are
// in (request, KV head, page) order, so a wave's range is a few runs of
// consecutive pages of one (request, KV head); the wave keeps running sums
// over a run and writes one partial per run, at the run's first unit index
// (a partial per page would add writes between the reads, which costs HBM
// time far beyond their size).  Per page, two passes: the keys (logits to
// the wave's LDS stage, the page maximum per head; the running maximum grows
// and the running sums are rescaled once if it does), then the weights
// exp(l - max) in place, then the values.  The wave's loads form one stream
// over its range: each page contributes its key steps, then its value steps
// (each part padded to an even number of steps), and two register buffers
// take alternate steps, refilled with the step two ahead as soon as they are
// consumed, so the next step's loads, also the first ones of the next page,
// are always in flight.
struct UnitRef {
  const uint16_t* kp;
  const uint16_t* vp;
  int rh, r, h, n_tok, ns, nsk, len;  // tokens, 32-token steps, first value step, stream length
  bool ok, valid;
};

__device__ __forceinline__ UnitRef unit_ref(const DecodeArgs& a, int u, int u_end) {
  UnitRef x{};
  x.valid = u < u_end;
  if (!x.valid) return x;
  const int2 e = a.units[u];
  x.rh = __builtin_amdgcn_readfirstlane(e.x);
  const int pg = __builtin_amdgcn_readfirstlane(e.y);
  x.r = x.rh / a.Hkv;
  x.h = x.rh % a.Hkv;
  const int begin = pg * kPage;
  x.n_tok = min(__builtin_amdgcn_readfirstlane(a.num_tokens[x.r]), begin + kPage) - begin;
  x.ns = (x.n_tok + kStep - 1) / kStep;
  x.nsk = x.ns + (x.ns & 1);
  x.len = 2 * x.nsk;
  const int page =
      __builtin_amdgcn_readfirstlane(a.block_table[(int64_t)x.r * a.max_pages + pg]);
  x.ok = page >= 0 && page < a.pool_pages;
  const int64_t base =
      (((int64_t)a.layer * a.pool_pages + (x.ok ? page : 0)) * a.Hkv + x.h) * (int64_t)kPage * kD;
  x.kp = a.k_pool + base;
  x.vp = a.v_pool + base;
  return x;
}

// units per wave range
__device__ __forceinline__ int unit_range(int n_units, int waves) {
  return (n_units + waves - 1) / waves;
}

__global__ __launch_bounds__(kDecT) void k_decode_units(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) float lgs[kDecWaves][kPage][kGroup];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_units = __builtin_amdgcn_readfirstlane(*a.n_units);
  const int R = unit_range(n_units, gridDim.x * kDecWaves);
  const int u_begin = (blockIdx.x * kDecWaves + w) * R;
  const int u_end = min(u_begin + R, n_units);
  if (u_begin >= u_end) return;
  const int sub = lane & 15, grp = lane >> 4;  // slice of d, token within a group of 4
  // lane bits within its row of 16, used by the transposed reduction
  const bool b3 = sub & 8, b2 = sub & 4, b1 = sub & 2, b0 = sub & 1;
  const int my_i = sub >> 1;  // token group whose logits of heads 2 b0, 2 b0 + 1 this lane ends with
  const int hl = lane & 3;    // head of this lane's weight entries
  float(*lw)[kGroup] = lgs[w];
  // step si of unit x's stream into buf (nothing for a pad or past the end);
  // element offsets of token group i of a step at slot c are clamped to the
  // step's first slot past the unit's end, so every load stays in the tile
  auto issue_x = [&](const UnitRef& x, int si, u32x4 (&buf)[8]) {
    if (!x.valid) return;
    const uint16_t* src;
    int c;
    if (si < x.ns) {
      src = x.kp;
      c = si * kStep;
    } else if (si >= x.nsk && si < x.nsk + x.ns) {
      src = x.vp;
      c = (si - x.nsk) * kStep;
    } else {
      return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = c + 4 * i + grp;
      const uint32_t off = (uint32_t)((tok < x.n_tok ? tok : c) * kD + sub * 8);  // < 2^15
      buf[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off));
    }
  };
  // the query slices of the 4 heads of unit x (loaded one unit ahead: the
  // load counter is in order, so loads issued after the stream would make
  // their first use wait for the whole stream)
  auto load_q = [&](const UnitRef& x, float (&q)[kGroup][8]) {
    if (!x.valid) return;
#pragma unroll
    for (int gg = 0; gg < kGroup; ++gg) {
      const float4* qp = reinterpret_cast<const float4*>(
          a.qhat + ((int64_t)x.r * a.Hq + x.h * kGroup + gg) * kD + sub * 8);
      const float4 x0 = qp[0], y0 = qp[1];
      q[gg][0] = x0.x; q[gg][1] = x0.y; q[gg][2] = x0.z; q[gg][3] = x0.w;
      q[gg][4] = y0.x; q[gg][5] = y0.y; q[gg][6] = y0.z; q[gg][7] = y0.w;
    }
  };
  // running state of the current run: maxima per head (all lanes), weight
  // sum of head hl (per lane), value sums (per lane, over its token rows)
  float M[kGroup], s_l, acc[kGroup][8];
  auto reset = [&]() {
#pragma unroll
    for (int gg = 0; gg < kGroup; ++gg) {
      M[gg] = -INFINITY;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[gg][k] = 0.0f;
    }
    s_l = 0.0f;
  };
  auto flush = [&](int u_first) {
    // sum over the lanes of one head (same lane & 3): row_ror 4 and 8, then rows
    float st = s_l;
    st += dpp_f<0x124>(st);
    st += dpp_f<0x128>(st);
    st += __shfl_xor(st, 16);
    st += __shfl_xor(st, 32);
    // merge the wave's 4 token rows (lanes l, l^16, l^32, l^48)
#pragma unroll
    for (int gg = 0; gg < kGroup; ++gg) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        acc[gg][k] += __shfl_xor(acc[gg][k], 16);
        acc[gg][k] += __shfl_xor(acc[gg][k], 32);
      }
    }
    float* pp = a.part + (int64_t)u_first * kPartStride;
    if (lane < 16) {
#pragma unroll
      for (int gg = 0; gg < kGroup; ++gg) {
        float4* o = reinterpret_cast<float4*>(pp + gg * kD + sub * 8);
        o[0] = make_float4(acc[gg][0], acc[gg][1], acc[gg][2], acc[gg][3]);
        o[1] = make_float4(acc[gg][4], acc[gg][5], acc[gg][6], acc[gg][7]);
      }
    }
    if (lane < kGroup) {
      pp[kGroup * kD + lane] = lane == 0 ? M[0] : lane == 1 ? M[1] : lane == 2 ? M[2] : M[3];
      pp[kGroup * kD + kGroup + lane] = st;
    }
  };

  int u = u_begin;
  UnitRef cur = unit_ref(a, u, u_end);
  float qs_next[kGroup][8];
  load_q(cur, qs_next);
  u32x4 bufA[8], bufB[8];
  issue_x(cur, 0, bufA);
  issue_x(cur, 1, bufB);
  int run_first = u, run_rh = cur.rh;
  reset();
  while (cur.valid) {
    const UnitRef nxt = unit_ref(a, u + 1, u_end);
    auto issue = [&](int si, u32x4 (&buf)[8]) {
      if (si < cur.len) issue_x(cur, si, buf);
      else issue_x(nxt, si - cur.len, buf);
    };
    if (cur.rh != run_rh) {  // a new (request, KV head): close the run
      flush(run_first);
      reset();
      run_first = u;
      run_rh = cur.rh;
    }
    const int n_tok = cur.n_tok, ns = cur.ns, nsk = cur.nsk;
    const bool ok = cur.ok;
    const int n_pad = ns * kStep;  // slots the steps cover
    if (!ok && lane == 0) atomicOr(a.err, GP_DEVERR_PAGE);
    float qs[kGroup][8];
#pragma unroll
    for (int gg = 0; gg < kGroup; ++gg)
#pragma unroll
      for (int k = 0; k < 8; ++k) qs[gg][k] = qs_next[gg][k];
    if (nxt.valid && nxt.rh != cur.rh) load_q(nxt, qs_next);
    float mx0 = -INFINITY, mx1 = -INFINITY;  // this lane's heads 2 b0, 2 b0 + 1

    // pass 1 step: logits of 32 tokens
    auto key_step = [&](int si, u32x4 (&kv)[8]) {
      const int c0 = si * kStep;
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
      issue(si + 2, kv);
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
      if (si != ns - 1) return;
      // end of pass 1: page maximum per head (lanes with the same bit 0 hold
      // the same heads) raises the running maximum; the running sums are
      // rescaled when it grows; then the weights exp(l - max) in place,
      // entry idx = 4 token + head, a lane's entries all of head hl
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
      bool grows = false;
#pragma unroll
      for (int gg = 0; gg < kGroup; ++gg) grows |= mh[gg] > M[gg];
      if (grows) {  // wave-uniform
        float f[kGroup];
#pragma unroll
        for (int gg = 0; gg < kGroup; ++gg) {
          const float m_new = fmaxf(M[gg], mh[gg]);
          f[gg] = exp_fast(M[gg] - m_new);  // 0 while M is -inf
          M[gg] = m_new;
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[gg][k] *= f[gg];
        }
        s_l *= hl == 0 ? f[0] : hl == 1 ? f[1] : hl == 2 ? f[2] : f[3];
      }
      wave_sync();
      const float m_l = hl == 0 ? M[0] : hl == 1 ? M[1] : hl == 2 ? M[2] : M[3];
      float* flat = &lw[0][0];
      for (int idx = lane; idx < n_pad * kGroup; idx += 64) {
        const float l = flat[idx];
        const float pv = l == -INFINITY ? 0.0f : exp_fast(l - m_l);
        flat[idx] = pv;
        s_l += pv;
      }
      wave_sync();
    };
    // pass 2 step: values of 32 tokens times their weights
    auto value_step = [&](int si, u32x4 (&vv)[8]) {
      const int c0 = (si - nsk) * kStep;
      float4 pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pr[i] = *reinterpret_cast<const float4*>(&lw[c0 + 4 * i + grp][0]);
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
      issue(si + 2, vv);
    };
    for (int si = 0; si < ns; si += 2) {
      key_step(si, bufA);
      if (si + 1 < ns) key_step(si + 1, bufB);
      else issue(si + 3, bufB);  // pad: buffer B takes the second value step
    }
    for (int si = nsk; si < cur.len; si += 2) {
      value_step(si, bufA);
      if (si + 1 < nsk + ns) value_step(si + 1, bufB);
      else issue(si + 3, bufB);  // pad: buffer B takes the next unit's second step
    }
    wave_sync();
    cur = nxt;
    ++u;
  }
  flush(run_first);
}

// ---- 3. merge -------------------------------------------------------------------
// o = sum_q e^(m_q - m) o_q / sum_q e^(m_q - m) S_q over the partials q of a
// (request, KV head), m the largest partial maximum.  The request's units
// are [U0, U0 + np); its partials sit at U0 and at every wave-range start
// inside it.
constexpr int kMergeT = 256;

__global__ __launch_bounds__(kMergeT) void k_decode_merge(DecodeArgs a, int waves) {
  __shared__ int s_idx[kMergeT];
  const int t = threadIdx.x;
  const int rh = blockIdx.x;
  const int r = rh / a.Hkv, h = rh % a.Hkv;
  const int g = t >> 6, j = t & 63;
  float* orow = a.out + ((int64_t)r * a.Hq + h * kGroup + g) * kD;
  const int N = decode_tokens(a, r);
  const int n_units = *a.n_units;
  if (N < 0 || n_units == 0) {
    orow[j] = 0.0f;
    orow[j + kD / 2] = 0.0f;
    return;
  }
  const int np = (N + kPage - 1) / kPage;
  const int R = unit_range(n_units, waves);
  const int U0 = a.page_pre[r] * a.Hkv + h * np, U1 = U0 + np;
  // partial indices: U0, then the range starts k R in (U0, U1)
  const int k0 = U0 / R + 1;
  const int nq = 1 + max(0, (U1 - 1) / R - k0 + 1);
  for (int q = t; q < nq; q += kMergeT) s_idx[q] = q == 0 ? U0 : (k0 + q - 1) * R;
  __syncthreads();
  const int nq_lds = min(nq, kMergeT);
  float m = -INFINITY;
  for (int q = 0; q < nq; ++q) {
    const int ui = q < nq_lds ? s_idx[q] : (k0 + q - 1) * R;
    m = fmaxf(m, a.part[(int64_t)ui * kPartStride + kGroup * kD + g]);
  }
  float o1 = 0.0f, o2 = 0.0f, ssum = 0.0f;
  for (int q = 0; q < nq; ++q) {
    const int ui = q < nq_lds ? s_idx[q] : (k0 + q - 1) * R;
    const float* ps = a.part + (int64_t)ui * kPartStride;
    const float mq = ps[kGroup * kD + g];
    const float f = mq == -INFINITY ? 0.0f : exp_fast(mq - m);
    o1 = __builtin_fmaf(f, ps[g * kD + j], o1);
    o2 = __builtin_fmaf(f, ps[g * kD + j + kD / 2], o2);
    ssum = __builtin_fmaf(f, ps[kGroup * kD + kGroup + g], ssum);
  }
  const float inv = ssum > 0.0f ? 1.0f / ssum : 0.0f;
  orow[j] = o1 * inv;
  orow[j + kD / 2] = o2 * inv;
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
  hipLaunchKernelGGL(k_decode_merge, dim3((unsigned)B * p.Hkv), dim3(kMergeT), 0, s, a,
                     unit_blocks * kDecWaves);
  return hipGetLastError();
}

}  // namespace gp
