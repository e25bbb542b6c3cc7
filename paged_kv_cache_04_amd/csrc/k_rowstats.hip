// A3 + A4: per-row attention distributions, per-token importance and the
// p-coverage demand D_p of both views.
// Citations are to "GrowPage: On-Demand KV Budgeting for Efficient LLM
// Reasoning Serving" (arXiv 2609.03494): §3.1 Eq. 2, §3.2 Eq. 7, §3.3 Eq. 9,
// App. E.1.
//
// One workgroup per row (request, layer, KV head).  From the 8 logits per
// token written by the scoring kernel:
//   * maxima over the historical candidates C_t = [0, N - b) and over all N
//     slots come from the per-page maxima;
//   * pass 1: exact normalisers Z = sum floor(exp(l - m) * 2^40) as uint64
//     (integer sums: any order, any split, same bits);
//   * pass 2: a = exp(l - m) * (1 / Z) per query head, the GQA mean over the
//     4 heads of each view (summed in head order), for C_t (demand) and for
//     all slots (importance); writes s = max(short, long) of the full-cache
//     distributions (Eq. 9) and the demand distributions;
//   * D_p of each view: radix select on the fp32 bit patterns (monotone for
//     non-negative values) weighted by the masses floor(abar * 2^40): four
//     8-bit digit passes find the key value at which the descending prefix
//     mass reaches p, then D_p = (count above) + ceil(remaining / mass).
#include "gp_internal.h"

namespace gp {

constexpr int kRS = 512;  // threads per row

__device__ __forceinline__ uint64_t shfl_down_u64(uint64_t v, int off) {
  const unsigned lo = __shfl_down((unsigned)v, off);
  const unsigned hi = __shfl_down((unsigned)(v >> 32), off);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const unsigned lo = __shfl_xor((unsigned)v, m);
  const unsigned hi = __shfl_xor((unsigned)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v += shfl_xor_u64(v, m);
  return v;
}

__global__ __launch_bounds__(kRS) void k_rowstats(int L, int Hkv, int b, int p_num, int p_den,
                                                  const WsHeader* __restrict__ hdr,
                                                  const int64_t* __restrict__ page_off,
                                                  const float* __restrict__ logits,
                                                  const float* __restrict__ pmax,
                                                  float* __restrict__ imp,
                                                  float* __restrict__ keys,
                                                  int32_t* __restrict__ k_short,
                                                  int32_t* __restrict__ k_long,
                                                  float* __restrict__ abar) {
  __shared__ float s_mdem[kNQ], s_mall[kNQ], s_rdem[kNQ], s_rall[kNQ];
  __shared__ uint64_t red64[kRS / 64][2 * kNQ];
  __shared__ uint32_t hcnt[256];
  __shared__ uint64_t hmass[256];
  __shared__ uint64_t s_W[2];
  __shared__ uint64_t s_above;
  __shared__ uint32_t s_cabove, s_prefix;
  if (!hdr->valid) return;
  const int LH = L * Hkv;
  const int row = blockIdx.x;
  const int r = row / LH, lh = row % LH;
  const int64_t P = page_off[r + 1] - page_off[r];
  const int64_t N = P * b, ndem = N - b;
  const int64_t row_tok = (int64_t)LH * page_off[r] * b + (int64_t)lh * N;
  const int64_t row_page = (int64_t)LH * page_off[r] + (int64_t)lh * P;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;

  if (t < kNQ) {
    float md = -INFINITY;
    for (int64_t pg = 0; pg < P - 1; ++pg) md = fmaxf(md, pmax[(row_page + pg) * kNQ + t]);
    s_mdem[t] = md;
    s_mall[t] = fmaxf(md, pmax[(row_page + P - 1) * kNQ + t]);
  }
  __syncthreads();
  float md[kNQ], ma[kNQ];
  bool same[kNQ];
#pragma unroll
  for (int q = 0; q < kNQ; ++q) {
    md[q] = s_mdem[q];
    ma[q] = s_mall[q];
    same[q] = md[q] == ma[q];
  }

  // pass 1: exact fixed-point normalisers
  uint64_t zd[kNQ], za[kNQ];
#pragma unroll
  for (int q = 0; q < kNQ; ++q) zd[q] = za[q] = 0;
  for (int64_t i = t; i < N; i += kRS) {
    const float4* lp = reinterpret_cast<const float4*>(logits + (row_tok + i) * kNQ);
    const float4 a = lp[0], c = lp[1];
    const float l[kNQ] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    const bool dem = i < ndem;
#pragma unroll
    for (int q = 0; q < kNQ; ++q) {
      const float ea = gp_exp(l[q] - ma[q]);
      za[q] += fix40(ea);
      if (dem) zd[q] += fix40(same[q] ? ea : gp_exp(l[q] - md[q]));
    }
  }
#pragma unroll
  for (int v = 0; v < 2 * kNQ; ++v) {
    const uint64_t s = wave_sum_u64(v < kNQ ? zd[v] : za[v - kNQ]);
    if (lane == 0) red64[wv][v] = s;
  }
  __syncthreads();
  if (t < 2 * kNQ) {
    uint64_t z = 0;
#pragma unroll
    for (int w = 0; w < kRS / 64; ++w) z += red64[w][t];
    const float zf = (float)z * kFixInv;
    if (t < kNQ) s_rdem[t] = ndem > 0 ? 1.0f / zf : 0.0f;
    else s_rall[t - kNQ] = 1.0f / zf;
  }
  __syncthreads();
  float rd[kNQ], ra[kNQ];
#pragma unroll
  for (int q = 0; q < kNQ; ++q) {
    rd[q] = s_rdem[q];
    ra[q] = s_rall[q];
  }

  // pass 2: distributions, importance, demand keys and their total masses
  uint64_t wsum0 = 0, wsum1 = 0;
  for (int64_t i = t; i < N; i += kRS) {
    const float4* lp = reinterpret_cast<const float4*>(logits + (row_tok + i) * kNQ);
    const float4 a = lp[0], c = lp[1];
    const float l[kNQ] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    const bool dem = i < ndem;
    float aa[2], ad[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      float sa = 0.0f, sd = 0.0f;
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        const int q = x * kGroup + g;
        const float ea = gp_exp(l[q] - ma[q]);
        sa = sa + ea * ra[q];
        if (dem) {
          const float ed = same[q] ? ea : gp_exp(l[q] - md[q]);
          sd = sd + ed * rd[q];
        }
      }
      aa[x] = sa / (float)kGroup;
      ad[x] = sd / (float)kGroup;
    }
    imp[row_tok + i] = fmaxf(aa[0], aa[1]);
    if (abar) reinterpret_cast<float2*>(abar)[row_tok + i] = make_float2(aa[0], aa[1]);
    if (dem) {
      reinterpret_cast<float2*>(keys)[row_tok + i] = make_float2(ad[0], ad[1]);
      wsum0 += fix40(ad[0]);
      wsum1 += fix40(ad[1]);
    }
  }
  wsum0 = wave_sum_u64(wsum0);
  wsum1 = wave_sum_u64(wsum1);
  if (lane == 0) {
    red64[wv][0] = wsum0;
    red64[wv][1] = wsum1;
  }
  __syncthreads();
  if (t < 2) {
    uint64_t s = 0;
#pragma unroll
    for (int w = 0; w < kRS / 64; ++w) s += red64[w][t];
    s_W[t] = s;
  }
  __syncthreads();

  // D_p of each view by mass-weighted radix select over C_t
  for (int x = 0; x < 2; ++x) {
    int32_t* out = x == 0 ? k_short : k_long;
    if (ndem <= 0) {
      if (t == 0) out[row] = 0;
      continue;
    }
    const uint64_t target = s_W[x] * (uint64_t)p_num;
    uint32_t prefix = 0, mask = 0, c_above = 0;
    uint64_t m_above = 0;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int k = t; k < 256; k += kRS) {
        hcnt[k] = 0;
        hmass[k] = 0;
      }
      __syncthreads();
      for (int64_t i = t; i < ndem; i += kRS) {
        const uint32_t key = __float_as_uint(keys[(row_tok + i) * 2 + x]);
        if ((key & mask) == prefix) {
          const uint32_t dig = (key >> shift) & 255u;
          atomicAdd(&hcnt[dig], 1u);
          atomicAdd((unsigned long long*)&hmass[dig], (unsigned long long)fix40(__uint_as_float(key)));
        }
      }
      __syncthreads();
      if (wv == 0) {
        uint64_t m[4];
        uint32_t c[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          m[u] = hmass[4 * lane + u];
          c[u] = hcnt[4 * lane + u];
        }
        const uint64_t lm = m[0] + m[1] + m[2] + m[3];
        const uint32_t lc = c[0] + c[1] + c[2] + c[3];
        uint64_t sm = lm;
        uint32_t sc = lc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint64_t vm = shfl_down_u64(sm, off);
          const uint32_t vc = __shfl_down(sc, off);
          if (lane + off < 64) {
            sm += vm;
            sc += vc;
          }
        }
        uint64_t cum = m_above + (sm - lm);
        uint32_t ccum = c_above + (sc - lc);
        int best = -1;
        uint64_t best_m = 0;
        uint32_t best_c = 0;
#pragma unroll
        for (int u = 3; u >= 0; --u) {
          const uint64_t before = cum;
          const uint32_t cbefore = ccum;
          cum += m[u];
          ccum += c[u];
          if (best < 0 && cum * (uint64_t)p_den >= target) {
            best = 4 * lane + u;
            best_m = before;
            best_c = cbefore;
          }
        }
        const unsigned long long ok = __ballot(best >= 0);
        const int hl = 63 - __clzll(ok);
        if (lane == hl) {
          s_prefix = prefix | ((uint32_t)best << shift);
          s_above = best_m;
          s_cabove = best_c;
        }
      }
      __syncthreads();
      prefix = s_prefix;
      m_above = s_above;
      c_above = s_cabove;
      mask |= 255u << shift;
      __syncthreads();
    }
    if (t == 0) {
      const uint64_t wt = fix40(__uint_as_float(prefix));
      const uint64_t need = target - m_above * (uint64_t)p_den;
      const uint64_t den = wt * (uint64_t)p_den;
      out[row] = (int32_t)(c_above + (need + den - 1) / den);
    }
  }
}

hipError_t launch_rowstats(const Params& p, const WsLayout& w, int B, void* ws,
                           int32_t* k_short, int32_t* k_long, float* abar, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  hipLaunchKernelGGL(k_rowstats, dim3((unsigned)w.rows), dim3(kRS), 0, s, p.L, p.Hkv, p.b,
                     p.p_num, p.p_den, reinterpret_cast<const WsHeader*>(base + w.header),
                     reinterpret_cast<const int64_t*>(base + w.page_off),
                     reinterpret_cast<const float*>(base + w.logits),
                     reinterpret_cast<const float*>(base + w.pmax),
                     reinterpret_cast<float*>(base + w.imp), reinterpret_cast<float*>(base + w.keys),
                     k_short, k_long, abar);
  (void)B;
  return hipGetLastError();
}

}  // namespace gp
