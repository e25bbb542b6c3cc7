// A2: score every cached key of every (layer, KV head) row against the 8
// calibrated summary queries of that KV head (2 views x 4 GQA query heads).
// Citations are to "GrowPage: On-Demand KV Budgeting for Efficient LLM
// Reasoning Serving" (arXiv 2609.03494): §3.2 "Attention-demand trend",
// App. E.1 "Demand estimation at capacity boundaries".
//
// One workgroup per (request, page, layer, KV head) tile: the 256 keys of a
// page for one KV head are a contiguous 64 KB block of the pool, so each wave
// streams 16 KB with 16-byte coalesced loads, stages it in LDS (rows padded
// to 272 B so the per-lane row reads hit distinct banks), and each lane then
// scores one key: 8 serial fmaf chains over j = 0..127 in index order (the
// fp32 arithmetic contract shared with the CPU reference).  The summary
// queries are wave-uniform and come through scalar loads.  Outputs: 8 fp32
// logits per token (32 B, token-major) and the per-page maxima.
#include "gp_internal.h"

namespace gp {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowPad = 272;               // bytes per staged key row
constexpr int kWaveStage = 64 * kRowPad;   // bytes per wave

__global__ __launch_bounds__(256) void k_score(const uint16_t* __restrict__ k_pool, int pool_pages,
                                               const int32_t* __restrict__ block_table,
                                               int max_pages, int L, int Hkv, int B,
                                               const WsHeader* __restrict__ hdr,
                                               const int64_t* __restrict__ page_off,
                                               const float* __restrict__ qhat,
                                               float* __restrict__ logits,
                                               float* __restrict__ pmax,
                                               int32_t* __restrict__ err) {
  __shared__ __attribute__((aligned(16))) unsigned char stage[4 * kWaveStage];
  __shared__ float red[4][kNQ];
  if (!hdr->valid) return;
  const int64_t LH = (int64_t)L * Hkv;
  const int64_t tile = blockIdx.x;
  // request r: largest r with LH * page_off[r] <= tile
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (LH * page_off[mid] <= tile) lo = mid; else hi = mid;
  }
  const int r = lo;
  const int64_t P = page_off[r + 1] - page_off[r];
  const int64_t local = tile - LH * page_off[r];
  const int lh = (int)(local / P);
  const int pg = (int)(local % P);
  const int l = lh / Hkv, h = lh % Hkv;
  const int page = block_table[(int64_t)r * max_pages + pg];
  const bool bad = page < 0 || page >= pool_pages;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;

  unsigned char* my = stage + w * kWaveStage;
  if (!bad) {
    const u32x4* src = reinterpret_cast<const u32x4*>(
        k_pool + ((((int64_t)l * pool_pages + page) * Hkv + h) * kPage) * kD) + w * 1024;
    u32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_nontemporal_load(src + i * 64 + lane);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = i * 64 + lane;  // 16-byte element index within the wave's 16 KB
      *reinterpret_cast<u32x4*>(my + (e >> 4) * kRowPad + (e & 15) * 16) = v[i];
    }
  } else if (threadIdx.x == 0) {
    atomicOr(err, GP_DEVERR_PAGE);
  }
  __syncthreads();

  float acc[kNQ];
#pragma unroll
  for (int qi = 0; qi < kNQ; ++qi) acc[qi] = 0.0f;
  if (!bad) {
    const float* __restrict__ q = qhat + ((int64_t)r * LH + lh) * (kNQ * kD);
    const unsigned char* rowp = my + lane * kRowPad;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(rowp + c * 16);
      float k[8];
      k[0] = bf16_lo(kv.x); k[1] = bf16_hi(kv.x);
      k[2] = bf16_lo(kv.y); k[3] = bf16_hi(kv.y);
      k[4] = bf16_lo(kv.z); k[5] = bf16_hi(kv.z);
      k[6] = bf16_lo(kv.w); k[7] = bf16_hi(kv.w);
      const float* qc = q + c * 64;
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int qi = 0; qi < kNQ; ++qi) acc[qi] = __builtin_fmaf(qc[qi * 8 + e], k[e], acc[qi]);
    }
  }

  const int64_t row_tok = LH * page_off[r] * kPage + (int64_t)lh * P * kPage;
  const int64_t tok = row_tok + (int64_t)pg * kPage + w * 64 + lane;
  float4* out = reinterpret_cast<float4*>(logits + tok * kNQ);
  out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);

#pragma unroll
  for (int qi = 0; qi < kNQ; ++qi) {
    float m = acc[qi];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) red[w][qi] = m;
  }
  __syncthreads();
  if (threadIdx.x < kNQ) {
    const int qi = threadIdx.x;
    const float m = fmaxf(fmaxf(red[0][qi], red[1][qi]), fmaxf(red[2][qi], red[3][qi]));
    const int64_t row_page = LH * page_off[r] + (int64_t)lh * P;
    pmax[(row_page + pg) * kNQ + qi] = m;
  }
}

hipError_t launch_score(const Params& p, const WsLayout& w, const uint16_t* k_pool,
                        int pool_pages, const int32_t* block_table, int max_pages, int B,
                        void* ws, int32_t* err, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  hipLaunchKernelGGL(k_score, dim3((unsigned)w.row_pages), dim3(256), 0, s, k_pool, pool_pages,
                     block_table, max_pages, p.L, p.Hkv, B,
                     reinterpret_cast<const WsHeader*>(base + w.header),
                     reinterpret_cast<const int64_t*>(base + w.page_off),
                     reinterpret_cast<const float*>(base + w.qhat),
                     reinterpret_cast<float*>(base + w.logits),
                     reinterpret_cast<float*>(base + w.pmax), err);
  return hipGetLastError();
}

}  // namespace gp
