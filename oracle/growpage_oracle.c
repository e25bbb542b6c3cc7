/*
 * GrowPage capacity-boundary event: plain, serial CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this file.  It shares no
 * code, header, table or constant with the HIP library: every constant below
 * is written here from its definition.
 *
 * Citations are to "GrowPage: On-Demand KV Budgeting for Efficient LLM
 * Reasoning Serving" (arXiv 2609.03494), by section / equation / appendix.
 *
 * Precision.  The pages fix no precision.  Every step that decides an
 * integer (D_p, the grow/compress decision, the kept set) is taken here in
 * fp32, the precision of the GPU path, following one written arithmetic
 * contract so that both sides reach identical bits:
 *   - every product-sum is an explicit fmaf in index order (no contraction:
 *     this file is built with -ffp-contract=off, no fast-math);
 *   - exp is orc_exp below (Cody-Waite reduction + degree-6 Taylor series);
 *   - softmax normalisers are exact integer sums of floor(e * 2^40);
 *   - probability masses for D_p are floor(abar * 2^40), compared exactly.
 * The fp64 textbook reading of the same steps lives in reference.py.
 *
 * Each function names the passage it follows and the pins that check it
 * (tests/test_oracle_*.py).  Nothing here is blocked, fused or reordered
 * beyond what the definition states: loops run in index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_GROW 1
#define ORC_COMPRESS 0
#define ORC_SHRINK 2

static float bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint32_t float_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

static float bits_float(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* ------------------------------------------------------------------------
 * exp for x <= 0 (softmax after subtracting the maximum).
 * Method: Cody & Waite argument reduction x = n ln2 + r with ln2 split in a
 * 16-bit head and an fp32 tail (so n*head is exact for |n| < 256), then the
 * Taylor series of e^r to degree 6 in Horner form, then scaling by 2^n.
 * Results below 2^-100 are returned as 0 (n < -100), which keeps every
 * later quantity a normal fp32 number.
 * Pins: within 3 ulp of the correctly rounded exp over [-69, 0]; exp(0) = 1.
 * ---------------------------------------------------------------------- */
float orc_exp(float x) {
  const float log2e = 0x1.715476p+0f;  /* fp32(1/ln 2) */
  const float ln2_head = 0x1.62e4p-1f; /* ln 2 rounded to 16 bits */
  const float ln2_tail = 0x1.7f7d1cp-20f; /* fp32(ln 2 - head) */
  float t = x * log2e;
  float n = rintf(t);
  if (n < -100.0f) return 0.0f;
  float r = fmaf(-n, ln2_head, x);
  r = fmaf(-n, ln2_tail, r);
  float p = 1.0f / 720.0f;
  p = fmaf(p, r, 1.0f / 120.0f);
  p = fmaf(p, r, 1.0f / 24.0f);
  p = fmaf(p, r, 1.0f / 6.0f);
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  int ni = (int)n;
  float scale = bits_float((uint32_t)(127 + ni) << 23);
  return p * scale;
}

/* ------------------------------------------------------------------------
 * Dual-timescale query summaries (§3.2 Eq. 6; Appendix E.1 "Initialization
 * and online update").  The pages write qbar_t = beta qbar_{t-1} +
 * (1 - beta) q_t with beta_S = 0.9, beta_L = 0.999.  Here alpha = 1 - beta is
 * the weight of the new query, given as an fp32 value, and the update is
 * written in the algebraically identical form
 *     qbar' = qbar + alpha (q - qbar) = fmaf(alpha, q - qbar, qbar),
 * which keeps a constant stream exactly constant (the two-product form
 * beta*qbar + alpha*q drifts because fp32 alpha + fp32 beta != 1).
 * On the first decoding step of a slot both summaries are set to q.
 * State layout is the pages' query-state pool, Appendix E.1 Eq. 11:
 *     state[L][M][2][Hq][d], index 0 = short (S), 1 = long (L).
 * q is [B][L][Hq][d], the normalised pre-RoPE query.
 * Pins: geometric closed form (fp64), constant stream stays constant.
 * ---------------------------------------------------------------------- */
void orc_ema(float* state, const float* q, const int32_t* slot,
             const uint8_t* first_step, int B, int L, int M, int Hq, int d,
             float alpha_short, float alpha_long) {
  const float alpha[2] = {alpha_short, alpha_long};
  for (int b = 0; b < B; ++b)
    for (int l = 0; l < L; ++l)
      for (int x = 0; x < 2; ++x)
        for (int h = 0; h < Hq; ++h)
          for (int j = 0; j < d; ++j) {
            size_t si = ((((size_t)l * M + slot[b]) * 2 + x) * Hq + h) * d + j;
            size_t qi = (((size_t)b * L + l) * Hq + h) * d + j;
            if (first_step[b]) {
              state[si] = q[qi];
            } else {
              float diff = q[qi] - state[si];
              state[si] = fmaf(alpha[x], diff, state[si]);
            }
          }
}

/* ------------------------------------------------------------------------
 * Calibrated, rotated summaries for one request (Appendix E.1 Eq. 12 and the
 * paragraph after it; §3.2 "calibrate their per-head RMS scales and apply
 * RoPE at the current position").
 *   gamma = RMS(q_t) / RMS(qbar) = sqrt(ss(q_t) / ss(qbar)) (the 1/d cancels;
 *           gamma = 0 when ss(qbar) = 0); sums of squares are serial fmaf.
 *   qtilde = gamma * qbar.
 *   Rotary embedding in the rotate-half pairing (j, j + d/2) with the
 *   (cos, sin) row of the current position:
 *     y_j       = fmaf(x_j,       c_j, -(x_{j+d/2} * s_j))
 *     y_{j+d/2} = fmaf(x_{j+d/2}, c_j,   x_j       * s_j)
 *   then the attention scale 1/sqrt(d) (fp32 of 1.0f / sqrtf(d)) is applied.
 * rope_row is [d]: cos for the d/2 frequencies, then sin.
 * qcur is [L][Hq][d]; output qhat is [L][2][Hq][d].
 * Pins: RMS(qtilde) = RMS(q_t); identity at cos=1, sin=0; norm preserved.
 * ---------------------------------------------------------------------- */
void orc_qhat(const float* state, int M, int slot, const float* qcur,
              const float* rope_row, int L, int Hq, int d, float* qhat) {
  const int half = d / 2;
  const float scale = 1.0f / sqrtf((float)d);
  float* tmp = (float*)malloc(sizeof(float) * (size_t)d);
  for (int l = 0; l < L; ++l)
    for (int h = 0; h < Hq; ++h) {
      const float* qt = qcur + ((size_t)l * Hq + h) * d;
      float ssq = 0.0f;
      for (int j = 0; j < d; ++j) ssq = fmaf(qt[j], qt[j], ssq);
      for (int x = 0; x < 2; ++x) {
        const float* qb = state + ((((size_t)l * M + slot) * 2 + x) * Hq + h) * d;
        float ssx = 0.0f;
        for (int j = 0; j < d; ++j) ssx = fmaf(qb[j], qb[j], ssx);
        float gamma = ssx > 0.0f ? sqrtf(ssq / ssx) : 0.0f;
        for (int j = 0; j < d; ++j) tmp[j] = gamma * qb[j];
        float* out = qhat + (((size_t)l * 2 + x) * Hq + h) * d;
        for (int j = 0; j < half; ++j) {
          float c = rope_row[j], s = rope_row[half + j];
          float y1 = fmaf(tmp[j], c, -(tmp[j + half] * s));
          float y2 = fmaf(tmp[j + half], c, tmp[j] * s);
          out[j] = y1 * scale;
          out[j + half] = y2 * scale;
        }
      }
    }
  free(tmp);
}

/* ------------------------------------------------------------------------
 * p-coverage demand D_p (§3.1 Eq. 2; §3.2 Eq. 7):
 *   D_p(a) = min{ k : sum of the k largest weights >= p }.
 * The weights are fp32 values abar_i; each is given the mass
 * w_i = floor(abar_i * 2^40) (exact: abar <= 1), the total W = sum w_i, and
 * the test "mass >= p" is read as p_den * (top-k mass) >= p_num * W, exact
 * in integers (p = p_num / p_den).  Steps in the pages' order: sort
 * descending, prefix-sum, first k that reaches the coverage.
 * v is read with a stride (in floats) so a column of [n][2] can be passed.
 * Pins: hand-made distributions (tests/golden/dp_cases.json), Theorem 3.1 by
 * brute force over all subsets for n <= 12.
 * ---------------------------------------------------------------------- */
static int cmp_u64_desc(const void* a, const void* b) {
  uint64_t x = *(const uint64_t*)a, y = *(const uint64_t*)b;
  return (x < y) - (x > y);
}

int orc_dp(const float* v, int stride, int n, int p_num, int p_den) {
  if (n <= 0) return 0;
  uint64_t* w = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)n);
  unsigned __int128 total = 0;
  for (int i = 0; i < n; ++i) {
    w[i] = (uint64_t)(v[(size_t)i * stride] * 0x1p40f);
    total += w[i];
  }
  qsort(w, (size_t)n, sizeof(uint64_t), cmp_u64_desc);
  unsigned __int128 need = total * (unsigned)p_num, run = 0;
  int k = n;
  for (int i = 0; i < n; ++i) {
    run += w[i];
    if (run * (unsigned)p_den >= need) { k = i + 1; break; }
  }
  free(w);
  return k;
}

/* ------------------------------------------------------------------------
 * One row = one (layer, KV head) of one request at a capacity boundary.
 * keys: [N][d] bf16 in logical slot order; N = P * b.
 * qh:   [2][G][d] calibrated rotated summaries of the G query heads that
 *       share this KV head (GQA grouping kept, Appendix E.1), short first.
 * Steps:
 *  logits l[x][g][i] = sum_j qh[x][g][j] * k_i[j], serial fmaf from j = 0.
 *  Demand distribution (§3.2 "historical candidate set ... excludes the most
 *  recent KV block"; Appendix E.1: 256 tokens): softmax over C_t = [0, N-b).
 *  Full distribution (used by Eq. 9): softmax over all N slots.
 *  Each softmax subtracts its own maximum, e = orc_exp(l - m),
 *  Z = (float)(sum floor(e * 2^40)) * 2^-40, a = e * (1.0f / Z).
 *  GQA: abar = (a_0 + a_1 + ... + a_{G-1}) / G, summed in head order: one
 *  distribution per KV head, as Eq. 7 and Eq. 9 are indexed.
 *  D_p of abar over C_t for x in {S, L} (Eq. 7).
 * Outputs (each may be NULL):
 *   logits [2][G][N], abar_all [N][2], abar_dem [N-b][2], dp [2].
 * ---------------------------------------------------------------------- */
void orc_row(const uint16_t* keys, int N, int d, int b, const float* qh,
             int G, int p_num, int p_den, float* logits, float* abar_all,
             float* abar_dem, int32_t* dp) {
  const int ndem = N - b > 0 ? N - b : 0;
  const int nq = 2 * G;
  float* lg = (float*)malloc(sizeof(float) * (size_t)nq * N);
  float* kf = (float*)malloc(sizeof(float) * (size_t)d);
  for (int i = 0; i < N; ++i) {
    for (int j = 0; j < d; ++j) kf[j] = bf16_value(keys[(size_t)i * d + j]);
    for (int q = 0; q < nq; ++q) {
      const float* qv = qh + (size_t)q * d;
      float acc = 0.0f;
      for (int j = 0; j < d; ++j) acc = fmaf(qv[j], kf[j], acc);
      lg[(size_t)q * N + i] = acc;
    }
  }
  if (logits) memcpy(logits, lg, sizeof(float) * (size_t)nq * N);

  float* rho_dem = (float*)malloc(sizeof(float) * nq);
  float* rho_all = (float*)malloc(sizeof(float) * nq);
  float* m_dem = (float*)malloc(sizeof(float) * nq);
  float* m_all = (float*)malloc(sizeof(float) * nq);
  for (int q = 0; q < nq; ++q) {
    const float* row = lg + (size_t)q * N;
    float md = -INFINITY, ma;
    for (int i = 0; i < ndem; ++i) md = fmaxf(md, row[i]);
    ma = md;
    for (int i = ndem; i < N; ++i) ma = fmaxf(ma, row[i]);
    m_dem[q] = md;
    m_all[q] = ma;
    uint64_t zd = 0, za = 0;
    for (int i = 0; i < ndem; ++i) zd += (uint64_t)(orc_exp(row[i] - md) * 0x1p40f);
    for (int i = 0; i < N; ++i) za += (uint64_t)(orc_exp(row[i] - ma) * 0x1p40f);
    rho_dem[q] = ndem > 0 ? 1.0f / ((float)zd * 0x1p-40f) : 0.0f;
    rho_all[q] = 1.0f / ((float)za * 0x1p-40f);
  }

  float* ad = (float*)malloc(sizeof(float) * (size_t)(ndem > 0 ? ndem : 1) * 2);
  for (int i = 0; i < N; ++i)
    for (int x = 0; x < 2; ++x) {
      float sum_all = 0.0f, sum_dem = 0.0f;
      for (int g = 0; g < G; ++g) {
        int q = x * G + g;
        float l = lg[(size_t)q * N + i];
        sum_all = sum_all + orc_exp(l - m_all[q]) * rho_all[q];
        if (i < ndem) sum_dem = sum_dem + orc_exp(l - m_dem[q]) * rho_dem[q];
      }
      if (abar_all) abar_all[(size_t)i * 2 + x] = sum_all / (float)G;
      if (i < ndem) ad[(size_t)i * 2 + x] = sum_dem / (float)G;
    }
  if (abar_dem) memcpy(abar_dem, ad, sizeof(float) * (size_t)ndem * 2);
  if (dp) {
    dp[0] = orc_dp(ad + 0, 2, ndem, p_num, p_den);
    dp[1] = orc_dp(ad + 1, 2, ndem, p_num, p_den);
  }
  free(ad);
  free(rho_dem);
  free(rho_all);
  free(m_dem);
  free(m_all);
  free(kf);
  free(lg);
}

/* ------------------------------------------------------------------------
 * Request-level trend and decision (§3.2 Eq. 8 and the threshold rule).
 * r^x = mean over the n_rows (layer, KV head) pairs of K^x / |C_t|,
 * Delta = r^S - r^L.  Written as one quotient:
 *   diff  = sum K^S - sum K^L                 (exact int64)
 *   Delta = (double)diff / ((double)n_rows * (double)|C_t|)
 * Grow iff Delta > tau, otherwise Compress & Hold.  |C_t| <= 0 (a request of
 * one page) has no historical candidates: Delta = 0 and the request grows.
 * Returns ORC_GROW or ORC_COMPRESS.
 * ---------------------------------------------------------------------- */
int orc_decide(const int32_t* ks, const int32_t* kl, int n_rows,
               int64_t card_c, double tau, int64_t* diff_out,
               double* delta_out) {
  int64_t diff = 0;
  for (int i = 0; i < n_rows; ++i) diff += (int64_t)ks[i] - (int64_t)kl[i];
  double delta = 0.0;
  int grow;
  if (card_c <= 0) {
    grow = 1;
  } else {
    delta = (double)diff / ((double)n_rows * (double)card_c);
    grow = delta > tau;
  }
  if (diff_out) *diff_out = diff;
  if (delta_out) *delta_out = delta;
  return grow ? ORC_GROW : ORC_COMPRESS;
}

/* ------------------------------------------------------------------------
 * The three-way GrowPage-Shrink rule (Appendix H.1 Eq. 13), on the same
 * Delta as orc_decide:
 *   Delta > tau                    -> Grow by One Page
 *   shrink_tau <= Delta <= tau     -> Compress & Hold
 *   Delta < shrink_tau             -> Shrink, unless the capacity left after
 *                                     it, (P - 1) b, would fall below
 *                                     min_tokens, or the request holds fewer
 *                                     than 3 pages (then Compress & Hold):
 *                                     Shrink keeps (P - 2) b slots including
 *                                     the recent window, so Eq. 10's budget
 *                                     (P - 2) b - R is negative below 3.
 * Shrink drops two pages worth of slots and returns one page to the pool
 * (orc_select_pages with 2 pages, orc_return_pages).  A request of one page
 * grows, as in orc_decide.
 * Pins: the three regions, both boundaries (Delta = shrink_tau and
 * Delta = tau are Compress & Hold), the capacity floor.
 * ---------------------------------------------------------------------- */
int orc_decide_shrink(const int32_t* ks, const int32_t* kl, int n_rows,
                      int64_t card_c, int num_pages, int b, double tau,
                      double shrink_tau, int min_tokens, int64_t* diff_out,
                      double* delta_out) {
  double delta = 0.0;
  const int base = orc_decide(ks, kl, n_rows, card_c, tau, diff_out, &delta);
  if (delta_out) *delta_out = delta;
  if (base == ORC_GROW) return ORC_GROW;
  if (delta < shrink_tau && num_pages >= 3 && (int64_t)(num_pages - 1) * b >= min_tokens)
    return ORC_SHRINK;
  return ORC_COMPRESS;
}

/* ------------------------------------------------------------------------
 * Grow by One Page with fallback (§3.3 "Grow by One Page"; §4.2 "Scheduler-
 * Aware Page Allocation and Fallback"; Appendix H.2 defines a fallback).
 * Requests are served in index order.  A growing request takes the page on
 * top of the free stack (free_stack[free_count - 1]) while more than
 * `reserve` pages are free and its block table has room, appends it to its
 * block table and increments its page count.  Otherwise it falls back to
 * Compress & Hold.  action[r] = 1 grown, 0 compress (incl. fallback); a
 * Shrink decision (orc_decide_shrink) passes through as action 2.
 * counters: [0] pages granted, [1] compress actions, [2] fallbacks.
 * ---------------------------------------------------------------------- */
void orc_grow(const int8_t* decision, int B, int32_t* block_table,
              int max_pages, int32_t* num_pages, const int32_t* free_stack,
              int32_t* free_count, int reserve, int8_t* action,
              int64_t* counters) {
  for (int r = 0; r < B; ++r) {
    if (decision[r] == ORC_GROW) {
      if (*free_count > reserve && num_pages[r] < max_pages) {
        int32_t page = free_stack[*free_count - 1];
        *free_count -= 1;
        block_table[(size_t)r * max_pages + num_pages[r]] = page;
        num_pages[r] += 1;
        action[r] = 1;
        counters[0] += 1;
      } else {
        action[r] = 0;
        counters[1] += 1;
        counters[2] += 1;
      }
    } else if (decision[r] == ORC_SHRINK) {
      action[r] = ORC_SHRINK;  /* needs no page; orc_return_pages frees one */
    } else {
      action[r] = 0;
      counters[1] += 1;
    }
  }
}

/* ------------------------------------------------------------------------
 * Compress & Hold selection for one row (§3.3 Eq. 9 and Eq. 10).
 * s_i = max(abar^S_i, abar^L_i) over the full-cache distributions (Eq. 9).
 * Candidates C = [0, N - R): the R most recent slots are protected (window
 * mask, §3.3 and §5.1: 16 tokens).  Blocks B_j = C intersected with logical
 * page j.  Order: larger s first; equal s, larger slot (newer token) first.
 *   S_loc = union over j of the top-min(k_loc, |B_j|) of B_j;
 *   K_t   = (P - m) b - R  (m pages of slots are freed: 1 for Compress &
 *           Hold, 2 for Shrink; orc_select is m = 1);
 *   S     = S_loc plus the top-(K_t - |S_loc|) of C \ S_loc;
 *   kept  = S plus the window.  |kept| = (P - m) b.
 * abar_all is [N][2]; keep is [N] (1 kept, 0 dropped).
 * Returns 0, or -1 when |S_loc| > K_t (the quota cannot fit the budget).
 * Pins: count, window, per-block quota, dominance of picks over drops,
 * equality with a plain sorted top-K when k_loc = 0.
 * ---------------------------------------------------------------------- */
typedef struct {
  float s;
  int slot;
} orc_cand;

/* larger s first; equal s, larger slot (newer token) first */
static int cmp_cand_desc(const void* a, const void* b) {
  const orc_cand* x = (const orc_cand*)a;
  const orc_cand* y = (const orc_cand*)b;
  if (x->s != y->s) return x->s > y->s ? -1 : 1;
  return x->slot > y->slot ? -1 : (x->slot < y->slot);
}

int orc_select_pages(const float* abar_all, int N, int b, int R, int k_loc,
                     int freed_pages, uint8_t* keep) {
  const int P = N / b;
  const int nc = N - R;
  const int kt = (P - freed_pages) * b - R;
  float* s = (float*)malloc(sizeof(float) * (size_t)N);
  for (int i = 0; i < N; ++i) s[i] = fmaxf(abar_all[(size_t)i * 2], abar_all[(size_t)i * 2 + 1]);
  orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)(nc > 0 ? nc : 1));
  memset(keep, 0, (size_t)N);
  int nloc = 0;
  for (int j = 0; j * b < nc; ++j) {
    int lo = j * b, hi = (j + 1) * b < nc ? (j + 1) * b : nc, n = 0;
    for (int i = lo; i < hi; ++i) {
      c[n].s = s[i];
      c[n].slot = i;
      ++n;
    }
    qsort(c, (size_t)n, sizeof(orc_cand), cmp_cand_desc);
    int take = k_loc < n ? k_loc : n;
    for (int t = 0; t < take; ++t) keep[c[t].slot] = 1;
    nloc += take;
  }
  if (nloc > kt) {
    free(c);
    free(s);
    return -1;
  }
  int n = 0;
  for (int i = 0; i < nc; ++i)
    if (!keep[i]) {
      c[n].s = s[i];
      c[n].slot = i;
      ++n;
    }
  qsort(c, (size_t)n, sizeof(orc_cand), cmp_cand_desc);
  for (int t = 0; t < kt - nloc && t < n; ++t) keep[c[t].slot] = 1;
  for (int i = nc; i < N; ++i) keep[i] = 1;
  free(c);
  free(s);
  return 0;
}

int orc_select(const float* abar_all, int N, int b, int R, int k_loc,
               uint8_t* keep) {
  return orc_select_pages(abar_all, N, b, R, k_loc, 1, keep);
}

/* ------------------------------------------------------------------------
 * Page return of Shrink (Appendix H.1): after the two-page compaction a
 * shrinking request keeps its first P - 1 pages; the last one goes back to
 * the global pool.  Requests are served in index order, each pushing its
 * page on top of the free stack (so a later Grow takes the most recently
 * returned page first); the block-table entry is cleared to -1 and P
 * decreases by one.  Requests with fewer than 3 pages are left alone.  With
 * reference counts (refcount != NULL, Appendix E.2) a last page that other
 * requests still reference is not pushed: the request only drops its
 * reference (refcount - 1).  Returns the number of pages pushed.
 * Pins: pool arithmetic and order, shared last pages.
 * ---------------------------------------------------------------------- */
int orc_return_pages(const int8_t* action, int B, int32_t* block_table,
                     int max_pages, int32_t* num_pages, int32_t* free_stack,
                     int32_t* free_count, int32_t* refcount) {
  int n = 0;
  for (int r = 0; r < B; ++r) {
    if (action[r] != ORC_SHRINK || num_pages[r] < 3) continue;
    const size_t at = (size_t)r * max_pages + (num_pages[r] - 1);
    const int32_t page = block_table[at];
    if (refcount && refcount[page] > 1) {
      refcount[page] -= 1;
    } else {
      free_stack[*free_count] = page;
      *free_count += 1;
      if (refcount) refcount[page] = 0;
      ++n;
    }
    block_table[at] = -1;
    num_pages[r] -= 1;
  }
  return n;
}

/* ------------------------------------------------------------------------
 * Prefix-cache-aware compression (Appendix E.2): a page referenced by more
 * than one request (refcount > 1) is never written by a request's
 * compression.  Each compressing request (action Compress & Hold or
 * Shrink) gets a new target page for every shared page it keeps: pages
 * 0 .. P-1 for Compress & Hold (the last page's slots are written by later
 * decoding), 0 .. P-2 for Shrink (its last page is released by
 * orc_return_pages).  Requests are served in index order from the top of
 * the free stack; a request whose pages cannot all be allocated, and every
 * later request that needs any, is not compressed (ok[r] = 0, its action
 * left to the caller: it is skipped).  target[r][i] = new page, or -1 to
 * keep page i.  Returns the number of pages allocated.
 * Pins: allocation order and counts, the all-or-nothing prefix rule.
 * ---------------------------------------------------------------------- */
int orc_share_plan(const int8_t* action, int B, const int32_t* block_table,
                   int max_pages, const int32_t* num_pages, const int32_t* refcount,
                   const int32_t* free_stack, int32_t* free_count, int32_t* target,
                   uint8_t* ok) {
  int used = 0;
  int blocked = 0;
  for (int r = 0; r < B; ++r) {
    for (int i = 0; i < max_pages; ++i) target[(size_t)r * max_pages + i] = -1;
    ok[r] = 1;
    const int m = action[r] == ORC_COMPRESS ? 1 : (action[r] == ORC_SHRINK ? 2 : 0);
    if (m == 0 || num_pages[r] < m + 1) continue;
    const int keep_pages = m == 1 ? num_pages[r] : num_pages[r] - 1;
    int need = 0;
    for (int i = 0; i < keep_pages; ++i)
      need += refcount[block_table[(size_t)r * max_pages + i]] > 1;
    if (need == 0) continue;
    if (blocked || used + need > *free_count) {
      blocked = 1;
      ok[r] = 0;
      continue;
    }
    for (int i = 0; i < keep_pages; ++i)
      if (refcount[block_table[(size_t)r * max_pages + i]] > 1)
        target[(size_t)r * max_pages + i] = free_stack[*free_count - 1 - used++];
  }
  *free_count -= used;
  return used;
}

/* After the compaction of the event: every replaced page of a served request
 * is swapped in its block table for its target; the request drops its
 * reference to the old page (refcount - 1) and owns the new one
 * (refcount 1).  Appendix E.2. */
void orc_share_release(int B, int32_t* block_table, int max_pages, const int32_t* target,
                       const uint8_t* ok, int32_t* refcount) {
  for (int r = 0; r < B; ++r) {
    if (!ok[r]) continue;
    for (int i = 0; i < max_pages; ++i) {
      const int32_t t = target[(size_t)r * max_pages + i];
      if (t < 0) continue;
      const size_t at = (size_t)r * max_pages + i;
      refcount[block_table[at]] -= 1;
      refcount[t] = 1;
      block_table[at] = t;
    }
  }
}

/* ------------------------------------------------------------------------
 * Compaction (§3.3 "compacted within the existing physical-page allocation";
 * §4.2; Appendix E.2: at most (P - 1) b occupied slots).  The kept rows, in
 * ascending slot order, are written to slots 0, 1, ... of the same row.
 * Slots at and beyond the kept count are left as they were.
 * rows: [N][width] 16-bit elements (a K or V row chain in logical order).
 * Returns the kept count.  Pins: equals a numpy gather of the kept slots.
 * ---------------------------------------------------------------------- */
int orc_compact(uint16_t* rows, const uint8_t* keep, int N, int width) {
  uint16_t* tmp = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)N * width);
  int j = 0;
  for (int i = 0; i < N; ++i)
    if (keep[i]) {
      memcpy(tmp + (size_t)j * width, rows + (size_t)i * width, sizeof(uint16_t) * width);
      ++j;
    }
  memcpy(rows, tmp, sizeof(uint16_t) * (size_t)j * width);
  free(tmp);
  return j;
}

/* Bit pattern helper for tests (order of non-negative fp32 values). */
uint32_t orc_float_bits(float f) { return float_bits(f); }
