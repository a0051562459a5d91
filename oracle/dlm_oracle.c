/*
 * dlm_oracle.c — fp64 CPU oracle for the per-step unmask decision.
 *
 * TEST INFRASTRUCTURE ONLY: the product path never loads this file's library.
 * It is the slow, obviously-correct reference that the HIP kernels are
 * checked against.  It shares nothing with the HIP library.
 *
 * Sources (page title, section):
 *   [DepCap]  "DepCap: Adaptive Block-Wise Parallel Decoding for Efficient
 *             Diffusion LM Inference" (gptget.net summary of arXiv 2604.15750):
 *             Methodology; Technical Contribution; AI Executive Summary; Experiments.
 *   [DAPD]    "DAPD: Dependency-Aware Parallel Decoding via Attention for
 *             Diffusion LLMs" (papernotes.org, ICML 2026): overall framework
 *             section; key designs 1-3; ablation table.
 *   [FastR]   "Fast-dLLM: Training-Free Acceleration of Diffusion LLMs via KV
 *             Cache and Parallel Decoding" (romaanj.github.io review): Method.
 *   [FastN]   "Fast-dLLM: Training-free Acceleration of Diffusion LLM by
 *             Enabling KV Cache and Parallel Decoding" (patrick-llgc notes):
 *             Key ideas; Technical details.
 *
 * Readings where the pages are silent are stated at each function.
 * Arithmetic: IEEE double, plain loops, summation in index order.
 */
#include "dlm_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- helpers */

/* Widen element idx of a bf16 or fp32 array to double (exact). */
static double elem(const void* base, int dtype, int64_t idx) {
  if (dtype == DLMO_F32) return (double)((const float*)base)[idx];
  uint32_t u = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

typedef void (*range_fn)(void* ctx, int64_t begin, int64_t end);
typedef struct {
  range_fn fn;
  void* ctx;
  int64_t begin, end;
} range_job;

static void* run_range(void* p) {
  range_job* j = (range_job*)p;
  j->fn(j->ctx, j->begin, j->end);
  return NULL;
}

/* Split [0, n) into contiguous slices, one per thread.  Parallelism is only
 * across independent rows or sequences; each slice is computed serially. */
static void parallel_for(int64_t n, int n_threads, range_fn fn, void* ctx) {
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if ((int64_t)n_threads > n) n_threads = (int)(n > 0 ? n : 1);
  if (n_threads == 1) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t th[256];
  range_job jobs[256];
  for (int t = 0; t < n_threads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].begin = n * t / n_threads;
    jobs[t].end = n * (t + 1) / n_threads;
    pthread_create(&th[t], NULL, run_range, &jobs[t]);
  }
  for (int t = 0; t < n_threads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------- step statistics */

/* Max over the non-NaN entries of a row and the lowest index attaining it.
 * A row with no non-NaN entry gives max = NaN and index 0. */
static void row_max(const void* row, int dtype, int64_t V, double* m_out, int32_t* idx_out) {
  double m = NAN;
  int64_t idx = 0;
  int found = 0;
  for (int64_t v = 0; v < V; ++v) {
    double x = elem(row, dtype, v);
    if (isnan(x)) continue;
    if (!found || x > m) {
      m = x;
      idx = v;
      found = 1;
    }
  }
  *m_out = m;
  *idx_out = (int32_t)idx;
}

/* The row's log-normaliser relative to its max m: log(sum exp(x - m)), so
 * that lse = m + row_logz(...) (the two-pass log-sum-exp).  Any NaN entry, a
 * +inf entry, or a row that is all -inf gives NaN. */
static double row_logz(const void* row, int dtype, int64_t V, double m) {
  double z = 0.0;
  for (int64_t v = 0; v < V; ++v) z += exp(elem(row, dtype, v) - m);
  return log(z);
}

/*
 * One row of step statistics.
 *
 * [FastR, Method] and [DepCap, Methodology]: confidence is the maximum
 * softmax probability c = max_v p(v), and the committed token is that
 * position's argmax.  [DepCap, Methodology]: H_k = H(p_curr^k) and
 * I_k = KL(p_curr^k || p_prev^k).
 *
 * Readings: natural logarithm; temperature 1 (greedy decoding); argmax ties
 * go to the lowest vocabulary index; 0*log 0 = 0, i.e. entries with
 * logit -inf (probability exactly 0) contribute nothing to H or KL, while an
 * entry with p > 0 and q = 0 (prev logit -inf) makes KL = +inf.  A row whose
 * log-normaliser is not finite (NaN entry, +inf entry, all -inf) gives NaN
 * conf, entropy and KL.
 */
static void stats_row(const void* cur, const void* prev, int dtype, int64_t V, double* conf,
                      int32_t* argmax, double* entropy, double* kl, double* lse_out) {
  double m;
  int32_t idx;
  row_max(cur, dtype, V, &m, &idx);
  /* log p_v = (x_v - m) - logz.  The difference x_v - m is exact in double
   * for fp32 and bf16 inputs; taking it before the normaliser keeps logz
   * from being absorbed by a max of huge magnitude (m + logz == m once
   * |m| > 2^52 logz), which x_v - lse would not. */
  double logz = row_logz(cur, dtype, V, m);
  double lse = m + logz;
  *argmax = idx;
  *lse_out = lse;
  /* conf = max_v p_v = exp((m - m) - logz) */
  *conf = exp(-logz);
  if (isnan(lse)) { /* no distribution: every statistic is NaN */
    *conf = NAN;
    *entropy = NAN;
    if (prev) *kl = NAN;
    return;
  }
  /* H = -sum_v p_v log p_v */
  double h = 0.0;
  for (int64_t v = 0; v < V; ++v) {
    double x = elem(cur, dtype, v);
    if (x == -INFINITY) continue; /* p_v = 0 */
    double lp = (x - m) - logz;
    h -= exp(lp) * lp;
  }
  *entropy = h;
  if (!prev) return;
  double mq;
  int32_t idxq;
  row_max(prev, dtype, V, &mq, &idxq);
  double logzq = row_logz(prev, dtype, V, mq);
  if (isnan(lse) || isnan(mq + logzq)) {
    *kl = NAN;
    return;
  }
  /* KL = sum_v p_v (log p_v - log q_v), log q_v = (x'_v - m') - logz' */
  double d = 0.0;
  int infinite = 0;
  for (int64_t v = 0; v < V; ++v) {
    double x = elem(cur, dtype, v);
    if (x == -INFINITY) continue; /* p_v = 0 */
    double xq = elem(prev, dtype, v);
    if (xq == -INFINITY) { /* p_v > 0, q_v = 0 */
      infinite = 1;
      continue;
    }
    double lp = (x - m) - logz;
    double lq = (xq - mq) - logzq;
    d += exp(lp) * (lp - lq);
  }
  *kl = infinite ? INFINITY : d;
}

typedef struct {
  const void *logits, *prev;
  int dtype;
  int64_t V, ld;
  const int64_t* row_index;
  double *conf, *entropy, *kl, *lse;
  int32_t* argmax;
} stats_ctx;

static void stats_range(void* p, int64_t b, int64_t e) {
  stats_ctx* c = (stats_ctx*)p;
  size_t es = c->dtype == DLMO_F32 ? 4 : 2;
  for (int64_t r = b; r < e; ++r) {
    int64_t off = c->row_index[r] * c->ld;
    const void* cur = (const char*)c->logits + off * es;
    const void* prv = c->prev ? (const char*)c->prev + off * es : NULL;
    double klv = NAN;
    stats_row(cur, prv, c->dtype, c->V, &c->conf[r], &c->argmax[r], &c->entropy[r], &klv,
              &c->lse[r]);
    if (c->kl) c->kl[r] = c->prev ? klv : NAN;
  }
}

int dlmo_step_stats(const void* logits, const void* prev, int dtype, int64_t vocab,
                    int64_t ld, const int64_t* row_index, int64_t n_rows, double* conf,
                    int32_t* argmax, double* entropy, double* kl, double* lse, int n_threads) {
  if (!logits || !row_index || !conf || !argmax || !entropy || !lse) return 1;
  if (prev && !kl) return 1;
  if (dtype != DLMO_BF16 && dtype != DLMO_F32) return 1;
  if (vocab <= 0 || ld < vocab || n_rows < 0) return 1;
  stats_ctx c = {logits, prev, dtype, vocab, ld, row_index, conf, entropy, kl, lse, argmax};
  parallel_for(n_rows, n_threads, stats_range, &c);
  return 0;
}

/* ------------------------------------------------------------- Fast-dLLM */

/*
 * [FastR, Method]; [FastN, Key ideas and Technical details]: commit every
 * masked position of the active block whose confidence exceeds tau; if none
 * does, commit the single highest-confidence position so that decoding
 * always progresses.
 *
 * Readings: "exceeds" is strict (>); the active block is the eligible mask;
 * fallback ties go to the lowest position; a NaN confidence never commits.
 */
int dlmo_fastdllm_select(const double* conf, const uint8_t* eligible,
                         const int32_t* seq_offsets, int32_t n_seq, double tau,
                         uint8_t* commit, int32_t* n_commit) {
  if (!conf || !seq_offsets || !commit || !n_commit || n_seq < 0 || isnan(tau)) return 1;
  for (int32_t b = 0; b < n_seq; ++b) {
    int32_t lo = seq_offsets[b], hi = seq_offsets[b + 1];
    int32_t cnt = 0, best = -1;
    for (int32_t r = lo; r < hi; ++r) {
      int el = eligible ? eligible[r] != 0 : 1;
      commit[r] = (uint8_t)(el && conf[r] > tau);
      cnt += commit[r];
      if (el && !isnan(conf[r]) && (best < 0 || conf[r] > conf[best])) best = r;
    }
    if (cnt == 0 && best >= 0) {
      commit[best] = 1;
      cnt = 1;
    }
    n_commit[b] = cnt;
  }
  return 0;
}

/* ---------------------------------------------------------- DepGA-Block */

/*
 * [DepCap, Methodology]: over the local window L_window = min(L_max, L_remain)
 * of future positions, take I_k (KL to the previous step) and H_k (entropy),
 * smooth and locally normalise them, and form S_k = I~_k - lambda * H~_k
 * ([DepCap, Technical Contribution]).
 *
 * Readings (the pages give no formula for either step):
 *   smoothing     = centred box mean of radius r over [k-r, k+r] clipped to
 *                   the window (r = 0 disables it);
 *   normalisation = divide by the window mean of the smoothed values, plus eps.
 * Cold start (no previous step): no scores, reported as NaN.
 */
int dlmo_depcap_scores(const double* kl, const double* entropy, const int32_t* seq_offsets,
                       int32_t n_seq, int32_t l_max, const uint8_t* has_prev, double lambda,
                       int32_t radius, double eps, double* score) {
  if (!kl || !entropy || !seq_offsets || !score || n_seq < 0 || l_max <= 0 || radius < 0)
    return 1;
  for (int32_t b = 0; b < n_seq; ++b) {
    int32_t lo = seq_offsets[b], hi = seq_offsets[b + 1];
    for (int32_t r = lo; r < hi; ++r) score[r] = NAN;
    int32_t n = hi - lo;
    int32_t W = n < l_max ? n : l_max;
    if (W <= 0 || (has_prev && !has_prev[b])) continue;
    double* ib = (double*)malloc(sizeof(double) * (size_t)W);
    double* hb = (double*)malloc(sizeof(double) * (size_t)W);
    for (int32_t k = 0; k < W; ++k) {
      /* the window's ends in 64-bit: k + radius must not overflow */
      int64_t lo64 = (int64_t)k - radius, hi64 = (int64_t)k + radius;
      int32_t j0 = lo64 < 0 ? 0 : (int32_t)lo64;
      int32_t j1 = hi64 > W - 1 ? W - 1 : (int32_t)hi64;
      double si = 0.0, sh = 0.0;
      for (int32_t j = j0; j <= j1; ++j) {
        si += kl[lo + j];
        sh += entropy[lo + j];
      }
      ib[k] = si / (double)(j1 - j0 + 1);
      hb[k] = sh / (double)(j1 - j0 + 1);
    }
    double mi = 0.0, mh = 0.0;
    for (int32_t k = 0; k < W; ++k) {
      mi += ib[k];
      mh += hb[k];
    }
    mi /= (double)W;
    mh /= (double)W;
    for (int32_t k = 0; k < W; ++k)
      score[lo + k] = ib[k] / (mi + eps) - lambda * (hb[k] / (mh + eps));
    free(ib);
    free(hb);
  }
  return 0;
}

/*
 * [DepCap, Methodology]: stop before the first S_k < 0 and clip the length to
 * [L_min, L_window]; use L_min on cold start.
 * Readings: the block is positions 0..k*-1, so its length is k* (W if no
 * score is negative); when W < L_min the clip gives W; a NaN score is not
 * negative.
 */
int dlmo_depcap_decide(const double* score, const int32_t* seq_offsets, int32_t n_seq,
                       int32_t l_max, const uint8_t* has_prev, int32_t l_min,
                       int32_t* block_len) {
  if (!score || !seq_offsets || !block_len || n_seq < 0 || l_max <= 0 || l_min < 0 ||
      l_min > l_max)
    return 1;
  for (int32_t b = 0; b < n_seq; ++b) {
    int32_t lo = seq_offsets[b], n = seq_offsets[b + 1] - lo;
    int32_t W = n < l_max ? n : l_max;
    if (W < 0) W = 0;
    if (has_prev && !has_prev[b]) {
      block_len[b] = l_min < W ? l_min : W;
      continue;
    }
    int32_t ks = W;
    for (int32_t k = 0; k < W; ++k)
      if (score[lo + k] < 0.0) {
        ks = k;
        break;
      }
    int32_t L = ks > l_min ? ks : l_min;
    block_len[b] = L < W ? L : W;
  }
  return 0;
}

/* --------------------------------------------------------- CAP-Decoding */

/*
 * [DepCap, Methodology]: within the selected block, confidence
 * c_i = max_v p_i(v), keep c_i >= tau_low; if no safe set exists decode the
 * highest-confidence position.  [DepCap, AI Executive Summary]: candidates
 * need confidence at least 0.8.
 *
 * Readings: the pool bound is >= as printed; a NaN confidence is never in
 * the pool; the K_max cap keeps the first k_max in (conf desc, index asc)
 * order; "no safe set" can only mean an empty pool (the greedy always admits
 * its first candidate), and the fallback then takes the top-1 eligible
 * position (lowest index on ties).
 */
int dlmo_cap_pool(const double* conf, const uint8_t* eligible, int32_t n, double tau_low,
                  int32_t k_max, int32_t* cand, int32_t* n_cand, int32_t* fallback) {
  if (!conf || !cand || !n_cand || !fallback || n < 0 || k_max <= 0) return 1;
  int32_t* all = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  int32_t np = 0, best = -1;
  for (int32_t i = 0; i < n; ++i) {
    int el = eligible ? eligible[i] != 0 : 1;
    if (!el || isnan(conf[i])) continue;
    if (best < 0 || conf[i] > conf[best]) best = i;
    if (conf[i] >= tau_low) all[np++] = i;
  }
  /* insertion sort by (conf desc, index asc): plain and stable */
  for (int32_t a = 1; a < np; ++a) {
    int32_t x = all[a], p = a - 1;
    while (p >= 0 && conf[all[p]] < conf[x]) {
      all[p + 1] = all[p];
      --p;
    }
    all[p + 1] = x;
  }
  int32_t k = np < k_max ? np : k_max;
  for (int32_t a = 0; a < k; ++a) cand[a] = all[a];
  *n_cand = k;
  *fallback = np == 0 ? best : -1;
  free(all);
  return 0;
}

/*
 * [DepCap, Technical Contribution]: D_ij = log p_i(yhat_j) + log p_j(yhat_i),
 * with log p_i(v) = logit_i[v] - lse_i.
 */
int dlmo_cap_dmatrix(const void* logits, int dtype, int64_t vocab, int64_t ld,
                     const int64_t* row_index, const int32_t* argmax, const double* lse,
                     const int32_t* cand_rows, int32_t n_cand, double* D, int32_t ldd) {
  if (!logits || !row_index || !argmax || !lse || !cand_rows || !D || n_cand < 0 ||
      ldd < n_cand || vocab <= 0)
    return 1;
  size_t es = dtype == DLMO_F32 ? 4 : 2;
  for (int32_t a = 0; a < n_cand; ++a) {
    for (int32_t b = 0; b < n_cand; ++b) {
      if (a == b) {
        D[(int64_t)a * ldd + b] = NAN;
        continue;
      }
      int32_t ra = cand_rows[a], rb = cand_rows[b];
      const void* la = (const char*)logits + row_index[ra] * ld * (int64_t)es;
      const void* lb = (const char*)logits + row_index[rb] * ld * (int64_t)es;
      double log_pa_yb = elem(la, dtype, argmax[rb]) - lse[ra];
      double log_pb_ya = elem(lb, dtype, argmax[ra]) - lse[rb];
      D[(int64_t)a * ldd + b] = log_pa_yb + log_pb_ya;
    }
  }
  return 0;
}

/*
 * [DepCap, Methodology]: select the tau_high candidates first, remove their
 * conflicts, then greedily add the remaining candidates by confidence while
 * deleting conflicts.  [DepCap, AI Executive Summary]: priority for
 * confidence above 0.95, gamma = -16.
 *
 * Readings: a pair conflicts when D_ij > gamma (large D means each position
 * puts real mass on the other's token); the tau_high set is committed
 * unconditionally (strict >); the rest, in (conf desc, index asc) order, are
 * added when they conflict with nothing already chosen.  Candidates arrive
 * in that order, so the tau_high set is a prefix of it.
 */
int dlmo_cap_greedy(const double* cand_conf, const double* D, int32_t ldd, int32_t n_cand,
                    double tau_high, double gamma, uint8_t* take) {
  if (!cand_conf || !D || !take || n_cand < 0 || ldd < n_cand) return 1;
  for (int32_t a = 0; a < n_cand; ++a) take[a] = 0;
  for (int32_t a = 0; a < n_cand; ++a)
    if (cand_conf[a] > tau_high) take[a] = 1;
  for (int32_t a = 0; a < n_cand; ++a) {
    if (take[a]) continue;
    int ok = 1;
    for (int32_t b = 0; b < n_cand && ok; ++b)
      if (take[b] && D[(int64_t)a * ldd + b] > gamma) ok = 0;
    if (ok) take[a] = 1;
  }
  return 0;
}

typedef struct {
  const void* logits;
  int dtype;
  int64_t vocab, ld;
  const int64_t* row_index;
  const int32_t* seq_offsets;
  const double *conf, *lse;
  const int32_t* argmax;
  const uint8_t* eligible;
  double tau_low, tau_high, gamma;
  int32_t k_max;
  uint8_t* commit;
  int32_t *n_commit, *cand_out;
  double* dmat_out;
} cap_ctx;

static void cap_range(void* p, int64_t b0, int64_t b1) {
  cap_ctx* c = (cap_ctx*)p;
  int32_t K = c->k_max;
  int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
  double* cc = (double*)malloc(sizeof(double) * (size_t)K);
  double* D = (double*)malloc(sizeof(double) * (size_t)K * (size_t)K);
  uint8_t* take = (uint8_t*)malloc((size_t)K);
  for (int64_t b = b0; b < b1; ++b) {
    int32_t lo = c->seq_offsets[b], n = c->seq_offsets[b + 1] - lo;
    for (int32_t i = 0; i < n; ++i) c->commit[lo + i] = 0;
    int32_t nc = 0, fb = -1;
    dlmo_cap_pool(c->conf + lo, c->eligible ? c->eligible + lo : NULL, n, c->tau_low, K, cand,
                  &nc, &fb);
    for (int32_t a = 0; a < nc; ++a) {
      rows[a] = lo + cand[a];
      cc[a] = c->conf[lo + cand[a]];
    }
    int32_t cnt = 0;
    if (nc == 0) {
      if (fb >= 0) {
        c->commit[lo + fb] = 1;
        cnt = 1;
      }
    } else {
      dlmo_cap_dmatrix(c->logits, c->dtype, c->vocab, c->ld, c->row_index, c->argmax, c->lse,
                       rows, nc, D, K);
      dlmo_cap_greedy(cc, D, K, nc, c->tau_high, c->gamma, take);
      for (int32_t a = 0; a < nc; ++a)
        if (take[a]) {
          c->commit[rows[a]] = 1;
          ++cnt;
        }
    }
    c->n_commit[b] = cnt;
    if (c->cand_out)
      for (int32_t a = 0; a < K; ++a) c->cand_out[b * K + a] = a < nc ? rows[a] : -1;
    if (c->dmat_out)
      for (int32_t a = 0; a < K; ++a)
        for (int32_t e = 0; e < K; ++e)
          c->dmat_out[(b * K + a) * K + e] = (a < nc && e < nc) ? D[a * K + e] : NAN;
  }
  free(cand);
  free(rows);
  free(cc);
  free(D);
  free(take);
}

int dlmo_cap_select(const void* logits, int dtype, int64_t vocab, int64_t ld,
                    const int64_t* row_index, const int32_t* seq_offsets, int32_t n_seq,
                    const double* conf, const int32_t* argmax, const double* lse,
                    const uint8_t* eligible, double tau_low, double tau_high, double gamma,
                    int32_t k_max, uint8_t* commit, int32_t* n_commit, int32_t* cand_out,
                    double* dmat_out, int n_threads) {
  if (!logits || !row_index || !seq_offsets || !conf || !argmax || !lse || !commit ||
      !n_commit || n_seq < 0 || k_max <= 0 || vocab <= 0)
    return 1;
  cap_ctx c = {logits, dtype,   vocab,    ld,       row_index, seq_offsets,
               conf,   lse,     argmax,   eligible, tau_low,   tau_high,
               gamma,  k_max,   commit,   n_commit, cand_out,  dmat_out};
  parallel_for(n_seq, n_threads, cap_range, &c);
  return 0;
}

/* ------------------------------------------------------------------ DAPD */

/*
 * [DAPD, overall framework]: average the attention of all heads of the last
 * ~30% of layers into a_ij.  The caller passes exactly the maps to average
 * (n_lh = layers x heads); the mean is equal-weight and the probabilities
 * are used as given (no renormalisation over the masked columns).
 */
int dlmo_dapd_average(const void* attn, int dtype, int32_t n_lh, int64_t S,
                      const int32_t* pos, int32_t M, double* a) {
  if (!attn || !pos || !a || n_lh <= 0 || S <= 0 || M < 0) return 1;
  for (int32_t i = 0; i < M; ++i)
    for (int32_t j = 0; j < M; ++j) {
      double sum = 0.0;
      for (int32_t l = 0; l < n_lh; ++l)
        sum += elem(attn, dtype, (int64_t)l * S * S + (int64_t)pos[i] * S + pos[j]);
      a[(int64_t)i * M + j] = sum / (double)n_lh;
    }
  return 0;
}

/*
 * [DAPD, key design 1]: s_ij = (a_ij + a_ji) / 2.
 * [DAPD, key design 2]: proxy degree d~_i = sum_{j != i} s_ij; the final
 * ordering key is d~_i * conf_i.
 */
int dlmo_dapd_graph(const double* a, int32_t M, const double* conf, double* s,
                    double* degree, double* key) {
  if (!a || !conf || !s || !degree || !key || M < 0) return 1;
  for (int32_t i = 0; i < M; ++i)
    for (int32_t j = 0; j < M; ++j)
      s[(int64_t)i * M + j] = 0.5 * (a[(int64_t)i * M + j] + a[(int64_t)j * M + i]);
  for (int32_t i = 0; i < M; ++i) {
    double d = 0.0;
    for (int32_t j = 0; j < M; ++j)
      if (j != i) d += s[(int64_t)i * M + j];
    degree[i] = d;
    key[i] = d * conf[i];
  }
  return 0;
}

/*
 * [DAPD, key design 1]: edge (i, j) exactly when s_ij > tau_t.
 * [DAPD, key design 2]: scan nodes by descending key and add each node that
 * is not adjacent to the current set S, giving a maximal (not maximum)
 * independent set.
 * Readings: ties in key go to the lower position; a node whose key is NaN
 * is never selected.
 */
int dlmo_dapd_greedy(const double* s, int32_t M, int64_t ld_s, double tau, const double* key,
                     uint8_t* take) {
  if (!s || !key || !take || M < 0 || ld_s < M || isnan(tau)) return 1;
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M > 0 ? M : 1));
  int32_t n = 0;
  for (int32_t i = 0; i < M; ++i) {
    take[i] = 0;
    if (!isnan(key[i])) order[n++] = i;
  }
  for (int32_t a = 1; a < n; ++a) { /* insertion sort: key desc, index asc */
    int32_t x = order[a], p = a - 1;
    while (p >= 0 && key[order[p]] < key[x]) {
      order[p + 1] = order[p];
      --p;
    }
    order[p + 1] = x;
  }
  for (int32_t t = 0; t < n; ++t) {
    int32_t i = order[t], ok = 1;
    for (int32_t j = 0; j < M && ok; ++j)
      if (take[j] && j != i && s[(int64_t)i * ld_s + j] > tau) ok = 0;
    if (ok) take[i] = 1;
  }
  free(order);
  return 0;
}

typedef struct {
  const void* attn;
  int dtype;
  int32_t n_lh;
  int64_t S, batch_stride;
  const int32_t *masked_pos, *seq_offsets;
  const double* conf;
  double tau;
  uint8_t* commit;
  int32_t* n_commit;
  double *degree, *sym, *key;
  int32_t m_max;
} dapd_ctx;

static void dapd_range(void* p, int64_t b0, int64_t b1) {
  dapd_ctx* c = (dapd_ctx*)p;
  size_t es = c->dtype == DLMO_F32 ? 4 : 2;
  for (int64_t b = b0; b < b1; ++b) {
    int32_t lo = c->seq_offsets[b], M = c->seq_offsets[b + 1] - lo;
    size_t mm = (size_t)(M > 0 ? M : 1);
    double* a = (double*)malloc(sizeof(double) * mm * mm);
    double* s = (double*)malloc(sizeof(double) * mm * mm);
    double* deg = (double*)malloc(sizeof(double) * mm);
    double* key = (double*)malloc(sizeof(double) * mm);
    uint8_t* take = (uint8_t*)malloc(mm);
    const void* base = (const char*)c->attn + (int64_t)b * c->batch_stride * (int64_t)es;
    dlmo_dapd_average(base, c->dtype, c->n_lh, c->S, c->masked_pos + lo, M, a);
    dlmo_dapd_graph(a, M, c->conf + lo, s, deg, key);
    dlmo_dapd_greedy(s, M, M, c->tau, key, take);
    int32_t cnt = 0;
    for (int32_t i = 0; i < M; ++i) {
      c->commit[lo + i] = take[i];
      cnt += take[i];
      if (c->degree) c->degree[lo + i] = deg[i];
      if (c->key) c->key[lo + i] = key[i];
    }
    c->n_commit[b] = cnt;
    if (c->sym) {
      int64_t mx = c->m_max;
      for (int64_t i = 0; i < mx; ++i)
        for (int64_t j = 0; j < mx; ++j)
          c->sym[(b * mx + i) * mx + j] = (i < M && j < M) ? s[i * M + j] : NAN;
    }
    free(a);
    free(s);
    free(deg);
    free(key);
    free(take);
  }
}

int dlmo_dapd_select(const void* attn, int dtype, int32_t n_lh, int64_t S, int64_t batch_stride,
                     const int32_t* masked_pos, const int32_t* seq_offsets, int32_t n_seq,
                     const double* conf, double tau, uint8_t* commit, int32_t* n_commit,
                     double* degree, double* sym, int32_t m_max, double* key, int n_threads) {
  if (!attn || !masked_pos || !seq_offsets || !conf || !commit || !n_commit || n_seq < 0 ||
      n_lh <= 0 || S <= 0 || isnan(tau))
    return 1;
  if (sym && m_max <= 0) return 1;
  dapd_ctx c = {attn, dtype,  n_lh,     S,      batch_stride, masked_pos, seq_offsets,
                conf, tau,    commit,   n_commit, degree,     sym,        key,
                m_max};
  parallel_for(n_seq, n_threads, dapd_range, &c);
  return 0;
}

/* ------------------------------------------------------ schedules (NEXT) */

/* A sequence's eligible rows with a non-NaN confidence, ordered by
 * (confidence desc, row asc); plain insertion sort.  Returns the count. */
static int32_t conf_order(const double* conf, const uint8_t* eligible, int32_t lo, int32_t hi,
                          int32_t* ord) {
  int32_t n = 0;
  for (int32_t r = lo; r < hi; ++r)
    if ((eligible ? eligible[r] != 0 : 1) && !isnan(conf[r])) ord[n++] = r;
  for (int32_t a = 1; a < n; ++a) {
    int32_t x = ord[a], p = a - 1;
    while (p >= 0 && conf[ord[p]] < conf[x]) {
      ord[p + 1] = ord[p];
      --p;
    }
    ord[p + 1] = x;
  }
  return n;
}

/*
 * [Fast-dLLM review, Prior limitations; Comparison]: LLaDA's default
 * schedule commits a fixed number K of tokens per step, the K most confident,
 * whatever their confidence.
 * Readings: ties go to the lower row; rows with NaN confidence are never
 * committed; with fewer than K eligible rows, all of them are committed.
 */
int dlmo_topk_select(const double* conf, const uint8_t* eligible, const int32_t* seq_offsets,
                     int32_t n_seq, int32_t k, uint8_t* commit, int32_t* n_commit) {
  if (!conf || !seq_offsets || !commit || !n_commit || n_seq < 0 || k < 1) return 1;
  for (int32_t b = 0; b < n_seq; ++b) {
    int32_t lo = seq_offsets[b], hi = seq_offsets[b + 1];
    int32_t* ord = (int32_t*)malloc(sizeof(int32_t) * (size_t)(hi > lo ? hi - lo : 1));
    int32_t n = conf_order(conf, eligible, lo, hi, ord);
    for (int32_t r = lo; r < hi; ++r) commit[r] = 0;
    int32_t take = n < k ? n : k;
    for (int32_t t = 0; t < take; ++t) commit[ord[t]] = 1;
    n_commit[b] = take;
    free(ord);
  }
  return 0;
}

/*
 * [Fast-dLLM review, Method (factor decoding); Key idea (Theorem 1)]: with
 * c(1) >= c(2) >= ... the eligible confidences in descending order, commit
 * the n most confident rows for the largest n with (n+1)(1 - c(n)) < f.
 * Readings:
 *   - the left side never decreases with n, so the admissible n form a
 *     prefix 1..n*; the test is evaluated in double precision on the given
 *     confidences (exact for fp32 inputs: 1 - c and the product by an integer
 *     below 2^29 are representable);
 *   - at least one row is committed when any is eligible (the progress
 *     guarantee of the threshold rule, [Fast-dLLM review, Method]);
 *   - ties go to the lower row; NaN confidences are never committed.
 * certificate[b] (optional) = 1 iff n >= 1 and (n+1)(1 - min committed c) <= 1,
 * Theorem 1's sufficient condition (its "(n+1) eps <= 1" form) for the
 * parallel commit to coincide with greedy one-at-a-time decoding.
 */
int dlmo_factor_select(const double* conf, const uint8_t* eligible, const int32_t* seq_offsets,
                       int32_t n_seq, double f, uint8_t* commit, int32_t* n_commit,
                       uint8_t* certificate) {
  if (!conf || !seq_offsets || !commit || !n_commit || n_seq < 0 || isnan(f)) return 1;
  for (int32_t b = 0; b < n_seq; ++b) {
    int32_t lo = seq_offsets[b], hi = seq_offsets[b + 1];
    int32_t* ord = (int32_t*)malloc(sizeof(int32_t) * (size_t)(hi > lo ? hi - lo : 1));
    int32_t n = conf_order(conf, eligible, lo, hi, ord);
    int32_t best = 0;
    for (int32_t m = 1; m <= n; ++m)
      if ((double)(m + 1) * (1.0 - conf[ord[m - 1]]) < f) best = m;
    if (best == 0 && n > 0) best = 1;
    for (int32_t r = lo; r < hi; ++r) commit[r] = 0;
    for (int32_t t = 0; t < best; ++t) commit[ord[t]] = 1;
    n_commit[b] = best;
    if (certificate)
      certificate[b] =
          (uint8_t)(best >= 1 && (double)(best + 1) * (1.0 - conf[ord[best - 1]]) <= 1.0);
    free(ord);
  }
  return 0;
}

/*
 * [DepCap summary, Experiments]: confidence decoding with fixed 16/32/64-token
 * blocks, as a baseline schedule.
 * Readings: blocks tile the generation in lengths of block_len from its first
 * position gen_start[b] (NULL: 0); the active block is the earliest block that
 * still holds a masked position; the eligible rows are the masked rows inside
 * it (the threshold rule then runs on them).  A masked position before
 * gen_start belongs to no block and is never eligible.
 */
int dlmo_fixed_block_eligible(const int32_t* masked_pos, const int32_t* seq_offsets,
                              int32_t n_seq, const int32_t* gen_start, int32_t block_len,
                              uint8_t* eligible) {
  if (!masked_pos || !seq_offsets || !eligible || n_seq < 0 || block_len < 1) return 1;
  for (int32_t b = 0; b < n_seq; ++b) {
    int32_t lo = seq_offsets[b], hi = seq_offsets[b + 1];
    int64_t g0 = gen_start ? gen_start[b] : 0, first = -1;
    for (int32_t r = lo; r < hi; ++r) {
      int64_t rel = (int64_t)masked_pos[r] - g0;
      if (rel < 0) continue;
      int64_t blk = rel / block_len;
      if (first < 0 || blk < first) first = blk;
    }
    for (int32_t r = lo; r < hi; ++r) {
      int64_t rel = (int64_t)masked_pos[r] - g0;
      eligible[r] = (uint8_t)(rel >= 0 && first >= 0 && rel / block_len == first);
    }
  }
  return 0;
}

/*
 * [DAPD note, overall framework; key design 3 (late-stage confidence
 * sparsification)]: the full DAPD step.  For sequence b with M_b masked rows
 * out of a generation of gen_len[b] tokens:
 *   - late stage iff M_b < late_frac * gen_len[b] (the remaining masks fell
 *     below 50%): no graph, commit every row with conf > late_tau (0.9);
 *   - otherwise the dependency-graph independent set (dlmo_dapd_select);
 *   - with pre_unmask, every row whose confidence is exactly 1.0 is also
 *     committed, in either stage (such a position takes the same token under
 *     every compatible joint distribution).
 * Readings: strict < for the switch and strict > for the threshold; a late
 * stage that commits nothing commits the most confident row (the threshold
 * rule's progress guarantee; the page gives none); pre-unmasked rows are added
 * to the set the stage chose, the graph being built over all masked rows as in
 * the plain step.  gen_len == NULL disables the late stage.  stage[b]
 * (optional) = 1 for a late-stage sequence.
 */
int dlmo_dapd_step(const void* attn, int dtype, int32_t n_lh, int64_t S, int64_t batch_stride,
                   const int32_t* masked_pos, const int32_t* seq_offsets, int32_t n_seq,
                   const double* conf, double tau, const int32_t* gen_len, double late_frac,
                   double late_tau, int pre_unmask, uint8_t* commit, int32_t* n_commit,
                   uint8_t* stage, int n_threads) {
  if (!attn || !masked_pos || !seq_offsets || !conf || !commit || !n_commit || n_seq < 0 ||
      isnan(tau) || isnan(late_frac) || isnan(late_tau))
    return 1;
  int rc = dlmo_dapd_select(attn, dtype, n_lh, S, batch_stride, masked_pos, seq_offsets, n_seq,
                            conf, tau, commit, n_commit, NULL, NULL, 0, NULL, n_threads);
  if (rc) return rc;
  for (int32_t b = 0; b < n_seq; ++b) {
    int32_t lo = seq_offsets[b], hi = seq_offsets[b + 1];
    int late = gen_len && (double)(hi - lo) < late_frac * (double)gen_len[b];
    if (stage) stage[b] = (uint8_t)late;
    if (late) {
      int32_t sub[2] = {0, hi - lo};
      dlmo_fastdllm_select(conf + lo, NULL, sub, 1, late_tau, commit + lo, n_commit + b);
    }
    if (pre_unmask) {
      int32_t cnt = 0;
      for (int32_t r = lo; r < hi; ++r) {
        if (conf[r] == 1.0) commit[r] = 1;
        cnt += commit[r];
      }
      n_commit[b] = cnt;
    }
  }
  return 0;
}
