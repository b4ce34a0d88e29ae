/*
 * msa_oracle.c — plain, slow, single-threaded CPU oracle of the MSA forward
 * pass and of the main branch's gradient.  TEST INFRASTRUCTURE ONLY (see msa_oracle.h for the pages followed,
 * the readings taken and the layouts).  Every loop here is the definition
 * written out; there is no tiling, fusion or reordering.
 */
#include "msa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Exact value of a bf16 bit pattern: the top half of an IEEE binary32. */
static double bf16_value(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static int problem_ok(const oracle_problem* p) {
  if (!p) return 0;
  if (p->batch <= 0 || p->seq_q <= 0 || p->seq_kv <= 0 || p->q_start < 0) return 0;
  if (p->n_q_heads <= 0 || p->n_kv_heads <= 0 || p->n_q_heads % p->n_kv_heads != 0) return 0;
  if (p->head_dim <= 0 || p->idx_head_dim <= 0 || p->block_size <= 0 || p->top_k <= 0) return 0;
  /* every KV head needs at least one index head attributed to it */
  if (p->n_idx_heads < p->n_kv_heads || p->n_idx_heads % p->n_kv_heads != 0) return 0;
  if (p->decode) {
    if (p->seq_q != 1) return 0;
  } else if ((int64_t)p->q_start + p->seq_q > p->seq_kv) {
    return 0;
  }
  return 1;
}

int32_t oracle_num_blocks(const oracle_problem* p) {
  return (p->seq_kv + p->block_size - 1) / p->block_size;
}

int32_t oracle_position(const oracle_problem* p, const int32_t* seq_lens, int32_t b, int32_t t) {
  if (!problem_ok(p) || b < 0 || b >= p->batch || t < 0 || t >= p->seq_q) return -1;
  if (p->decode) {
    if (!seq_lens) return -1;
    int32_t L = seq_lens[b];
    if (L < 1 || L > p->seq_kv) return -1;
    return L - 1;
  }
  return p->q_start + t;
}

/* Index score of token j against index head i of row (b, t): the raw dot
 * product of index-query and index-key ([A] index branch: 4 query heads
 * against one key head). */
static double index_score(const oracle_problem* p, const uint16_t* iq, const uint16_t* ik,
                          int32_t b, int32_t t, int32_t i, int32_t j) {
  const int Di = p->idx_head_dim;
  const uint16_t* qv = iq + (((int64_t)b * p->seq_q + t) * p->n_idx_heads + i) * Di;
  const uint16_t* kv = ik + ((int64_t)b * p->seq_kv + j) * Di;
  double s = 0.0;
  for (int d = 0; d < Di; ++d) s += bf16_value(qv[d]) * bf16_value(kv[d]);
  return s;
}

int oracle_block_scores_row(const oracle_problem* p, const uint16_t* iq, const uint16_t* ik,
                            const int32_t* seq_lens, int32_t b, int32_t t, float* out) {
  int32_t pos = oracle_position(p, seq_lens, b, t);
  if (pos < 0 || !iq || !ik || !out) return ORACLE_EBADARG;
  const int32_t nblk = oracle_num_blocks(p);
  const int32_t bs = p->block_size;
  const int32_t cur = pos / bs;
  for (int32_t h = 0; h < p->n_kv_heads; ++h) {
    for (int32_t c = 0; c < nblk; ++c) {
      float value;
      if (c < cur) {
        /* every token of block c precedes the query's own block, so all of
         * them are causal */
        double best = -INFINITY;
        for (int32_t i = 0; i < p->n_idx_heads; ++i) {
          if (i % p->n_kv_heads != h) continue; /* index head i drives KV head i mod Hkv */
          for (int32_t j = c * bs; j < (c + 1) * bs; ++j) {
            double s = index_score(p, iq, ik, b, t, i, j);
            if (isnan(s)) return ORACLE_ENAN;
            if (s > best) best = s;
          }
        }
        value = (float)best; /* round to nearest fp32: the decision precision */
      } else if (c == cur) {
        value = INFINITY; /* own block always kept */
      } else {
        value = -INFINITY; /* future block: never a candidate */
      }
      out[(int64_t)h * nblk + c] = value;
    }
  }
  return ORACLE_OK;
}

int oracle_select_row(const oracle_problem* p, const float* scores, int32_t cur, int32_t* sel) {
  if (!p || !scores || !sel || cur < 0 || p->top_k <= 0) return ORACLE_EBADARG;
  const int32_t n = cur + 1;
  const int32_t m = p->top_k < n ? p->top_k : n;
  char* chosen = (char*)calloc((size_t)n, 1);
  if (!chosen) return ORACLE_ENOMEM;
  for (int32_t c = 0; c < n; ++c)
    if (isnan(scores[c])) { free(chosen); return ORACLE_ENAN; }
  /* m rounds of "take the best remaining candidate": best = highest score,
   * and among equal scores the lowest block index (the ascending scan with a
   * strict comparison keeps the first, i.e. lowest, index).  -0 and +0 compare
   * equal as reals. */
  for (int32_t r = 0; r < m; ++r) {
    int32_t best = -1;
    for (int32_t c = 0; c < n; ++c) {
      if (chosen[c]) continue;
      if (best < 0 || scores[c] > scores[best]) best = c;
    }
    chosen[best] = 1;
  }
  int32_t w = 0;
  for (int32_t c = 0; c < n; ++c)
    if (chosen[c]) sel[w++] = c;
  for (; w < p->top_k; ++w) sel[w] = -1;
  free(chosen);
  return ORACLE_OK;
}

int oracle_attend_row(const oracle_problem* p, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const int32_t* seq_lens, const int32_t* sel,
                      int32_t b, int32_t t, double* out, double* lse) {
  int32_t pos = oracle_position(p, seq_lens, b, t);
  if (pos < 0 || !q || !k || !v || !sel || !out || !lse) return ORACLE_EBADARG;
  const int32_t D = p->head_dim, bs = p->block_size, K = p->top_k;
  const int32_t G = p->n_q_heads / p->n_kv_heads;
  const int32_t nblk = oracle_num_blocks(p);
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)K * bs);
  double* z = (double*)malloc(sizeof(double) * (size_t)K * bs);
  if (!tok || !z) { free(tok); free(z); return ORACLE_ENOMEM; }
  int rc = ORACLE_OK;
  for (int32_t hq = 0; hq < p->n_q_heads && rc == ORACLE_OK; ++hq) {
    const int32_t h = hq / G; /* contiguous query-head groups per KV head */
    /* T: the tokens of the blocks KV head h selected, causal (j <= pos) */
    int32_t n = 0;
    for (int32_t r = 0; r < K; ++r) {
      int32_t c = sel[(int64_t)h * K + r];
      if (c < 0) continue;
      if (c >= nblk) { rc = ORACLE_EBADARG; break; }
      for (int32_t j = c * bs; j < (c + 1) * bs && j <= pos; ++j) tok[n++] = j;
    }
    if (rc != ORACLE_OK) break;
    double* o = out + (int64_t)hq * D;
    if (n == 0) { /* nothing to attend: defined as zero output, lse -inf */
      for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
      lse[hq] = -INFINITY;
      continue;
    }
    const uint16_t* qv = q + (((int64_t)b * p->seq_q + t) * p->n_q_heads + hq) * D;
    double zmax = -INFINITY;
    for (int32_t a = 0; a < n; ++a) {
      const uint16_t* kv = k + (((int64_t)b * p->n_kv_heads + h) * p->seq_kv + tok[a]) * D;
      double s = 0.0;
      for (int32_t d = 0; d < D; ++d) s += bf16_value(qv[d]) * bf16_value(kv[d]);
      z[a] = p->softmax_scale * s;
      if (z[a] > zmax) zmax = z[a];
    }
    double l = 0.0;
    for (int32_t a = 0; a < n; ++a) { z[a] = exp(z[a] - zmax); l += z[a]; }
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int32_t a = 0; a < n; ++a) {
      const uint16_t* vv = v + (((int64_t)b * p->n_kv_heads + h) * p->seq_kv + tok[a]) * D;
      for (int32_t d = 0; d < D; ++d) o[d] += z[a] * bf16_value(vv[d]);
    }
    for (int32_t d = 0; d < D; ++d) o[d] /= l;
    lse[hq] = zmax + log(l);
  }
  free(tok);
  free(z);
  return rc;
}

int oracle_dense_row(const oracle_problem* p, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, const int32_t* seq_lens, int32_t b, int32_t t,
                     double* out, double* lse) {
  int32_t pos = oracle_position(p, seq_lens, b, t);
  if (pos < 0 || !q || !k || !v || !out || !lse) return ORACLE_EBADARG;
  const int32_t D = p->head_dim;
  const int32_t nkeys = pos + 1;
  double* w = (double*)malloc(sizeof(double) * (size_t)nkeys);
  if (!w) return ORACLE_ENOMEM;
  for (int32_t hq = 0; hq < p->n_q_heads; ++hq) {
    const int32_t kvh = hq / (p->n_q_heads / p->n_kv_heads);
    const uint16_t* qrow = q + ((int64_t)(b * p->seq_q + t) * p->n_q_heads + hq) * D;
    const uint16_t* kbase = k + ((int64_t)b * p->n_kv_heads + kvh) * p->seq_kv * D;
    const uint16_t* vbase = v + ((int64_t)b * p->n_kv_heads + kvh) * p->seq_kv * D;
    /* pass 1: logits and their maximum */
    double top = -INFINITY;
    for (int32_t j = 0; j < nkeys; ++j) {
      double acc = 0.0;
      for (int32_t d = 0; d < D; ++d)
        acc += bf16_value(qrow[d]) * bf16_value(kbase[(int64_t)j * D + d]);
      w[j] = acc * p->softmax_scale;
      if (w[j] > top) top = w[j];
    }
    /* pass 2: normaliser */
    double denom = 0.0;
    for (int32_t j = 0; j < nkeys; ++j) denom += exp(w[j] - top);
    /* pass 3: probabilities */
    for (int32_t j = 0; j < nkeys; ++j) w[j] = exp(w[j] - top) / denom;
    /* pass 4: probability-weighted values, one output element at a time */
    for (int32_t d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int32_t j = 0; j < nkeys; ++j) acc += w[j] * bf16_value(vbase[(int64_t)j * D + d]);
      out[(int64_t)hq * D + d] = acc;
    }
    lse[hq] = top + log(denom);
  }
  free(w);
  return ORACLE_OK;
}

int oracle_forward_rows(const oracle_problem* p, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const uint16_t* iq, const uint16_t* ik,
                        const int32_t* seq_lens, int64_t n_rows, const int64_t* rows,
                        int32_t* sel_out, double* out, double* lse, float* scores_out) {
  if (!problem_ok(p) || n_rows < 0 || (n_rows > 0 && !rows) || !sel_out || !out || !lse)
    return ORACLE_EBADARG;
  const int32_t nblk = oracle_num_blocks(p);
  const int32_t Hkv = p->n_kv_heads, K = p->top_k;
  float* bsrow = (float*)malloc(sizeof(float) * (size_t)Hkv * nblk);
  if (!bsrow) return ORACLE_ENOMEM;
  int rc = ORACLE_OK;
  for (int64_t r = 0; r < n_rows && rc == ORACLE_OK; ++r) {
    const int64_t row = rows[r];
    if (row < 0 || row >= (int64_t)p->batch * p->seq_q) { rc = ORACLE_EBADARG; break; }
    const int32_t b = (int32_t)(row / p->seq_q), t = (int32_t)(row % p->seq_q);
    const int32_t cur = oracle_position(p, seq_lens, b, t) / p->block_size;
    rc = oracle_block_scores_row(p, iq, ik, seq_lens, b, t, bsrow);
    if (rc != ORACLE_OK) break;
    if (scores_out) memcpy(scores_out + r * Hkv * nblk, bsrow, sizeof(float) * (size_t)Hkv * nblk);
    int32_t* sel = sel_out + r * Hkv * K;
    for (int32_t h = 0; h < Hkv && rc == ORACLE_OK; ++h)
      rc = oracle_select_row(p, bsrow + (int64_t)h * nblk, cur, sel + (int64_t)h * K);
    if (rc != ORACLE_OK) break;
    rc = oracle_attend_row(p, q, k, v, seq_lens, sel, b, t, out + r * p->n_q_heads * p->head_dim,
                           lse + r * p->n_q_heads);
  }
  free(bsrow);
  return rc;
}

/* Tokens of the blocks in sel_h[0..top_k) (one KV head's selection, -1 =
 * none) that row position pos may attend (j <= pos), in list order.
 * Returns the count, or -1 for a block id past the cache. */
static int32_t selected_tokens(const oracle_problem* p, const int32_t* sel_h, int32_t pos,
                               int32_t* tok) {
  const int32_t bs = p->block_size, nblk = oracle_num_blocks(p);
  int32_t n = 0;
  for (int32_t r = 0; r < p->top_k; ++r) {
    int32_t c = sel_h[r];
    if (c < 0) continue;
    if (c >= nblk) return -1;
    for (int32_t j = c * bs; j <= pos && j < (c + 1) * bs; ++j) tok[n++] = j;
  }
  return n;
}

int oracle_attend_row_f64(const oracle_problem* p, const double* q, const double* k,
                          const double* v, const int32_t* seq_lens, const int32_t* sel,
                          int32_t b, int32_t t, double* out, double* lse) {
  int32_t pos = oracle_position(p, seq_lens, b, t);
  if (pos < 0 || !q || !k || !v || !sel || !out || !lse) return ORACLE_EBADARG;
  const int32_t D = p->head_dim, K = p->top_k;
  const int32_t G = p->n_q_heads / p->n_kv_heads;
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)K * p->block_size);
  double* z = (double*)malloc(sizeof(double) * (size_t)K * p->block_size);
  if (!tok || !z) { free(tok); free(z); return ORACLE_ENOMEM; }
  int rc = ORACLE_OK;
  for (int32_t hq = 0; hq < p->n_q_heads; ++hq) {
    const int32_t h = hq / G;
    const int32_t n = selected_tokens(p, sel + (int64_t)h * K, pos, tok);
    if (n < 0) { rc = ORACLE_EBADARG; break; }
    double* o = out + (int64_t)hq * D;
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    if (n == 0) { lse[hq] = -INFINITY; continue; }
    const double* qv = q + (((int64_t)b * p->seq_q + t) * p->n_q_heads + hq) * D;
    double zmax = -INFINITY;
    for (int32_t a = 0; a < n; ++a) {
      const double* kv = k + (((int64_t)b * p->n_kv_heads + h) * p->seq_kv + tok[a]) * D;
      double s = 0.0;
      for (int32_t d = 0; d < D; ++d) s += qv[d] * kv[d];
      z[a] = s * p->softmax_scale;
      if (z[a] > zmax) zmax = z[a];
    }
    double l = 0.0;
    for (int32_t a = 0; a < n; ++a) { z[a] = exp(z[a] - zmax); l += z[a]; }
    for (int32_t a = 0; a < n; ++a) {
      const double* vv = v + (((int64_t)b * p->n_kv_heads + h) * p->seq_kv + tok[a]) * D;
      for (int32_t d = 0; d < D; ++d) o[d] += z[a] * vv[d];
    }
    for (int32_t d = 0; d < D; ++d) o[d] = o[d] / l;
    lse[hq] = log(l) + zmax;
  }
  free(tok);
  free(z);
  return rc;
}

int oracle_attend_backward(const oracle_problem* p, const double* q, const double* k,
                           const double* v, const double* dout, const int32_t* seq_lens,
                           const int32_t* sel_all, double* dq, double* dk, double* dv) {
  if (!problem_ok(p) || !q || !k || !v || !dout || !sel_all || !dq || !dk || !dv)
    return ORACLE_EBADARG;
  const int32_t D = p->head_dim, K = p->top_k, Hq = p->n_q_heads, Hkv = p->n_kv_heads;
  const int32_t G = Hq / Hkv;
  const int64_t nq = (int64_t)p->batch * p->seq_q * Hq * D;
  const int64_t nkv = (int64_t)p->batch * Hkv * p->seq_kv * D;
  for (int64_t i = 0; i < nq; ++i) dq[i] = 0.0;
  for (int64_t i = 0; i < nkv; ++i) { dk[i] = 0.0; dv[i] = 0.0; }
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)K * p->block_size);
  double* w = (double*)malloc(sizeof(double) * (size_t)K * p->block_size);
  double* o = (double*)malloc(sizeof(double) * (size_t)D);
  if (!tok || !w || !o) { free(tok); free(w); free(o); return ORACLE_ENOMEM; }
  int rc = ORACLE_OK;
  for (int32_t b = 0; b < p->batch && rc == ORACLE_OK; ++b) {
    for (int32_t t = 0; t < p->seq_q && rc == ORACLE_OK; ++t) {
      const int32_t pos = oracle_position(p, seq_lens, b, t);
      if (pos < 0) { rc = ORACLE_EBADARG; break; }
      const int32_t* sel_row = sel_all + ((int64_t)b * p->seq_q + t) * Hkv * K;
      for (int32_t hq = 0; hq < Hq; ++hq) {
        const int32_t h = hq / G;
        const int32_t n = selected_tokens(p, sel_row + (int64_t)h * K, pos, tok);
        if (n < 0) { rc = ORACLE_EBADARG; break; }
        if (n == 0) continue;
        const int64_t qoff = (((int64_t)b * p->seq_q + t) * Hq + hq) * D;
        const int64_t kvbase = ((int64_t)b * Hkv + h) * p->seq_kv;
        const double* qv = q + qoff;
        const double* g = dout + qoff;
        /* softmax weights over the attended tokens */
        double zmax = -INFINITY;
        for (int32_t a = 0; a < n; ++a) {
          const double* kv = k + (kvbase + tok[a]) * D;
          double s = 0.0;
          for (int32_t d = 0; d < D; ++d) s += qv[d] * kv[d];
          w[a] = p->softmax_scale * s;
          if (w[a] > zmax) zmax = w[a];
        }
        double l = 0.0;
        for (int32_t a = 0; a < n; ++a) { w[a] = exp(w[a] - zmax); l += w[a]; }
        for (int32_t a = 0; a < n; ++a) w[a] /= l;
        /* the row's output and Dsum = dout . out */
        for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
        for (int32_t a = 0; a < n; ++a) {
          const double* vv = v + (kvbase + tok[a]) * D;
          for (int32_t d = 0; d < D; ++d) o[d] += w[a] * vv[d];
        }
        double dsum = 0.0;
        for (int32_t d = 0; d < D; ++d) dsum += g[d] * o[d];
        /* per token: dp, ds, and the three accumulations */
        for (int32_t a = 0; a < n; ++a) {
          const double* kv = k + (kvbase + tok[a]) * D;
          const double* vv = v + (kvbase + tok[a]) * D;
          double dp = 0.0;
          for (int32_t d = 0; d < D; ++d) dp += g[d] * vv[d];
          const double ds = w[a] * (dp - dsum);
          double* dkv = dk + (kvbase + tok[a]) * D;
          double* dvv = dv + (kvbase + tok[a]) * D;
          for (int32_t d = 0; d < D; ++d) {
            dq[qoff + d] += p->softmax_scale * ds * kv[d];
            dkv[d] += p->softmax_scale * ds * qv[d];
            dvv[d] += w[a] * g[d];
          }
        }
      }
    }
  }
  free(tok);
  free(w);
  free(o);
  return rc;
}

/* Index-branch KL loss and its gradient (see msa_oracle.h).  Per row (b, t)
 * and index head i with KV head h = i mod Hkv, over the tokens T that h
 * attends: P = the main branch's softmax over T averaged over h's query heads
 * (a target: nothing flows back into q or k), Q = softmax over T of the raw
 * index dot products, loss = sum_j P_j (log P_j - log Q_j); the loss's
 * derivative by index score j is Q_j - P_j. */
int oracle_index_kl(const oracle_problem* p, const double* q, const double* k, const double* iq,
                    const double* ik, const int32_t* seq_lens, const int32_t* sel_all,
                    double* loss, double* diq, double* dik) {
  if (!problem_ok(p) || !q || !k || !iq || !ik || !sel_all || !loss || !diq || !dik)
    return ORACLE_EBADARG;
  const int32_t D = p->head_dim, Di = p->idx_head_dim, K = p->top_k;
  const int32_t Hq = p->n_q_heads, Hkv = p->n_kv_heads, Hi = p->n_idx_heads;
  const int32_t G = Hq / Hkv;
  for (int64_t x = 0; x < (int64_t)p->batch * p->seq_q * Hi; ++x) loss[x] = 0.0;
  for (int64_t x = 0; x < (int64_t)p->batch * p->seq_q * Hi * Di; ++x) diq[x] = 0.0;
  for (int64_t x = 0; x < (int64_t)p->batch * p->seq_kv * Di; ++x) dik[x] = 0.0;
  const size_t cap = (size_t)K * p->block_size;
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * cap);
  double* P = (double*)malloc(sizeof(double) * cap);
  double* w = (double*)malloc(sizeof(double) * cap);
  double* Q = (double*)malloc(sizeof(double) * cap);
  if (!tok || !P || !w || !Q) { free(tok); free(P); free(w); free(Q); return ORACLE_ENOMEM; }
  int rc = ORACLE_OK;
  for (int32_t b = 0; b < p->batch && rc == ORACLE_OK; ++b) {
    for (int32_t t = 0; t < p->seq_q && rc == ORACLE_OK; ++t) {
      const int32_t pos = oracle_position(p, seq_lens, b, t);
      if (pos < 0) { rc = ORACLE_EBADARG; break; }
      const int32_t* sel_row = sel_all + ((int64_t)b * p->seq_q + t) * Hkv * K;
      for (int32_t i = 0; i < Hi; ++i) {
        const int32_t h = i % Hkv;
        const int32_t n = selected_tokens(p, sel_row + (int64_t)h * K, pos, tok);
        if (n < 0) { rc = ORACLE_EBADARG; break; }
        if (n == 0) continue;
        const int64_t kvbase = ((int64_t)b * Hkv + h) * p->seq_kv;
        /* P: the G query heads' softmax weights, averaged */
        for (int32_t a = 0; a < n; ++a) P[a] = 0.0;
        for (int32_t hq = h * G; hq < (h + 1) * G; ++hq) {
          const double* qv = q + (((int64_t)b * p->seq_q + t) * Hq + hq) * D;
          double zmax = -INFINITY;
          for (int32_t a = 0; a < n; ++a) {
            const double* kv = k + (kvbase + tok[a]) * D;
            double s = 0.0;
            for (int32_t d = 0; d < D; ++d) s += qv[d] * kv[d];
            w[a] = p->softmax_scale * s;
            if (w[a] > zmax) zmax = w[a];
          }
          double l = 0.0;
          for (int32_t a = 0; a < n; ++a) { w[a] = exp(w[a] - zmax); l += w[a]; }
          for (int32_t a = 0; a < n; ++a) P[a] += w[a] / l / G;
        }
        /* Q: softmax of the raw index dot products */
        const double* iv = iq + (((int64_t)b * p->seq_q + t) * Hi + i) * Di;
        double smax = -INFINITY;
        for (int32_t a = 0; a < n; ++a) {
          const double* kv = ik + ((int64_t)b * p->seq_kv + tok[a]) * Di;
          double s = 0.0;
          for (int32_t d = 0; d < Di; ++d) s += iv[d] * kv[d];
          Q[a] = s;
          if (s > smax) smax = s;
        }
        double lq = 0.0;
        for (int32_t a = 0; a < n; ++a) lq += exp(Q[a] - smax);
        const double lse = smax + log(lq);
        double kl = 0.0;
        for (int32_t a = 0; a < n; ++a) {
          const double logq = Q[a] - lse;
          Q[a] = exp(logq);
          if (P[a] > 0.0) kl += P[a] * (log(P[a]) - logq);
        }
        loss[((int64_t)b * p->seq_q + t) * Hi + i] = kl;
        /* d loss / d score_j = Q_j - P_j, into both factors of the dot product */
        double* dq_row = diq + (((int64_t)b * p->seq_q + t) * Hi + i) * Di;
        for (int32_t a = 0; a < n; ++a) {
          const double g = Q[a] - P[a];
          const double* kv = ik + ((int64_t)b * p->seq_kv + tok[a]) * Di;
          double* dk_row = dik + ((int64_t)b * p->seq_kv + tok[a]) * Di;
          for (int32_t d = 0; d < Di; ++d) {
            dq_row[d] += g * kv[d];
            dk_row[d] += g * iv[d];
          }
        }
      }
    }
  }
  free(tok);
  free(P);
  free(w);
  free(Q);
  return rc;
}
