/*
 * xattn_oracle.c -- CPU oracle for staged beam-search decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * Source of the method: the xGR technical summary (gist.science, paper
 * 2512.11529), section 2.1 "xAttention".  That section describes
 *   - a KV cache split into a Shared part (the prompt / user history, written
 *     once at prefill and read for every beam) and an Unshared part (only the
 *     tokens generated during decode, kept per token rather than per block,
 *     so no block is copied when beams branch);
 *   - attention computed in three stages: Shared and Unshared each produce
 *     local scores plus max/sum statistics on their own, and a Merging stage
 *     combines the two with OnlineSoftmax.
 * The page gives no formula.  Because the split-and-merge is an exact
 * identity in real arithmetic, the result is by definition ordinary softmax
 * attention of each query over the concatenated key sequence
 *     [ shared rows 0..L_r-1 ; the beam's own generated token at every level
 *       0..s, found by following the per-step parent indices back from the
 *       beam's current slot ].
 * oracle_attend() below is that definition written out in float64.
 * oracle_stage_partials() and oracle_merge() are the per-stage statistics
 * and the OnlineSoftmax combine (the standard online-normaliser / split
 * softmax combine), used only to check a kernel's stage outputs.
 *
 * Readings taken where the page is silent (each one is listed with its
 * reason in the design notes of the repository):
 *   - levels are 0-based; at step s levels 0..s are all attended (the current
 *     token's K/V is written before attention runs);
 *   - parent_idx[r][t][b] is the level t-1 slot that the level-t beam in slot
 *     b descends from; row t = 0 is never read;
 *   - query head h reads KV head h / (Hq / Hkv) (contiguous GQA groups);
 *   - no masking inside the valid ranges; shared rows j >= L_r and levels
 *     above s are never read;
 *   - L_r = 0 is allowed: the shared partial is then empty (m = -inf, l = 0,
 *     o = 0) and the result is attention over the ancestor tokens only.
 *
 * Inputs are read in their stored type (fp32, or bf16 bit patterns) and
 * widened exactly to double before any arithmetic.
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t R;       /* requests */
  int32_t BW;      /* beam width (slots per level) */
  int32_t Hq;      /* query heads */
  int32_t Hkv;     /* key/value heads; Hq % Hkv == 0 */
  int32_t D;       /* head dimension */
  int32_t Lmax;    /* row capacity of the shared cache */
  int32_t S;       /* level capacity of the unshared cache */
  int32_t dtype;   /* 0 = float32, 1 = bfloat16 (raw 16-bit patterns) */
  double scale;    /* softmax scale applied to q.k */
} oracle_shape;

/* Exact widening of one stored element to double. */
static double elem(const void *base, int64_t i, int32_t dtype) {
  if (dtype == 0) return (double)((const float *)base)[i];
  uint32_t w = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* Ancestor slots of every beam: anc[r][b][t] for t = 0..step.
 * The beam in slot b at level `step` is its own level-`step` token; its
 * level t-1 ancestor is parent_idx[r][t][its level-t slot].
 * Returns 0, or -1 if a parent index lies outside [0, BW). */
int oracle_ancestors(int32_t R, int32_t BW, int32_t S, const int32_t *parent_idx,
                     int32_t step, int32_t *anc) {
  if (step < 0 || step >= S) return -1;
  for (int32_t r = 0; r < R; ++r) {
    for (int32_t b = 0; b < BW; ++b) {
      int32_t *row = anc + ((int64_t)r * BW + b) * (step + 1);
      int32_t a = b;
      row[step] = a;
      for (int32_t t = step; t >= 1; --t) {
        a = parent_idx[((int64_t)r * S + t) * BW + a];
        if (a < 0 || a >= BW) return -1;
        row[t - 1] = a;
      }
    }
  }
  return 0;
}

/* Offsets of the row vectors the definition refers to. */
static int64_t q_off(const oracle_shape *s, int32_t r, int32_t b, int32_t h) {
  return (((int64_t)r * s->BW + b) * s->Hq + h) * s->D;
}
static int64_t shared_off(const oracle_shape *s, int32_t r, int32_t k, int32_t j) {
  return (((int64_t)r * s->Hkv + k) * s->Lmax + j) * s->D;
}
static int64_t unshared_off(const oracle_shape *s, int32_t r, int32_t k, int32_t t,
                            int32_t slot) {
  return ((((int64_t)r * s->Hkv + k) * s->S + t) * s->BW + slot) * s->D;
}

/* One attended key: a dot product with the query, times the scale. */
static double score(const oracle_shape *s, const void *q, int64_t qo, const void *kbuf,
                    int64_t ko) {
  double acc = 0.0;
  for (int32_t d = 0; d < s->D; ++d)
    acc += elem(q, qo + d, s->dtype) * elem(kbuf, ko + d, s->dtype);
  return s->scale * acc;
}

/* Rows to evaluate: rows == NULL means every (r, b, h) in row-major order. */
static void row_at(const oracle_shape *s, const int32_t *rows, int64_t i, int32_t *r,
                   int32_t *b, int32_t *h) {
  if (rows) {
    *r = rows[3 * i];
    *b = rows[3 * i + 1];
    *h = rows[3 * i + 2];
  } else {
    *h = (int32_t)(i % s->Hq);
    *b = (int32_t)((i / s->Hq) % s->BW);
    *r = (int32_t)(i / ((int64_t)s->Hq * s->BW));
  }
}

static int check_args(const oracle_shape *s, int32_t step) {
  if (!s || s->R < 1 || s->BW < 1 || s->Hkv < 1 || s->Hq < s->Hkv || s->Hq % s->Hkv)
    return -1;
  if (s->D < 1 || s->Lmax < 0 || s->S < 1 || step < 0 || step >= s->S) return -1;
  if (s->dtype != 0 && s->dtype != 1) return -1;
  return 0;
}

/* The definition: softmax attention of query (r, b, h) over the
 * concatenation of its request's first L_r shared rows and its beam's
 * ancestor tokens at levels 0..step.  out is n_rows x D, lse is n_rows
 * (log of the softmax denominator, scores in the scaled units). */
int oracle_attend(const oracle_shape *s, const void *q, const void *shared_k,
                  const void *shared_v, const int32_t *prompt_len,
                  const void *unshared_k, const void *unshared_v,
                  const int32_t *parent_idx, int32_t step, int64_t n_rows,
                  const int32_t *rows, double *out, double *lse) {
  if (check_args(s, step)) return -1;
  const int32_t G = s->Hq / s->Hkv;
  const int64_t n_total = rows ? n_rows : (int64_t)s->R * s->BW * s->Hq;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
  for (int64_t i = 0; i < n_total; ++i) {
    int32_t r, b, h;
    row_at(s, rows, i, &r, &b, &h);
    if (r < 0 || r >= s->R || b < 0 || b >= s->BW || h < 0 || h >= s->Hq) {
      bad = 1;
      continue;
    }
    const int32_t k = h / G;
    const int32_t L = prompt_len[r];
    if (L < 0 || L > s->Lmax) {
      bad = 1;
      continue;
    }
    /* ancestor slot at each level */
    int32_t *anc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(step + 1));
    int32_t a = b;
    anc[step] = a;
    for (int32_t t = step; t >= 1; --t) {
      a = parent_idx[((int64_t)r * s->S + t) * s->BW + a];
      if (a < 0 || a >= s->BW) {
        bad = 1;
        a = 0;
      }
      anc[t - 1] = a;
    }
    const int64_t n_keys = (int64_t)L + step + 1;
    double *x = (double *)malloc(sizeof(double) * (size_t)n_keys);
    const int64_t qo = q_off(s, r, b, h);
    for (int64_t j = 0; j < L; ++j) x[j] = score(s, q, qo, shared_k, shared_off(s, r, k, (int32_t)j));
    for (int32_t t = 0; t <= step; ++t)
      x[L + t] = score(s, q, qo, unshared_k, unshared_off(s, r, k, t, anc[t]));
    double mx = -INFINITY;
    for (int64_t n = 0; n < n_keys; ++n) mx = x[n] > mx ? x[n] : mx;
    double z = 0.0;
    for (int64_t n = 0; n < n_keys; ++n) {
      x[n] = exp(x[n] - mx);
      z += x[n];
    }
    double *o = out + i * s->D;
    for (int32_t d = 0; d < s->D; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < L; ++j) {
      const int64_t vo = shared_off(s, r, k, (int32_t)j);
      for (int32_t d = 0; d < s->D; ++d) o[d] += x[j] * elem(shared_v, vo + d, s->dtype);
    }
    for (int32_t t = 0; t <= step; ++t) {
      const int64_t vo = unshared_off(s, r, k, t, anc[t]);
      for (int32_t d = 0; d < s->D; ++d) o[d] += x[L + t] * elem(unshared_v, vo + d, s->dtype);
    }
    for (int32_t d = 0; d < s->D; ++d) o[d] /= z;
    if (lse) lse[i] = mx + log(z);
    free(x);
    free(anc);
  }
  return bad ? -1 : 0;
}

/* Local softmax statistics of one stage over its own key set:
 * m = max score, l = sum exp(score - m), o = sum exp(score - m) v / l.
 * An empty key set gives m = -inf, l = 0, o = 0. */
static void softmax_stats(const double *x, int64_t n, double *m, double *l) {
  double mx = -INFINITY;
  for (int64_t j = 0; j < n; ++j) mx = x[j] > mx ? x[j] : mx;
  double z = 0.0;
  for (int64_t j = 0; j < n; ++j) z += exp(x[j] - mx);
  *m = mx;
  *l = n ? z : 0.0;
}

/* Stage partials for the Shared stage (shared rows 0..L_r-1) and the
 * Unshared stage (ancestor tokens, levels 0..step), each on its own.
 * *_ml is n_rows x 2 (m, l); *_o is n_rows x D (normalised output). */
int oracle_stage_partials(const oracle_shape *s, const void *q, const void *shared_k,
                          const void *shared_v, const int32_t *prompt_len,
                          const void *unshared_k, const void *unshared_v,
                          const int32_t *parent_idx, int32_t step, int64_t n_rows,
                          const int32_t *rows, double *shared_ml, double *shared_o,
                          double *unshared_ml, double *unshared_o) {
  if (check_args(s, step)) return -1;
  const int32_t G = s->Hq / s->Hkv;
  const int64_t n_total = rows ? n_rows : (int64_t)s->R * s->BW * s->Hq;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
  for (int64_t i = 0; i < n_total; ++i) {
    int32_t r, b, h;
    row_at(s, rows, i, &r, &b, &h);
    if (r < 0 || r >= s->R || b < 0 || b >= s->BW || h < 0 || h >= s->Hq) {
      bad = 1;
      continue;
    }
    const int32_t k = h / G;
    const int32_t L = prompt_len[r];
    if (L < 0 || L > s->Lmax) {
      bad = 1;
      continue;
    }
    const int64_t qo = q_off(s, r, b, h);
    /* Shared stage */
    double *xs = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    for (int64_t j = 0; j < L; ++j) xs[j] = score(s, q, qo, shared_k, shared_off(s, r, k, (int32_t)j));
    double ms, ls;
    softmax_stats(xs, L, &ms, &ls);
    double *os = shared_o + i * s->D;
    for (int32_t d = 0; d < s->D; ++d) os[d] = 0.0;
    for (int64_t j = 0; j < L; ++j) {
      const double w = exp(xs[j] - ms);
      const int64_t vo = shared_off(s, r, k, (int32_t)j);
      for (int32_t d = 0; d < s->D; ++d) os[d] += w * elem(shared_v, vo + d, s->dtype);
    }
    if (L > 0)
      for (int32_t d = 0; d < s->D; ++d) os[d] /= ls;
    shared_ml[2 * i] = ms;
    shared_ml[2 * i + 1] = ls;
    free(xs);
    /* Unshared stage: the beam's ancestor token at every level */
    double *xu = (double *)malloc(sizeof(double) * (size_t)(step + 1));
    int32_t *anc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(step + 1));
    int32_t a = b;
    anc[step] = a;
    for (int32_t t = step; t >= 1; --t) {
      a = parent_idx[((int64_t)r * s->S + t) * s->BW + a];
      if (a < 0 || a >= s->BW) {
        bad = 1;
        a = 0;
      }
      anc[t - 1] = a;
    }
    for (int32_t t = 0; t <= step; ++t)
      xu[t] = score(s, q, qo, unshared_k, unshared_off(s, r, k, t, anc[t]));
    double mu, lu;
    softmax_stats(xu, step + 1, &mu, &lu);
    double *ou = unshared_o + i * s->D;
    for (int32_t d = 0; d < s->D; ++d) ou[d] = 0.0;
    for (int32_t t = 0; t <= step; ++t) {
      const double w = exp(xu[t] - mu);
      const int64_t vo = unshared_off(s, r, k, t, anc[t]);
      for (int32_t d = 0; d < s->D; ++d) ou[d] += w * elem(unshared_v, vo + d, s->dtype);
    }
    for (int32_t d = 0; d < s->D; ++d) ou[d] /= lu;
    unshared_ml[2 * i] = mu;
    unshared_ml[2 * i + 1] = lu;
    free(xu);
    free(anc);
  }
  return bad ? -1 : 0;
}

/* OnlineSoftmax combine of two stage partials (m, l, o) for n rows:
 *   m = max(m_a, m_b); w_a = l_a e^{m_a - m}; w_b = l_b e^{m_b - m};
 *   out = (w_a o_a + w_b o_b) / (w_a + w_b);  lse = m + ln(w_a + w_b).
 * A partial with l = 0 (an empty key set, m = -inf) gets weight 0 and its
 * m is never subtracted from itself.  Both empty gives out = 0, lse = -inf. */
void oracle_merge(int64_t n, int32_t D, const double *ml_a, const double *o_a,
                  const double *ml_b, const double *o_b, double *out, double *lse) {
  for (int64_t i = 0; i < n; ++i) {
    const double ma = ml_a[2 * i], la = ml_a[2 * i + 1];
    const double mb = ml_b[2 * i], lb = ml_b[2 * i + 1];
    const double m = ma > mb ? ma : mb;
    const double wa = la > 0.0 ? la * exp(ma - m) : 0.0;
    const double wb = lb > 0.0 ? lb * exp(mb - m) : 0.0;
    const double z = wa + wb;
    for (int32_t d = 0; d < D; ++d)
      out[i * D + d] = z > 0.0 ? (wa * o_a[i * D + d] + wb * o_b[i * D + d]) / z : 0.0;
    if (lse) lse[i] = z > 0.0 ? m + log(z) : -INFINITY;
  }
}
