/*
 * beam_topk_oracle.c -- CPU oracle for beam selection (one decode step).
 *
 * TEST INFRASTRUCTURE ONLY, like xattn_oracle.c: only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg use it; it shares no
 * code with the HIP library.
 *
 * Source: the xGR technical summary (gist.science, paper 2512.11529),
 * section 2.2 "xBeam": after each decode step every live beam proposes
 * candidates (its sorted next-token log-probabilities), a candidate's
 * score is the beam's cumulative score plus its log-probability, and the BW
 * best of all BW x V candidates become the next step's beams; the page's
 * kernel finds them with a global min-heap and stops scanning a beam once
 * its next candidate cannot enter the heap.  That search returns, by
 * definition, the BW largest candidates, so this oracle writes the
 * definition out: every candidate, one full sort, the first BW.
 *
 * Readings taken where the page is silent:
 *   - a score is the float32 sum cum[b] + logp[b][j] (the float decides
 *     integer outputs, so both sides round it the same way: one IEEE
 *     float32 addition);
 *   - the order is score descending, then parent beam ascending, then token
 *     id ascending (a total order, so the selection is unique);
 *   - the result is listed in that order: new beam i descends from
 *     parent[i] through token[i] and carries score[i].
 */
#include <stdint.h>
#include <stdlib.h>

typedef struct {
  float score;
  int32_t beam;
  int32_t token;
} cand_t;

/* qsort comparator: "a comes first" is negative */
static int cand_cmp(const void *pa, const void *pb) {
  const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  if (a->beam != b->beam) return a->beam < b->beam ? -1 : 1;
  if (a->token != b->token) return a->token < b->token ? -1 : 1;
  return 0;
}

/* For each of R requests: cum [BW], logp [BW][V] (each row sorted
 * descending; the oracle does not rely on it), token [BW][V].  Writes the
 * BW selected candidates to score [BW], parent [BW], new_token [BW].
 * Returns 0, or -1 for a bad size or a NaN input. */
int oracle_beam_topk(int32_t R, int32_t BW, int32_t V, const float *cum, const float *logp,
                     const int32_t *token, float *score, int32_t *parent, int32_t *new_token) {
  if (R < 1 || BW < 1 || V < 1) return -1;
  const int64_t n = (int64_t)BW * V;
  cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)n);
  if (!c) return -1;
  int bad = 0;
  for (int32_t r = 0; r < R; ++r) {
    for (int32_t b = 0; b < BW; ++b) {
      for (int32_t j = 0; j < V; ++j) {
        const int64_t e = ((int64_t)r * BW + b) * V + j;
        const float s = cum[(int64_t)r * BW + b] + logp[e];
        if (s != s) bad = 1;
        c[(int64_t)b * V + j].score = s;
        c[(int64_t)b * V + j].beam = b;
        c[(int64_t)b * V + j].token = token[e];
      }
    }
    qsort(c, (size_t)n, sizeof(cand_t), cand_cmp);
    for (int32_t i = 0; i < BW; ++i) {
      score[(int64_t)r * BW + i] = c[i].score;
      parent[(int64_t)r * BW + i] = c[i].beam;
      new_token[(int64_t)r * BW + i] = c[i].token;
    }
  }
  free(c);
  return bad ? -1 : 0;
}
