/*
 * moe_oracle.c -- plain, slow CPU oracle of the sparse Mixture-of-Experts layer
 * forward pass, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  It is called by the tests, by the smoke check and
 * by the CPU-baseline leg of the benchmark, and by nothing on the product path.
 * It shares no code, header or table with the HIP library.
 *
 * What it computes (the pages' definition, written out):
 *
 *   router        l_e = b_g[e] + sum_j x[j] W_g[e,j]
 *                 ("Mixture of Experts (MoE) and Mixtral", code block under
 *                 "Expert Routing": self.router is an nn.Linear; "Mixture of
 *                 Experts" (roadtointelligence), router formula x . W_g)
 *   softmax       p_e = exp(l_e - max l) / sum_e' exp(l_e' - max l)
 *   top-k         the k largest scores, slots in descending order, lowest
 *                 expert index first on equal scores
 *   renormalise   g_i = p_{e_i} / sum_j p_{e_j}
 *                 ("Mixture of Experts (MoE) and Mixtral", "Expert Routing",
 *                 renormalise step; matteuscruz "Architecture: router +
 *                 experts"); renormalize=0 keeps g_i = p_{e_i} as in the
 *                 codingnowai "Code" block
 *   capacity      per expert, walking tokens in index order, the first C
 *                 routed (token, slot) pairs are kept and the rest dropped
 *                 (matteuscruz "Load balancing", expert capacity buffer;
 *                 roadtointelligence "Keeping the experts busy")
 *   expert        E_e(x) = W2[e] act(W1[e] x + b1[e]) + b2[e], act = exact
 *                 GELU 0.5 z (1 + erf(z / sqrt 2)) or ReLU
 *                 ("Expert Routing" nn.Sequential(Linear, GELU, Linear);
 *                 codingnowai "Code" with ReLU)
 *   combine       y = sum_{kept slots i, ascending} g_i E_{e_i}(x)
 *                 (roadtointelligence display equation for y;
 *                 matteuscruz y = sum g_i Expert_i(x))
 *   shared        y += S(x), an always-on expert of gate 1.0
 *                 (roadtointelligence "Total versus active parameters":
 *                 1 shared expert beside 256 routed ones)
 *   statistics    mean_prob[e] = mean over tokens of p_e;
 *                 balance = unbiased variance of mean_prob over experts
 *                 ("Load Balancing: The Hidden Challenge", moe_loss:
 *                 torch.std(...) ** 2)
 *   expert choice each expert takes the C tokens of largest p_e, lower token
 *                 index first among equals; a token's output is the sum over
 *                 the experts that took it, in expert order, of p_e E_e(x)
 *                 (matteuscruz "Load balancing", expert choice routing)
 *
 * Precision: everything is fp64 except one decision: the top-k selection is
 * taken on the scores rounded to fp32, the precision the GPU router decides in.
 * Inputs stored as bf16 are widened exactly.
 *
 * Pins: tests/test_oracle_pins.py checks this file against the worked example of
 * the roadtointelligence page ("Tiny example"), closed forms and special cases
 * that reduce to torch CPU library routines.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_GELU 0
#define ORC_RELU 1

typedef struct {
  int64_t T;
  int32_t d, F, E, k;
  int32_t act;         /* ORC_GELU / ORC_RELU */
  int32_t dtype;       /* storage of x, W1, b1, W2, b2 and the shared expert */
  int32_t capacity;    /* < 0: unlimited */
  int32_t renormalize; /* 1: g_i = p_i / sum p over the top-k; 0: g_i = p_i */
  int32_t Fs;          /* shared expert d_ff, 0 = none */
} orc_config;

static double ld(const void *p, int32_t dtype, int64_t i) {
  if (dtype == ORC_F32) return (double)((const float *)p)[i];
  uint32_t u = ((uint32_t)((const uint16_t *)p)[i]) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double act_fn(int32_t act, double z) {
  if (act == ORC_RELU) return z > 0.0 ? z : 0.0;
  return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
}

/* Router scores of one token in fp64. */
static void scores(const orc_config *c, const void *x, const float *Wg, const float *bg, int64_t t,
                   double *l) {
  for (int32_t e = 0; e < c->E; ++e) {
    double s = 0.0;
    for (int32_t j = 0; j < c->d; ++j)
      s += ld(x, c->dtype, t * (int64_t)c->d + j) * (double)Wg[(int64_t)e * c->d + j];
    l[e] = (bg ? (double)bg[e] : 0.0) + s;
  }
}

/*
 * Routing for every token.
 *   topk_idx[T*k], topk_w[T*k]: slots in descending score order
 *   probs[T*E] (may be NULL): the full softmax
 *   counts[E]: routed (token, slot) pairs per expert; kept[E]: after capacity
 *   keep[T*k]: 1 if the slot survives capacity, else 0
 *   mean_prob[E], balance[1]: load statistics (NaN when undefined)
 * Returns 0, or -1 on bad arguments.
 */
int orc_route(const orc_config *c, const void *x, const float *Wg, const float *bg,
              int32_t *topk_idx, double *topk_w, double *probs, int32_t *counts, int32_t *kept,
              int32_t *keep, double *mean_prob, double *balance) {
  if (!c || c->E < 1 || c->k < 1 || c->k > c->E || c->d < 1 || c->T < 0) return -1;
  const int64_t T = c->T;
  const int32_t E = c->E, k = c->k;
  double *psum = (double *)calloc((size_t)E, sizeof(double));
  if (!psum) return -1;

#pragma omp parallel
  {
    double *l = (double *)malloc(sizeof(double) * E);
    double *p = (double *)malloc(sizeof(double) * E);
    float *l32 = (float *)malloc(sizeof(float) * E);
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      scores(c, x, Wg, bg, t, l);
      double m = l[0];
      for (int32_t e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
      double z = 0.0;
      for (int32_t e = 0; e < E; ++e) {
        p[e] = exp(l[e] - m);
        z += p[e];
      }
      for (int32_t e = 0; e < E; ++e) p[e] /= z;
      if (probs)
        for (int32_t e = 0; e < E; ++e) probs[t * E + e] = p[e];
      /* selection on fp32 scores, lowest index first among equals */
      for (int32_t e = 0; e < E; ++e) {
        l32[e] = (float)l[e];
        taken[e] = 0;
      }
      double sel = 0.0;
      for (int32_t i = 0; i < k; ++i) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e)
          if (!taken[e] && (best < 0 || l32[e] > l32[best])) best = e;
        taken[best] = 1;
        topk_idx[t * k + i] = best;
        sel += p[best];
      }
      for (int32_t i = 0; i < k; ++i) {
        double pi = p[topk_idx[t * k + i]];
        topk_w[t * k + i] = c->renormalize ? pi / sel : pi;
      }
    }
    free(l);
    free(p);
    free(l32);
    free(taken);
  }

  /* statistics: sums over tokens in token order */
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t i = 0; i < k; ++i) counts[topk_idx[t * k + i]] += 1;
  if (mean_prob || balance) {
    double *pt = (double *)malloc(sizeof(double) * E);
    double *lt = (double *)malloc(sizeof(double) * E);
    if (!probs) {
      /* recompute the softmax per token without storing it */
      for (int64_t t = 0; t < T; ++t) {
        scores(c, x, Wg, bg, t, lt);
        double m = lt[0], z = 0.0;
        for (int32_t e = 1; e < E; ++e) m = lt[e] > m ? lt[e] : m;
        for (int32_t e = 0; e < E; ++e) {
          pt[e] = exp(lt[e] - m);
          z += pt[e];
        }
        for (int32_t e = 0; e < E; ++e) psum[e] += pt[e] / z;
      }
    } else {
      for (int64_t t = 0; t < T; ++t)
        for (int32_t e = 0; e < E; ++e) psum[e] += probs[t * E + e];
    }
    free(pt);
    free(lt);
    double mean = 0.0;
    for (int32_t e = 0; e < E; ++e) {
      double mp = T > 0 ? psum[e] / (double)T : NAN;
      if (mean_prob) mean_prob[e] = mp;
      mean += mp;
    }
    mean /= (double)E;
    double v = 0.0;
    for (int32_t e = 0; e < E; ++e) {
      double mp = T > 0 ? psum[e] / (double)T : NAN;
      v += (mp - mean) * (mp - mean);
    }
    if (balance) *balance = E > 1 ? v / (double)(E - 1) : NAN;
  }
  free(psum);

  /* capacity: per expert, first C pairs in token order are kept */
  for (int32_t e = 0; e < E; ++e) kept[e] = 0;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t i = 0; i < k; ++i) {
      int32_t e = topk_idx[t * k + i];
      if (c->capacity < 0 || kept[e] < c->capacity) {
        keep[t * k + i] = 1;
        kept[e] += 1;
      } else {
        keep[t * k + i] = 0;
      }
    }
  return 0;
}

/*
 * The grouping that dispatch produces, derived from the routing: rows are
 * expert-major, token-ascending inside an expert, then one row per token for
 * the shared expert (if any).
 *   offsets[E+2]: offsets[e] = first row of expert e, offsets[E] = routed rows,
 *                 offsets[E+1] = offsets[E] + (Fs > 0 ? T : 0)
 *   row_token/row_slot[offsets[E+1]]: token and slot of each row (slot -1: shared)
 *   inv[T*k]: row of each (token, slot), -1 when dropped
 */
int orc_dispatch(const orc_config *c, const int32_t *topk_idx, const int32_t *keep,
                 int32_t *offsets, int32_t *row_token, int32_t *row_slot, int32_t *inv) {
  const int64_t T = c->T;
  const int32_t E = c->E, k = c->k;
  int32_t *n = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  int32_t *cur = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  if (!n || !cur) return -1;
  for (int64_t f = 0; f < T * k; ++f)
    if (keep[f]) n[topk_idx[f]] += 1;
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + n[e];
  for (int64_t t = 0; t < T; ++t)
    for (int32_t i = 0; i < k; ++i) {
      int64_t f = t * k + i;
      if (!keep[f]) {
        inv[f] = -1;
        continue;
      }
      int32_t e = topk_idx[f];
      int32_t r = offsets[e] + cur[e]++;
      row_token[r] = (int32_t)t;
      row_slot[r] = i;
      inv[f] = r;
    }
  offsets[E + 1] = offsets[E] + (c->Fs > 0 ? (int32_t)T : 0);
  if (c->Fs > 0)
    for (int64_t t = 0; t < T; ++t) {
      row_token[offsets[E] + t] = (int32_t)t;
      row_slot[offsets[E] + t] = -1;
    }
  free(n);
  free(cur);
  return 0;
}

/* out[0..d) = W2 act(W1 xt + b1) + b2 for one MLP; h is scratch of size Fm. */
static void mlp(const orc_config *c, int32_t Fm, const void *W1, const void *b1, const void *W2,
                const void *b2, int64_t w1off, int64_t b1off, int64_t w2off, int64_t b2off,
                const double *xt, double *h, double *out) {
  const int32_t d = c->d, dt = c->dtype;
  for (int32_t f = 0; f < Fm; ++f) {
    double s = 0.0;
    for (int32_t j = 0; j < d; ++j) s += ld(W1, dt, w1off + (int64_t)f * d + j) * xt[j];
    h[f] = act_fn(c->act, (b1 ? ld(b1, dt, b1off + f) : 0.0) + s);
  }
  for (int32_t o = 0; o < d; ++o) {
    double s = 0.0;
    for (int32_t f = 0; f < Fm; ++f) s += ld(W2, dt, w2off + (int64_t)o * Fm + f) * h[f];
    out[o] = (b2 ? ld(b2, dt, b2off + o) : 0.0) + s;
  }
}

/*
 * Layer outputs y[n*d + c] for the n_tok tokens listed in tokens[], given the
 * routing from orc_route.  W1 [E,F,d], b1 [E,F], W2 [E,d,F], b2 [E,d] in
 * nn.Linear layout; Ws1 [Fs,d], bs1 [Fs], Ws2 [d,Fs], bs2 [d] (NULL if none).
 * Bias pointers may be NULL (zero bias).
 */
int orc_experts(const orc_config *c, const void *x, const void *W1, const void *b1, const void *W2,
                const void *b2, const void *Ws1, const void *bs1, const void *Ws2, const void *bs2,
                const int32_t *topk_idx, const double *topk_w, const int32_t *keep,
                const int64_t *tokens, int64_t n_tok, double *y) {
  const int32_t d = c->d, F = c->F, k = c->k, Fs = c->Fs;
  const int32_t Fm = F > Fs ? F : Fs;
  int bad = 0;
#pragma omp parallel
  {
    double *xt = (double *)malloc(sizeof(double) * d);
    double *h = (double *)malloc(sizeof(double) * (Fm > 0 ? Fm : 1));
    double *o = (double *)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < n_tok; ++n) {
      int64_t t = tokens[n];
      if (t < 0 || t >= c->T) {
        bad = 1;
        continue;
      }
      for (int32_t j = 0; j < d; ++j) xt[j] = ld(x, c->dtype, t * d + j);
      double *yt = y + n * d;
      for (int32_t j = 0; j < d; ++j) yt[j] = 0.0;
      for (int32_t i = 0; i < k; ++i) {
        if (!keep[t * k + i]) continue;
        int64_t e = topk_idx[t * k + i];
        double g = topk_w[t * k + i];
        mlp(c, F, W1, b1, W2, b2, e * F * d, e * F, e * d * F, e * d, xt, h, o);
        for (int32_t j = 0; j < d; ++j) yt[j] += g * o[j];
      }
      if (Fs > 0) {
        mlp(c, Fs, Ws1, bs1, Ws2, bs2, 0, 0, 0, 0, xt, h, o);
        for (int32_t j = 0; j < d; ++j) yt[j] += o[j];
      }
    }
    free(xt);
    free(h);
    free(o);
  }
  return bad ? -1 : 0;
}

/*
 * One expert's (or the shared expert's, e = -1) gated output for one token:
 * out[0..d) = g * E_e(x_t).  Used to check per-row expert outputs.
 */
int orc_expert_row(const orc_config *c, const void *x, const void *W1, const void *b1,
                   const void *W2, const void *b2, const void *Ws1, const void *bs1,
                   const void *Ws2, const void *bs2, int64_t t, int32_t e, double g, double *out) {
  const int32_t d = c->d, F = c->F, Fs = c->Fs;
  const int32_t Fm = F > Fs ? F : Fs;
  if (t < 0 || t >= c->T || e >= c->E || (e < 0 && Fs <= 0)) return -1;
  double *xt = (double *)malloc(sizeof(double) * d);
  double *h = (double *)malloc(sizeof(double) * (Fm > 0 ? Fm : 1));
  for (int32_t j = 0; j < d; ++j) xt[j] = ld(x, c->dtype, t * d + j);
  if (e >= 0)
    mlp(c, F, W1, b1, W2, b2, (int64_t)e * F * d, (int64_t)e * F, (int64_t)e * d * F,
        (int64_t)e * d, xt, h, out);
  else
    mlp(c, Fs, Ws1, bs1, Ws2, bs2, 0, 0, 0, 0, xt, h, out);
  for (int32_t j = 0; j < d; ++j) out[j] *= g;
  free(xt);
  free(h);
  return 0;
}

/* Threads the parallel loops above use. */
int orc_threads(void) { return omp_get_max_threads(); }

/*
 * Squared coefficient of variation of the per-expert counts (invest-in.ai
 * "Common Usage Examples": cv_squared of the expert counts; matteuscruz "Load
 * balancing": the coefficient of variation of expert load): the unbiased
 * variance over the E experts divided by the squared mean.  0/0 gives NaN when
 * E = 1 or there are no pairs.
 */
double orc_cv2(const int32_t *counts, int32_t E) {
  double mean = 0.0;
  for (int32_t e = 0; e < E; ++e) mean += (double)counts[e];
  mean /= (double)E;
  double var = 0.0;
  for (int32_t e = 0; e < E; ++e) var += ((double)counts[e] - mean) * ((double)counts[e] - mean);
  var /= (double)(E - 1);
  return var / (mean * mean);
}

/* one (key, token) pair of an expert's ranking */
typedef struct {
  float key;
  int64_t t;
} orc_rank;

/* descending key, then ascending token */
static int orc_rank_cmp(const void *a, const void *b) {
  const orc_rank *x = (const orc_rank *)a, *y = (const orc_rank *)b;
  if (x->key != y->key) return x->key > y->key ? -1 : 1;
  return x->t < y->t ? -1 : (x->t > y->t ? 1 : 0);
}

/*
 * Expert-choice routing (matteuscruz "Load balancing": each expert selects its
 * top tokens instead of each token its top experts).  p[t*E + e] gets the fp64
 * router probabilities (softmax over experts, as in orc_route); expert e takes
 * the C tokens with the largest p[., e], the decision taken on p rounded to
 * fp32 (the precision the GPU decides in), lower token index first among
 * equals; sel[t*E + e] = 1 for the taken pairs, else 0.  C is clamped to [0, T].
 * Returns 0, or -1 on bad arguments.
 */
int orc_ec_select(const orc_config *c, const void *x, const float *Wg, const float *bg,
                  int64_t C, int32_t *sel, double *p) {
  if (!c || c->E < 1 || c->d < 1 || c->T < 0 || C < 0) return -1;
  const int64_t T = c->T;
  const int32_t E = c->E;
  if (C > T) C = T;
#pragma omp parallel
  {
    double *l = (double *)malloc(sizeof(double) * E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      scores(c, x, Wg, bg, t, l);
      double m = l[0];
      for (int32_t e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
      double z = 0.0;
      for (int32_t e = 0; e < E; ++e) {
        p[t * E + e] = exp(l[e] - m);
        z += p[t * E + e];
      }
      for (int32_t e = 0; e < E; ++e) {
        p[t * E + e] /= z;
        sel[t * E + e] = 0;
      }
    }
    free(l);
  }
  int bad = 0;
#pragma omp parallel
  {
    orc_rank *r = (orc_rank *)malloc(sizeof(orc_rank) * (T > 0 ? T : 1));
    if (!r) bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (int32_t e = 0; e < E; ++e) {
      if (!r) continue;
      for (int64_t t = 0; t < T; ++t) {
        r[t].key = (float)p[t * E + e];
        r[t].t = t;
      }
      qsort(r, (size_t)T, sizeof(orc_rank), orc_rank_cmp);
      for (int64_t i = 0; i < C; ++i) sel[r[i].t * E + e] = 1;
    }
    free(r);
  }
  return bad ? -1 : 0;
}
