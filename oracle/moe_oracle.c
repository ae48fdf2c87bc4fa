/*
 * moe_oracle.c -- plain, slow CPU oracle of the sparse Mixture-of-Experts layer
 * forward and backward passes, in fp64.
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
 *   backward      gradients of sum_t <dy_t, y_t> + alpha * balance with the
 *                 selection and the drops held fixed (the chain rule written
 *                 out above orc_backward); expert choice is the same chain
 *                 rule with every expert a slot, the selection as the keep
 *                 mask, gates p[t, e] and no renormalisation
 *
 * Precision: everything is fp64 except one decision: the top-k selection is
 * taken on the scores rounded to fp32, the precision the GPU router decides in.
 * Inputs stored as bf16 are widened exactly.
 *
 * Pins: tests/test_oracle_pins.py checks this file against the worked example of
 * the roadtointelligence page ("Tiny example"), closed forms and special cases
 * that reduce to torch CPU library routines; tests/test_oracle_backward_pins.py
 * checks the backward against torch autograd, central finite differences of
 * the forward, and closed forms.
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

/* ------------------------------------------------------------------------- */
/*
 * Backward pass of the token-choice layer.
 *
 * The loss whose gradients are returned is
 *     L = sum_t <dy_t, y_t> + alpha * balance
 * (dy: the upstream gradient of the layer output; balance: the unbiased
 * variance over experts of the mean router probability, the statistic of
 * botmartz "Load Balancing: The Hidden Challenge" moe_loss, which the training
 * objective adds with a small coefficient: botmartz total_loss with 0.01,
 * roadtointelligence "Keeping the experts busy", matteuscruz "Load
 * balancing").  The top-k selection and the capacity drops are taken as fixed
 * (they are piecewise constant in the inputs), as autograd treats them.
 *
 * Chain rule, per token t and kept slot i (expert e, gate g_i, MLP output o_i):
 *   dO_i   = g_i dy_t
 *   dW2[e] += dO_i h_i^T      db2[e] += dO_i      dh_i = W2[e]^T dO_i
 *   dz_i   = dh_i * act'(z_i) (GELU: Phi(z) + z phi(z); ReLU: 1 if z > 0 else 0)
 *   dW1[e] += dz_i x_t^T      db1[e] += dz_i      dx_t += W1[e]^T dz_i
 *   dg_i   = <dy_t, o_i>      (0 for a dropped slot)
 * the shared expert likewise with gate 1 and no dg; then the gates:
 *   renormalised g_i = p_{e_i} / S, S = sum over all k slots of p:
 *       dp_{e_j} = (dg_j - sum_i dg_i g_i) / S;  otherwise dp_{e_j} = dg_j;
 *       dp_e = 0 for experts outside the top-k
 *   auxiliary term (E > 1): balance = sum_e (m_e - mean m)^2 / (E - 1) with
 *       m_e = (1/T) sum_t p_{t,e}, so dp_{t,e} += alpha 2 (m_e - mean m) / ((E-1) T)
 *       (E = 1: the variance is undefined and the term is taken as zero)
 *   softmax: dl_e = p_e (dp_e - sum_f p_f dp_f)
 *   router:  dWg[e] += dl_e x_t,  dbg[e] += dl_e,  dx_t += sum_e dl_e Wg[e]
 */

typedef struct {
  const float *Wg, *bg;
  const void *W1, *b1, *W2, *b2, *Ws1, *bs1, *Ws2, *bs2;
} orc_weights;

/* fp64 gradients; any member may be NULL (not wanted) */
typedef struct {
  double *dx, *dWg, *dbg, *dW1, *db1, *dW2, *db2, *dWs1, *dbs1, *dWs2, *dbs2;
} orc_grads;

static double act_grad(int32_t act, double z) {
  if (act == ORC_RELU) return z > 0.0 ? 1.0 : 0.0;
  const double inv_sqrt_2pi = 0.39894228040143267794;
  return 0.5 * (1.0 + erf(z / sqrt(2.0))) + z * exp(-0.5 * z * z) * inv_sqrt_2pi;
}

/*
 * One MLP (d -> Fm -> d) for one token: xt, and go = the gradient of its
 * output.  Writes its output to o (if given), adds W1^T dz to dxt, and adds to
 * the weight-gradient accumulators that are given.  z, h, dz: scratch [Fm].
 */
static void mlp_bwd(const orc_config *c, int32_t Fm, const void *W1, const void *b1,
                    const void *W2, const void *b2, int64_t w1off, int64_t b1off, int64_t w2off,
                    int64_t b2off, const double *xt, const double *go, double *o, double *dxt,
                    double *z, double *h, double *dz, double *dW1, double *db1, double *dW2,
                    double *db2) {
  const int32_t d = c->d, dt = c->dtype;
  for (int32_t f = 0; f < Fm; ++f) {
    double s = 0.0;
    for (int32_t j = 0; j < d; ++j) s += ld(W1, dt, w1off + (int64_t)f * d + j) * xt[j];
    z[f] = (b1 ? ld(b1, dt, b1off + f) : 0.0) + s;
    h[f] = act_fn(c->act, z[f]);
  }
  if (o)
    for (int32_t j = 0; j < d; ++j) {
      double s = 0.0;
      for (int32_t f = 0; f < Fm; ++f) s += ld(W2, dt, w2off + (int64_t)j * Fm + f) * h[f];
      o[j] = (b2 ? ld(b2, dt, b2off + j) : 0.0) + s;
    }
  for (int32_t f = 0; f < Fm; ++f) {
    double s = 0.0;
    for (int32_t j = 0; j < d; ++j) s += ld(W2, dt, w2off + (int64_t)j * Fm + f) * go[j];
    dz[f] = s * act_grad(c->act, z[f]);
  }
  for (int32_t j = 0; j < d; ++j) {
    double s = 0.0;
    for (int32_t f = 0; f < Fm; ++f) s += ld(W1, dt, w1off + (int64_t)f * d + j) * dz[f];
    dxt[j] += s;
  }
  if (dW2)
    for (int32_t j = 0; j < d; ++j)
      for (int32_t f = 0; f < Fm; ++f) dW2[(int64_t)j * Fm + f] += go[j] * h[f];
  if (db2)
    for (int32_t j = 0; j < d; ++j) db2[j] += go[j];
  if (dW1)
    for (int32_t f = 0; f < Fm; ++f)
      for (int32_t j = 0; j < d; ++j) dW1[(int64_t)f * d + j] += dz[f] * xt[j];
  if (db1)
    for (int32_t f = 0; f < Fm; ++f) db1[f] += dz[f];
}

/* scratch of one token's backward */
typedef struct {
  double *xt, *l, *p, *dp, *go, *o, *z, *h, *dz, *dg;
} bwd_scratch;

static int scratch_alloc(bwd_scratch *s, const orc_config *c) {
  const int32_t Fm = c->F > c->Fs ? c->F : c->Fs;
  s->xt = (double *)malloc(sizeof(double) * c->d);
  s->l = (double *)malloc(sizeof(double) * c->E);
  s->p = (double *)malloc(sizeof(double) * c->E);
  s->dp = (double *)malloc(sizeof(double) * c->E);
  s->go = (double *)malloc(sizeof(double) * c->d);
  s->o = (double *)malloc(sizeof(double) * c->d);
  s->z = (double *)malloc(sizeof(double) * (Fm > 0 ? Fm : 1));
  s->h = (double *)malloc(sizeof(double) * (Fm > 0 ? Fm : 1));
  s->dz = (double *)malloc(sizeof(double) * (Fm > 0 ? Fm : 1));
  s->dg = (double *)malloc(sizeof(double) * c->k);
  return s->xt && s->l && s->p && s->dp && s->go && s->o && s->z && s->h && s->dz && s->dg;
}

static void scratch_free(bwd_scratch *s) {
  free(s->xt);
  free(s->l);
  free(s->p);
  free(s->dp);
  free(s->go);
  free(s->o);
  free(s->z);
  free(s->h);
  free(s->dz);
  free(s->dg);
}

/*
 * Backward of token t.  idx, gw, keep: the token's k slots from orc_route;
 * mean_prob [E] from orc_route.  Writes dxt [d], dlt [E] (router-score
 * gradient) and dgt [k] (gate gradient) when given; adds to the accumulators
 * of acc (dx is not used there) that are given.
 */
static void bwd_token(const orc_config *c, const void *x, const orc_weights *w, int64_t t,
                      const double *dyt, double alpha, const int32_t *idx, const double *gw,
                      const int32_t *keep, const double *mean_prob, bwd_scratch *s, double *dxt,
                      double *dlt, double *dgt, const orc_grads *acc) {
  const int32_t d = c->d, E = c->E, k = c->k, F = c->F, Fs = c->Fs;
  for (int32_t j = 0; j < d; ++j) {
    s->xt[j] = ld(x, c->dtype, t * d + j);
    dxt[j] = 0.0;
  }
  scores(c, x, w->Wg, w->bg, t, s->l);
  double m = s->l[0], zsum = 0.0;
  for (int32_t e = 1; e < E; ++e) m = s->l[e] > m ? s->l[e] : m;
  for (int32_t e = 0; e < E; ++e) {
    s->p[e] = exp(s->l[e] - m);
    zsum += s->p[e];
  }
  for (int32_t e = 0; e < E; ++e) s->p[e] /= zsum;

  /* routed experts */
  double *dg = dgt ? dgt : s->dg;
  for (int32_t i = 0; i < k; ++i) {
    dg[i] = 0.0;
    if (!keep[i]) continue;
    const int64_t e = idx[i];
    for (int32_t j = 0; j < d; ++j) s->go[j] = gw[i] * dyt[j];
    mlp_bwd(c, F, w->W1, w->b1, w->W2, w->b2, e * F * d, e * F, e * d * F, e * d, s->xt, s->go,
            s->o, dxt, s->z, s->h, s->dz, acc && acc->dW1 ? acc->dW1 + e * F * d : NULL,
            acc && acc->db1 ? acc->db1 + e * F : NULL,
            acc && acc->dW2 ? acc->dW2 + e * d * F : NULL,
            acc && acc->db2 ? acc->db2 + e * d : NULL);
    double g = 0.0;
    for (int32_t j = 0; j < d; ++j) g += dyt[j] * s->o[j];
    dg[i] = g;
  }
  /* shared expert: gate 1, nothing flows to the router */
  if (Fs > 0)
    mlp_bwd(c, Fs, w->Ws1, w->bs1, w->Ws2, w->bs2, 0, 0, 0, 0, s->xt, dyt, NULL, dxt, s->z,
            s->h, s->dz, acc ? acc->dWs1 : NULL, acc ? acc->dbs1 : NULL,
            acc ? acc->dWs2 : NULL, acc ? acc->dbs2 : NULL);

  /* gates -> probabilities */
  for (int32_t e = 0; e < E; ++e) s->dp[e] = 0.0;
  if (c->renormalize) {
    double S = 0.0, dot = 0.0;
    for (int32_t i = 0; i < k; ++i) {
      S += s->p[idx[i]];
      dot += dg[i] * gw[i];
    }
    for (int32_t i = 0; i < k; ++i) s->dp[idx[i]] = (dg[i] - dot) / S;
  } else {
    for (int32_t i = 0; i < k; ++i) s->dp[idx[i]] = dg[i];
  }
  if (alpha != 0.0 && E > 1) {
    double mbar = 0.0;
    for (int32_t e = 0; e < E; ++e) mbar += mean_prob[e];
    mbar /= (double)E;
    for (int32_t e = 0; e < E; ++e)
      s->dp[e] += alpha * 2.0 * (mean_prob[e] - mbar) / ((double)(E - 1) * (double)c->T);
  }
  /* softmax -> scores -> router parameters and x */
  double sp = 0.0;
  for (int32_t e = 0; e < E; ++e) sp += s->p[e] * s->dp[e];
  for (int32_t e = 0; e < E; ++e) {
    const double dl = s->p[e] * (s->dp[e] - sp);
    if (dlt) dlt[e] = dl;
    for (int32_t j = 0; j < d; ++j) dxt[j] += dl * (double)w->Wg[(int64_t)e * d + j];
    if (acc && acc->dWg)
      for (int32_t j = 0; j < d; ++j) acc->dWg[(int64_t)e * d + j] += dl * s->xt[j];
    if (acc && acc->dbg) acc->dbg[e] += dl;
  }
}

/*
 * The whole backward: every gradient of g that is not NULL, over all tokens
 * in token order (serial; small shapes).  dy [T*d] fp64; topk_idx, topk_w,
 * keep, mean_prob from orc_route.  Returns 0, or -1 on bad arguments.
 */
int orc_backward(const orc_config *c, const void *x, const orc_weights *w, const double *dy,
                 double alpha, const int32_t *topk_idx, const double *topk_w,
                 const int32_t *keep, const double *mean_prob, const orc_grads *g) {
  if (!c || c->k < 1 || c->T < 0) return -1;
  const int64_t T = c->T;
  const int32_t d = c->d, E = c->E, F = c->F, Fs = c->Fs;
  /* zero every requested output */
  struct {
    double *p;
    int64_t n;
  } outs[] = {{g->dx, T * d},
              {g->dWg, (int64_t)E * d},
              {g->dbg, E},
              {g->dW1, (int64_t)E * F * d},
              {g->db1, (int64_t)E * F},
              {g->dW2, (int64_t)E * d * F},
              {g->db2, (int64_t)E * d},
              {g->dWs1, (int64_t)Fs * d},
              {g->dbs1, Fs},
              {g->dWs2, (int64_t)d * Fs},
              {g->dbs2, Fs > 0 ? d : 0}};
  for (size_t i = 0; i < sizeof outs / sizeof outs[0]; ++i)
    if (outs[i].p) memset(outs[i].p, 0, sizeof(double) * (size_t)outs[i].n);
  bwd_scratch s;
  double *dxt = (double *)malloc(sizeof(double) * d);
  int ok = scratch_alloc(&s, c) && dxt;
  for (int64_t t = 0; ok && t < T; ++t) {
    bwd_token(c, x, w, t, dy + t * d, alpha, topk_idx + t * c->k, topk_w + t * c->k,
              keep + t * c->k, mean_prob, &s, dxt, NULL, NULL, g);
    if (g->dx) memcpy(g->dx + t * d, dxt, sizeof(double) * d);
  }
  scratch_free(&s);
  free(dxt);
  return ok ? 0 : -1;
}

/*
 * Input gradient, router-score gradient and gate gradient of the n_tok tokens
 * listed in tokens[] (each token's backward is independent given mean_prob):
 * dx [n*d], dl [n*E], dg [n*k] (each may be NULL).
 */
int orc_backward_tokens(const orc_config *c, const void *x, const orc_weights *w,
                        const double *dy, double alpha, const int32_t *topk_idx,
                        const double *topk_w, const int32_t *keep, const double *mean_prob,
                        const int64_t *tokens, int64_t n_tok, double *dx, double *dl,
                        double *dg) {
  if (!c || c->k < 1) return -1;
  const int32_t d = c->d, E = c->E, k = c->k;
  int bad = 0;
#pragma omp parallel
  {
    bwd_scratch s;
    double *dxt = (double *)malloc(sizeof(double) * d);
    if (!scratch_alloc(&s, c) || !dxt) bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < n_tok; ++n) {
      const int64_t t = tokens[n];
      if (bad || t < 0 || t >= c->T) {
        bad = 1;
        continue;
      }
      bwd_token(c, x, w, t, dy + t * d, alpha, topk_idx + t * k, topk_w + t * k, keep + t * k,
                mean_prob, &s, dxt, dl ? dl + n * E : NULL, dg ? dg + n * k : NULL, NULL);
      if (dx) memcpy(dx + n * d, dxt, sizeof(double) * d);
    }
    scratch_free(&s);
    free(dxt);
  }
  return bad ? -1 : 0;
}

/*
 * Selected entries of one expert's weight gradients (e = -1: the shared
 * expert), summed over the rows that expert received, in token order:
 *   dW1[a*nj + b] = dW1[e][f_list[a]][j_list[b]]   db1[a] = db1[e][f_list[a]]
 *   dW2[b*nf + a] = dW2[e][j_list[b]][f_list[a]]   db2[b] = db2[e][j_list[b]]
 * Each row costs O(nf * d), so entries of large layers are cheap to check.
 */
int orc_backward_expert_entries(const orc_config *c, const void *x, const orc_weights *w,
                                const double *dy, const int32_t *topk_idx, const double *topk_w,
                                const int32_t *keep, int32_t e, int32_t nf,
                                const int32_t *f_list, int32_t nj, const int32_t *j_list,
                                double *dW1, double *db1, double *dW2, double *db2) {
  if (!c || e >= c->E || (e < 0 && c->Fs <= 0)) return -1;
  const int64_t T = c->T;
  const int32_t d = c->d, k = c->k, dt = c->dtype;
  const int32_t Fm = e >= 0 ? c->F : c->Fs;
  const void *W1 = e >= 0 ? w->W1 : w->Ws1, *b1 = e >= 0 ? w->b1 : w->bs1;
  const void *W2 = e >= 0 ? w->W2 : w->Ws2;
  const int64_t w1off = e >= 0 ? (int64_t)e * Fm * d : 0, b1off = e >= 0 ? (int64_t)e * Fm : 0;
  const int64_t w2off = e >= 0 ? (int64_t)e * d * Fm : 0;
  for (int32_t a = 0; a < nf; ++a) {
    if (f_list[a] < 0 || f_list[a] >= Fm) return -1;
    db1[a] = 0.0;
    for (int32_t b = 0; b < nj; ++b) dW1[(int64_t)a * nj + b] = dW2[(int64_t)b * nf + a] = 0.0;
  }
  for (int32_t b = 0; b < nj; ++b) {
    if (j_list[b] < 0 || j_list[b] >= d) return -1;
    db2[b] = 0.0;
  }
  double *xt = (double *)malloc(sizeof(double) * d);
  double *go = (double *)malloc(sizeof(double) * d);
  if (!xt || !go) return -1;
  for (int64_t t = 0; t < T; ++t) {
    double g = -1.0;
    if (e < 0) {
      g = 1.0;
    } else {
      for (int32_t i = 0; i < k; ++i)
        if (keep[t * k + i] && topk_idx[t * k + i] == e) g = topk_w[t * k + i];
    }
    if (g < 0.0) continue; /* expert e did not receive token t */
    for (int32_t j = 0; j < d; ++j) {
      xt[j] = ld(x, dt, t * d + j);
      go[j] = g * dy[t * d + j];
    }
    for (int32_t a = 0; a < nf; ++a) {
      const int32_t f = f_list[a];
      double zf = b1 ? ld(b1, dt, b1off + f) : 0.0, dh = 0.0;
      for (int32_t j = 0; j < d; ++j) zf += ld(W1, dt, w1off + (int64_t)f * d + j) * xt[j];
      for (int32_t j = 0; j < d; ++j) dh += ld(W2, dt, w2off + (int64_t)j * Fm + f) * go[j];
      const double hf = act_fn(c->act, zf), dz = dh * act_grad(c->act, zf);
      for (int32_t b = 0; b < nj; ++b) {
        dW1[(int64_t)a * nj + b] += dz * xt[j_list[b]];
        dW2[(int64_t)b * nf + a] += go[j_list[b]] * hf;
      }
      db1[a] += dz;
    }
    for (int32_t b = 0; b < nj; ++b) db2[b] += go[j_list[b]];
  }
  free(xt);
  free(go);
  return 0;
}
