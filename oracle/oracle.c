/*
 * CPU oracle for the MoE router and token dispatch -- TEST INFRASTRUCTURE.
 * See oracle.h for the sources and the readings this file follows.  Plain
 * fp64 C, built with -O2 -ffp-contract=off and no fast-math; one token at a
 * time, library qsort for every ordering.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- inputs ------------------------------------------------------------ */

/* One element of x or W as a double.  bf16 is the top half of an IEEE
 * binary32, so the conversion is exact. */
static double input_at(int32_t dtype, const void* base, size_t i) {
  if (dtype == ORC_BF16) {
    uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[i];
}

/* ---- gate: [DSV3.2] gate-forward excerpt, first step ---------------------
 * The gate is a linear map of the token's hidden state onto one logit per
 * routed expert, computed in fp32 there and in fp64 here. */
static void gate_row(const orc_params* p, const void* x, const void* W,
                     const float* logit_bias, int32_t t, double* l) {
  for (int32_t e = 0; e < p->E; ++e) {
    double acc = 0.0;
    for (int32_t i = 0; i < p->d; ++i)
      acc += input_at(p->dtype, x, (size_t)t * p->d + i) *
             input_at(p->dtype, W, (size_t)e * p->d + i);
    if (logit_bias) acc += (double)logit_bias[e];
    l[e] = acc;
  }
}

void orc_gate(const orc_params* p, const void* x, const void* W,
              const float* logit_bias, double* logits) {
  for (int32_t t = 0; t < p->T; ++t)
    gate_row(p, x, W, logit_bias, t, logits + (size_t)t * p->E);
}

/* ---- scoring -------------------------------------------------------------
 * softmax over all experts: [DSV3.2] excerpt; [ferrox] route_top_k_softmax.
 * sigmoid per expert: [DSV3.2] excerpt; [ferrox] route_top_k_sigmoid.
 * sqrt(softplus(l)) per expert: [ferrox] route_top_k_sqrtsoftplus.
 * softmax_topk selects on the raw logit: [ferrox] route_top_k_softmax_weight. */
static double softplus(double l) { return fmax(l, 0.0) + log1p(exp(-fabs(l))); }

static void scores(const orc_params* p, const double* l, double* s) {
  const int32_t E = p->E;
  if (p->score == ORC_SOFTMAX) {
    double m = -INFINITY, sum = 0.0;
    for (int32_t e = 0; e < E; ++e) m = fmax(m, l[e]);
    for (int32_t e = 0; e < E; ++e) sum += exp(l[e] - m);
    for (int32_t e = 0; e < E; ++e) s[e] = exp(l[e] - m) / sum;
  } else {
    for (int32_t e = 0; e < E; ++e) {
      switch (p->score) {
        case ORC_SIGMOID: s[e] = 1.0 / (1.0 + exp(-l[e])); break;
        case ORC_SQRT_SOFTPLUS: s[e] = sqrt(softplus(l[e])); break;
        default: s[e] = l[e]; break; /* ORC_SOFTMAX_TOPK */
      }
    }
  }
}

/* ---- ordering ------------------------------------------------------------
 * One total order everywhere: larger key first, equal keys by lower id. */
typedef struct {
  double key;
  int32_t id;
} keyed;

static int by_key_desc_id_asc(const void* a, const void* b) {
  const keyed* x = (const keyed*)a;
  const keyed* y = (const keyed*)b;
  if (x->key > y->key) return -1;
  if (x->key < y->key) return 1;
  return (x->id > y->id) - (x->id < y->id);
}

/* ---- weights ---------------------------------------------------------------
 * Each selected expert is weighted by its UNBIASED score ([DSV3.2]
 * "Explanation": the bias only chooses; [ferrox] route_top_k_sigmoid_with_bias
 * warns that biasing the weight is a silent error).  softmax_topk weights are
 * the softmax over just the selected logits ([ferrox]
 * route_top_k_softmax_weight).  Renormalise to sum one when asked, then
 * multiply by route_scale ([DSV3.2] excerpt: renorm, then route_scale). */
static void token_weights(const orc_params* p, const double* l,
                          const int32_t* ids, double* w) {
  const int32_t K = p->k, E = p->E;
  double m = -INFINITY, denom = 0.0;
  if (p->score == ORC_SOFTMAX) {
    for (int32_t e = 0; e < E; ++e) m = fmax(m, l[e]);
    for (int32_t e = 0; e < E; ++e) denom += exp(l[e] - m);
  } else if (p->score == ORC_SOFTMAX_TOPK) {
    for (int32_t j = 0; j < K; ++j)
      if (ids[j] >= 0 && ids[j] < E) m = fmax(m, l[ids[j]]);
    for (int32_t j = 0; j < K; ++j)
      if (ids[j] >= 0 && ids[j] < E) denom += exp(l[ids[j]] - m);
  }
  int32_t nvalid = 0;
  for (int32_t j = 0; j < K; ++j) {
    const int32_t e = ids[j];
    if (e < 0 || e >= E) {
      w[j] = 0.0;
      continue;
    }
    ++nvalid;
    switch (p->score) {
      case ORC_SOFTMAX:
      case ORC_SOFTMAX_TOPK: w[j] = exp(l[e] - m) / denom; break;
      case ORC_SIGMOID: w[j] = 1.0 / (1.0 + exp(-l[e])); break;
      default: w[j] = sqrt(softplus(l[e])); break;
    }
  }
  if (p->renormalize && nvalid > 0) {
    double sum = 0.0;
    for (int32_t j = 0; j < K; ++j) sum += w[j];
    for (int32_t j = 0; j < K; ++j) w[j] /= sum;
  }
  for (int32_t j = 0; j < K; ++j) w[j] *= p->route_scale;
}

void orc_weights_for_ids(const orc_params* p, const double* logits,
                         const int32_t* ids, double* weights) {
  for (int32_t t = 0; t < p->T; ++t)
    token_weights(p, logits + (size_t)t * p->E, ids + (size_t)t * p->k,
                  weights + (size_t)t * p->k);
}

/* ---- selection of one token -------------------------------------------------
 * [DSV3.2] excerpt and "Explanation": q = s + b (bias for choosing only);
 * with groups, view q as [groups][E/groups]; a group's score is the sum of its
 * two largest q when a bias exists, else its largest q; keep the best
 * topk_groups groups, drop every expert of the others, take the top-k of
 * what is left.  [ferrox] route_top_k_grouped (k_per_group > 0): split the
 * experts into the same contiguous groups, keep the k_per_group largest q of
 * each group (by the flat rule's score), then the global top-k of those.
 * [dyn-k]: k_t can differ per request over the same scores.
 * Returns 0, or 1 when k_t is outside [1, k] (then the row is emptied). */
static int route_token(const orc_params* p, const double* l, const float* sb,
                       int32_t kt, int32_t* ids, double* w, double* mk,
                       double* mg, double* ms, double* mo, double* q_out,
                       double* g_out) {
  const int32_t E = p->E, K = p->k, G = p->n_groups, TG = p->topk_groups;
  double* s = (double*)malloc(sizeof(double) * E);
  double* q = (double*)malloc(sizeof(double) * E);
  keyed* order = (keyed*)malloc(sizeof(keyed) * E);
  int bad = (kt < 1 || kt > K);

  scores(p, l, s);
  for (int32_t e = 0; e < E; ++e) q[e] = s[e] + (sb ? (double)sb[e] : 0.0);

  *mg = INFINITY;
  if (G > 1) {
    const int32_t gs = E / G;
    keyed* gorder = (keyed*)malloc(sizeof(keyed) * G);
    keyed* member = (keyed*)malloc(sizeof(keyed) * gs);
    for (int32_t g = 0; g < G; ++g) {
      for (int32_t i = 0; i < gs; ++i) {
        member[i].key = q[g * gs + i];
        member[i].id = g * gs + i;
      }
      qsort(member, gs, sizeof(keyed), by_key_desc_id_asc);
      double gscore = member[0].key;
      if (p->group_score == ORC_GROUP_TOP2_SUM && gs >= 2) gscore += member[1].key;
      gorder[g].key = gscore;
      gorder[g].id = g;
      if (g_out) g_out[g] = gscore;
    }
    qsort(gorder, G, sizeof(keyed), by_key_desc_id_asc);
    if (TG < G && p->k_per_group <= 0) {
      *mg = gorder[TG - 1].key - gorder[TG].key;
      for (int32_t r = TG; r < G; ++r) {
        const int32_t g = gorder[r].id;
        for (int32_t i = 0; i < gs; ++i) q[g * gs + i] = -INFINITY;
      }
    }
    free(member);
    free(gorder);
  }
  if (p->k_per_group > 0) {
    /* each group keeps its k_per_group largest q; g_out holds the last kept
     * value (-inf when the group keeps every member), margin_g the smallest
     * gap at a group's cut */
    const int32_t gs = E / G, kpg = p->k_per_group;
    keyed* member = (keyed*)malloc(sizeof(keyed) * gs);
    for (int32_t g = 0; g < G; ++g) {
      for (int32_t i = 0; i < gs; ++i) {
        member[i].key = q[g * gs + i];
        member[i].id = g * gs + i;
      }
      qsort(member, gs, sizeof(keyed), by_key_desc_id_asc);
      if (g_out) g_out[g] = kpg < gs ? member[kpg - 1].key : -INFINITY;
      if (kpg < gs) {
        *mg = fmin(*mg, member[kpg - 1].key - member[kpg].key);
        for (int32_t i = kpg; i < gs; ++i) q[member[i].id] = -INFINITY;
      }
    }
    free(member);
  }
  if (q_out) memcpy(q_out, q, sizeof(double) * E);

  for (int32_t e = 0; e < E; ++e) {
    order[e].key = q[e];
    order[e].id = e;
  }
  qsort(order, E, sizeof(keyed), by_key_desc_id_asc);
  int32_t ncand = 0;
  for (int32_t e = 0; e < E; ++e) ncand += (q[e] > -INFINITY);

  for (int32_t j = 0; j < K; ++j) ids[j] = (!bad && j < kt) ? order[j].id : -1;

  /* margins at the k-th boundary */
  *ms = (!bad && kt < ncand) ? order[kt - 1].key - order[kt].key : INFINITY;
  const int monotone = (sb == NULL) && !(G > 1 && TG < G) && p->k_per_group <= 0;
  *mo = INFINITY;
  if (bad) {
    *mk = INFINITY;
  } else if (monotone) {
    /* every score function is strictly increasing in the logit, so the
     * same choice is the top-k of the logits; its gap is the logit gap */
    keyed* lo = (keyed*)malloc(sizeof(keyed) * E);
    for (int32_t e = 0; e < E; ++e) {
      lo[e].key = l[e];
      lo[e].id = e;
    }
    qsort(lo, E, sizeof(keyed), by_key_desc_id_asc);
    *mk = (kt < E) ? lo[kt - 1].key - lo[kt].key : INFINITY;
    for (int32_t j = 0; j + 1 < kt; ++j) *mo = fmin(*mo, lo[j].key - lo[j + 1].key);
    free(lo);
  } else {
    *mk = *ms;
    for (int32_t j = 0; j + 1 < kt; ++j)
      *mo = fmin(*mo, order[j].key - order[j + 1].key);
  }

  if (bad) {
    for (int32_t j = 0; j < K; ++j) w[j] = 0.0;
  } else {
    token_weights(p, l, ids, w);
  }
  free(order);
  free(q);
  free(s);
  return bad;
}

int32_t orc_route_logits(const orc_params* p, const double* logits,
                         const float* select_bias, const int32_t* k_per_token,
                         int32_t* ids, double* weights, double* margin_k,
                         double* margin_g, double* margin_s, double* margin_o,
                         double* q_out, double* g_out) {
  int32_t nbad = 0;
  for (int32_t t = 0; t < p->T; ++t) {
    const int32_t kt = k_per_token ? k_per_token[t] : p->k;
    nbad += route_token(p, logits + (size_t)t * p->E, select_bias, kt,
                        ids + (size_t)t * p->k, weights + (size_t)t * p->k,
                        margin_k + t, margin_g + t, margin_s + t, margin_o + t,
                        q_out ? q_out + (size_t)t * p->E : NULL,
                        g_out ? g_out + (size_t)t * p->n_groups : NULL);
  }
  return nbad;
}

/* ---- hash routing: [ferrox] route_hash ------------------------------------
 * The expert ids of a hash layer are the token id's row of a fixed
 * token-id -> expert-id table; nothing is selected by score. */
int32_t orc_hash_ids(int32_t T, int32_t k, int32_t E, const int32_t* tok,
                     const int32_t* tid2eid, int32_t vocab, int32_t* ids) {
  int32_t nerr = 0;
  for (int32_t t = 0; t < T; ++t) {
    const int32_t v = tok[t];
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = -1;
      if (v >= 0 && v < vocab) {
        e = tid2eid[(size_t)v * k + j];
        if (e < 0 || e >= E) {
          ++nerr;
          e = -1;
        }
      }
      ids[(size_t)t * k + j] = e;
    }
    if (v < 0 || v >= vocab) ++nerr;
  }
  return nerr;
}

/* ---- dispatch ----------------------------------------------------------------
 * Group the routed (token, slot) pairs by expert: a stable counting sort of
 * route indices r = t*k_stride + j, ascending r inside each expert. */
int32_t orc_dispatch(const int32_t* ids, int32_t T, int32_t k_stride, int32_t E,
                     int32_t* counts, int32_t* offsets, int32_t* perm,
                     int32_t* inv) {
  const int64_t R = (int64_t)T * k_stride;
  int32_t nerr = 0;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t r = 0; r < R; ++r) {
    const int32_t e = ids[r];
    if (e < 0) continue;
    if (e >= E) {
      ++nerr;
      continue;
    }
    ++counts[e];
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (E > 0 ? E : 1));
  for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t r = 0; r < R; ++r) {
    const int32_t e = ids[r];
    if (inv) inv[r] = -1;
    if (e < 0 || e >= E) continue;
    const int32_t pos = cursor[e]++;
    perm[pos] = (int32_t)r;
    if (inv) inv[r] = pos;
  }
  free(cursor);
  return nerr;
}

/* ---- load statistic: [router-survey] MaxVio ------------------------------- */
double orc_maxvio(const int32_t* counts, int32_t E) {
  int64_t R = 0;
  int32_t mx = 0;
  for (int32_t e = 0; e < E; ++e) {
    R += counts[e];
    if (counts[e] > mx) mx = counts[e];
  }
  if (R == 0) return 0.0;
  return (double)mx / ((double)R / (double)E) - 1.0;
}

/* ---- expert parallelism: [router-survey] -- with experts spread over GPUs
 * every routing choice becomes all-to-all traffic.  With N ranks owning E/N
 * contiguous experts each, the dispatch order (by expert) is already the
 * send order: rank n's share is the block of experts [n*E/N, (n+1)*E/N),
 * and the send buffer holds each route's token row in dispatch order. */
void orc_ep_layout(const int32_t* offsets, int32_t E, int32_t N, int32_t* send_counts,
                   int32_t* send_offsets) {
  for (int32_t n = 0; n <= N; ++n) send_offsets[n] = offsets[(int64_t)n * E / N];
  for (int32_t n = 0; n < N; ++n) send_counts[n] = send_offsets[n + 1] - send_offsets[n];
}

void orc_permute_rows(int32_t k_stride, int32_t d, int32_t dtype, const void* x,
                      const int32_t* perm, int32_t R, double* out) {
  for (int32_t p = 0; p < R; ++p) {
    const int32_t t = perm[p] / k_stride;
    for (int32_t i = 0; i < d; ++i) out[(size_t)p * d + i] = input_at(dtype, x, (size_t)t * d + i);
  }
}

/* ---- capacity: [router-survey] names top-1 routing with a capacity in the
 * manner of the Switch Transformer and gives no rule; the plainest one: an
 * expert takes its routes in route order (ascending r, the order of the
 * stable dispatch) up to its capacity C and drops the rest.  A kept route
 * of expert e with rank q among e's routes goes to slot e*C + q. */
int32_t orc_capacity(const int32_t* ids, int32_t T, int32_t k_stride, int32_t E, int32_t C,
                     int32_t* slot, int32_t* kept) {
  const int64_t R = (int64_t)T * k_stride;
  int32_t* seen = (int32_t*)calloc((size_t)(E > 0 ? E : 1), sizeof(int32_t));
  int32_t dropped = 0;
  for (int64_t r = 0; r < R; ++r) {
    const int32_t e = ids[r];
    slot[r] = -1;
    if (e < 0 || e >= E) continue;  /* empty slot or error: not a route */
    const int32_t q = seen[e]++;
    if (q < C)
      slot[r] = e * C + q;
    else
      ++dropped;
  }
  for (int32_t e = 0; e < E; ++e) kept[e] = seen[e] < C ? seen[e] : C;
  free(seen);
  return dropped;
}

/* ---- combine: [dyn-k] "Possible Implementation" (the output is the sum of
 * the selected experts' outputs, each times its weight) and [ferrox]
 * combine_expert_outputs (routed plus shared expert outputs of a token).
 * Row p of Yp is the expert output for the route placed at position p by
 * the dispatch, so slot j of token t reads row inv[t*k + j]; the shared
 * output enters with weight 1, after the routed slots. */
int32_t orc_combine(int32_t T, int32_t k, int32_t d, int32_t dtype, const void* Yp, int32_t R,
                    const int32_t* inv, const float* weights, const void* shared,
                    double* y) {
  int32_t nerr = 0;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t i = 0; i < d; ++i) y[(size_t)t * d + i] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      const int32_t p = inv[(size_t)t * k + j];
      if (p < 0) continue;          /* empty slot */
      if (p >= R) {                 /* no such row: counted, left out */
        ++nerr;
        continue;
      }
      const double w = (double)weights[(size_t)t * k + j];
      for (int32_t i = 0; i < d; ++i)
        y[(size_t)t * d + i] += w * input_at(dtype, Yp, (size_t)p * d + i);
    }
    if (shared)
      for (int32_t i = 0; i < d; ++i)
        y[(size_t)t * d + i] += input_at(dtype, shared, (size_t)t * d + i);
  }
  return nerr;
}

/* ---- the same per-token functions, split over host threads by token ------
 * Tokens are independent, so splitting them over threads changes nothing in
 * any token's arithmetic; these exist only to make full-size checks fast. */
typedef struct {
  const orc_params* p;
  const void *x, *W;
  const float* logit_bias;
  const double* logits_in;
  const float* select_bias;
  const int32_t* k_per_token;
  double* logits_out;
  int32_t* ids;
  double *weights, *mk, *mg, *ms, *mo, *q_out, *g_out;
  int32_t t0, t1;
  int32_t nbad;
} token_job;

static void* gate_worker(void* arg) {
  token_job* j = (token_job*)arg;
  for (int32_t t = j->t0; t < j->t1; ++t)
    gate_row(j->p, j->x, j->W, j->logit_bias, t, j->logits_out + (size_t)t * j->p->E);
  return NULL;
}

static void* route_worker(void* arg) {
  token_job* j = (token_job*)arg;
  const orc_params* p = j->p;
  for (int32_t t = j->t0; t < j->t1; ++t) {
    const int32_t kt = j->k_per_token ? j->k_per_token[t] : p->k;
    j->nbad += route_token(p, j->logits_in + (size_t)t * p->E, j->select_bias, kt,
                           j->ids + (size_t)t * p->k, j->weights + (size_t)t * p->k,
                           j->mk + t, j->mg + t, j->ms + t, j->mo + t,
                           j->q_out ? j->q_out + (size_t)t * p->E : NULL,
                           j->g_out ? j->g_out + (size_t)t * p->n_groups : NULL);
  }
  return NULL;
}

static int32_t run_token_jobs(const token_job* proto, int32_t T, int32_t nthreads,
                              void* (*fn)(void*)) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > T) nthreads = T > 0 ? T : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  token_job* jobs = (token_job*)malloc(sizeof(token_job) * nthreads);
  for (int32_t i = 0; i < nthreads; ++i) {
    jobs[i] = *proto;
    jobs[i].t0 = (int32_t)((int64_t)T * i / nthreads);
    jobs[i].t1 = (int32_t)((int64_t)T * (i + 1) / nthreads);
    jobs[i].nbad = 0;
    pthread_create(&th[i], NULL, fn, &jobs[i]);
  }
  int32_t nbad = 0;
  for (int32_t i = 0; i < nthreads; ++i) {
    pthread_join(th[i], NULL);
    nbad += jobs[i].nbad;
  }
  free(jobs);
  free(th);
  return nbad;
}

void orc_gate_mt(const orc_params* p, const void* x, const void* W,
                 const float* logit_bias, double* logits, int32_t nthreads) {
  token_job j;
  memset(&j, 0, sizeof j);
  j.p = p;
  j.x = x;
  j.W = W;
  j.logit_bias = logit_bias;
  j.logits_out = logits;
  run_token_jobs(&j, p->T, nthreads, gate_worker);
}

int32_t orc_route_logits_mt(const orc_params* p, const double* logits,
                            const float* select_bias, const int32_t* k_per_token,
                            int32_t* ids, double* weights, double* margin_k,
                            double* margin_g, double* margin_s, double* margin_o,
                            double* q_out, double* g_out, int32_t nthreads) {
  token_job j;
  memset(&j, 0, sizeof j);
  j.p = p;
  j.logits_in = logits;
  j.select_bias = select_bias;
  j.k_per_token = k_per_token;
  j.ids = ids;
  j.weights = weights;
  j.mk = margin_k;
  j.mg = margin_g;
  j.ms = margin_s;
  j.mo = margin_o;
  j.q_out = q_out;
  j.g_out = g_out;
  return run_token_jobs(&j, p->T, nthreads, route_worker);
}

/* ---- whole path, threaded over tokens ------------------------------------- */
typedef struct {
  const orc_params* p;
  const void *x, *W;
  const float *logit_bias, *select_bias;
  const int32_t* k_per_token;
  int32_t* ids;
  double* weights;
  int32_t t0, t1;
  int32_t nbad;
} full_job;

static void* full_worker(void* arg) {
  full_job* j = (full_job*)arg;
  const orc_params* p = j->p;
  double* l = (double*)malloc(sizeof(double) * p->E);
  double mk, mg, ms, mo;
  for (int32_t t = j->t0; t < j->t1; ++t) {
    gate_row(p, j->x, j->W, j->logit_bias, t, l);
    const int32_t kt = j->k_per_token ? j->k_per_token[t] : p->k;
    j->nbad += route_token(p, l, j->select_bias, kt, j->ids + (size_t)t * p->k,
                           j->weights + (size_t)t * p->k, &mk, &mg, &ms, &mo,
                           NULL, NULL);
  }
  free(l);
  return NULL;
}

int32_t orc_route_full(const orc_params* p, const void* x, const void* W,
                       const float* logit_bias, const float* select_bias,
                       const int32_t* k_per_token, int32_t* ids,
                       double* weights, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* inv, int32_t nthreads) {
  if (nthreads < 1) nthreads = 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  full_job* jobs = (full_job*)malloc(sizeof(full_job) * nthreads);
  for (int32_t i = 0; i < nthreads; ++i) {
    full_job j = {p, x, W, logit_bias, select_bias, k_per_token, ids, weights,
                  (int32_t)((int64_t)p->T * i / nthreads),
                  (int32_t)((int64_t)p->T * (i + 1) / nthreads), 0};
    jobs[i] = j;
    pthread_create(&th[i], NULL, full_worker, &jobs[i]);
  }
  int32_t nbad = 0;
  for (int32_t i = 0; i < nthreads; ++i) {
    pthread_join(th[i], NULL);
    nbad += jobs[i].nbad;
  }
  free(jobs);
  free(th);
  orc_dispatch(ids, p->T, p->k, p->E, counts, offsets, perm, inv);
  return nbad;
}
