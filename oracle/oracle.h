/*
 * CPU oracle for the MoE router and token dispatch -- TEST INFRASTRUCTURE.
 *
 * Plain, slow, obviously-correct fp64 C.  It exists to check the HIP
 * library; it is not part of the product path.  Only the tests, the smoke
 * entry point and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * Sources (web pages; cited by title and section):
 *  [DSV3.2]  "DeepSeek-V3.2-Exp - Select experts" (atlas.klimoza.dev): the
 *            selection formula, its "Explanation" section and the gate-forward
 *            code excerpt (linear in fp32 -> softmax/sigmoid -> selection
 *            bias -> group limit -> top-k -> unbiased weights -> renorm ->
 *            route_scale).
 *  [ferrox]  "ferrox_moe" crate documentation (docs.rs, 0.9.1): function
 *            items route_top_k_softmax, route_top_k_softmax_weight,
 *            route_top_k_sigmoid(_with_bias), route_top_k_sqrtsoftplus
 *            (_with_bias), route_hash, RoutingDecision.
 *  [dyn-k]   "Feature Request: dynamic number of experts (hyperparam per
 *            request)" (llama.cpp issue 13572): k chosen per request over the
 *            same gate scores.
 *  [router-survey] "I modelli MoE open hanno router opposti" (millebit.com):
 *            MaxVio as the load statistic; the routed-expert configurations;
 *            shared experts kept always on beside the routed ones; top-1
 *            routing with a Switch-style capacity; under expert parallelism
 *            every routing choice becomes all-to-all traffic.
 *  [ferrox] also: combine_expert_outputs (routed + shared outputs of a
 *            token); [dyn-k] "Possible Implementation": the output is the
 *            weighted sum of the selected experts' outputs.
 *
 * Readings where the pages are silent are fixed here:
 * ties go to the lower expert (group) id; slot order is descending selection
 * score; unused dynamic-k slots hold id -1 / weight 0; the token permutation
 * is the stable counting sort of route indices r = t*k_stride + j by expert.
 *
 * Parity pins: every function is pinned by tests/test_oracle_*.py (hand
 * cases, brute-force subset enumeration, closed forms, library reductions).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_SOFTMAX = 0, ORC_SIGMOID = 1, ORC_SQRT_SOFTPLUS = 2, ORC_SOFTMAX_TOPK = 3 };
enum { ORC_GROUP_MAX = 0, ORC_GROUP_TOP2_SUM = 1 };

typedef struct {
  int32_t T, d, E;
  int32_t k;            /* row stride of ids/weights (k_max when k varies) */
  int32_t dtype;        /* ORC_F32 / ORC_BF16 for x and W */
  int32_t score;        /* ORC_SOFTMAX ... */
  int32_t n_groups;     /* 1 = no group limit */
  int32_t topk_groups;
  int32_t group_score;  /* ORC_GROUP_MAX / ORC_GROUP_TOP2_SUM */
  int32_t renormalize;
  double route_scale;
  int32_t k_per_group;  /* > 0: at most this many experts per group, the
                           global top-k over the groups' best (ferrox
                           route_top_k_grouped); 0 = off */
} orc_params;

/* logits[T][E] = x[T][d] . W[E][d]^T (+ logit_bias[E]) in fp64, index order. */
void orc_gate(const orc_params* p, const void* x, const void* W,
              const float* logit_bias, double* logits);

/* Selection + weights from fp64 logits, one token at a time.
 *   ids[T][k], weights[T][k]: slots j >= k_t hold -1 / 0.
 *   margin_k[T]: gap at the k-th boundary in the compared quantity (logit
 *     when selection is a monotone function of the logit, else q = s + b);
 *     +inf when every candidate is taken.
 *   margin_g[T]: gap at the kept-group boundary (+inf without a group limit).
 *   margin_s[T]: gap at the k-th boundary in score units (reporting only).
 *   margin_o[T]: smallest gap between consecutive selected experts in the
 *     compared quantity (slot order); +inf when k_t <= 1.
 *   q_out[T][E] (may be NULL): the selection quantity after the group mask
 *     (-inf for experts of dropped groups).
 *   g_out[T][n_groups] (may be NULL): group scores.
 * Returns the number of tokens with an invalid k_t (outside [1, k]); those
 * tokens get ids -1 and weights 0. */
int32_t orc_route_logits(const orc_params* p, const double* logits,
                         const float* select_bias, const int32_t* k_per_token,
                         int32_t* ids, double* weights, double* margin_k,
                         double* margin_g, double* margin_s, double* margin_o,
                         double* q_out, double* g_out);

/* Combine weights for given expert ids (hash routing, near-tie checks).
 * ids[T][k]; negative ids are empty slots (weight 0, left out of the sum). */
void orc_weights_for_ids(const orc_params* p, const double* logits,
                         const int32_t* ids, double* weights);

/* Hash routing: ids[t][j] = tid2eid[tok[t]][j] (row-major [vocab][k]).
 * A token id outside [0, vocab) empties the token's row; a table entry
 * outside [0, E) empties its slot.  Returns the number of such errors. */
int32_t orc_hash_ids(int32_t T, int32_t k, int32_t E, const int32_t* tok,
                     const int32_t* tid2eid, int32_t vocab, int32_t* ids);

/* Stable counting sort of routes by expert.
 *   ids[T*k_stride]; ids < 0 are empty slots, ids >= E are errors (skipped).
 *   counts[E], offsets[E+1], perm[T*k_stride] (first offsets[E] valid),
 *   inv[T*k_stride] (-1 for skipped slots; may be NULL).
 * Returns the number of ids >= E. */
int32_t orc_dispatch(const int32_t* ids, int32_t T, int32_t k_stride, int32_t E,
                     int32_t* counts, int32_t* offsets, int32_t* perm,
                     int32_t* inv);

/* MaxVio = max_e counts[e] / (R / E) - 1, R = sum of counts. */
double orc_maxvio(const int32_t* counts, int32_t E);

/* Expert-parallel send layout over N ranks owning E/N contiguous experts
 * each (N divides E): send_offsets[n] = offsets[n*E/N] (n <= N) and
 * send_counts[n] = the routes of rank n's experts. */
void orc_ep_layout(const int32_t* offsets, int32_t E, int32_t N, int32_t* send_counts,
                   int32_t* send_offsets);

/* The send buffer: out[p][i] = x[perm[p] / k_stride][i] for p < R (the
 * token row of each route, in dispatch order); x is ORC_F32 or ORC_BF16. */
void orc_permute_rows(int32_t k_stride, int32_t d, int32_t dtype, const void* x,
                      const int32_t* perm, int32_t R, double* out);

/* Capacity-limited dispatch: expert e keeps the first C of its routes in
 * route order; route r of expert e with rank q < C gets slot[r] = e*C + q,
 * a later route slot[r] = -1 (dropped); ids < 0 or >= E are not routes
 * (slot -1, not counted).  kept[e] = min(routes of e, C).  Returns the
 * number of dropped routes. */
int32_t orc_capacity(const int32_t* ids, int32_t T, int32_t k_stride, int32_t E, int32_t C,
                     int32_t* slot, int32_t* kept);

/* Combine: y[t][i] = sum over slots j with 0 <= inv[t*k+j] < R of
 * weights[t][j] * Yp[inv[t*k+j]][i], plus shared[t][i] (weight 1) when
 * shared is not NULL, in fp64 (slots in order, the shared term last).
 * Yp[R][d] holds the expert outputs in dispatch order; Yp and shared are
 * ORC_F32 or ORC_BF16 (dtype).  inv < 0 marks an empty slot; inv >= R is an
 * error (counted and left out).  Returns the number of errors. */
int32_t orc_combine(int32_t T, int32_t k, int32_t d, int32_t dtype, const void* Yp, int32_t R,
                    const int32_t* inv, const float* weights, const void* shared,
                    double* y);

/* orc_gate and orc_route_logits with the tokens split over nthreads host
 * threads (tokens are independent: the results are those of the one-thread
 * calls, bit for bit).  For full-size checks. */
void orc_gate_mt(const orc_params* p, const void* x, const void* W,
                 const float* logit_bias, double* logits, int32_t nthreads);
int32_t orc_route_logits_mt(const orc_params* p, const double* logits,
                            const float* select_bias, const int32_t* k_per_token,
                            int32_t* ids, double* weights, double* margin_k,
                            double* margin_g, double* margin_s, double* margin_o,
                            double* q_out, double* g_out, int32_t nthreads);

/* Whole path (gate + route + dispatch) split over nthreads host threads by
 * token; dispatch runs on one thread.  Used to time the oracle. */
int32_t orc_route_full(const orc_params* p, const void* x, const void* W,
                       const float* logit_bias, const float* select_bias,
                       const int32_t* k_per_token, int32_t* ids,
                       double* weights, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* inv, int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
