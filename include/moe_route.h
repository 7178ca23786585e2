/*
 * moe_route.h -- C ABI of the MI355X (gfx950) MoE router and token dispatch.
 *
 * A Mixture-of-Experts router scores every routed expert for each token,
 * keeps k of them and returns, per token, which experts fire and their
 * combination weights (ferrox_moe crate docs, "RoutingDecision"; the gate of
 * "DeepSeek-V3.2-Exp - Select experts" returns (weights, indices)).  Dispatch
 * then groups the routed (token, slot) pairs by expert.
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers (hipMalloc / torch CUDA tensors) unless
 *    stated otherwise; arrays are dense, row-major, caller-owned.  The
 *    library never allocates, frees or synchronises and keeps no state
 *    between calls; inputs are never modified.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without waiting.  Results are valid once the stream
 *    reaches them.
 *  - Argument errors are detected on the host before anything is enqueued:
 *    the call returns MOE_EINVAL or MOE_EUNSUPPORTED and moe_last_error()
 *    describes the problem.  A failed launch returns MOE_EDEVICE.
 *  - Data-dependent errors (a token id outside the vocabulary, a table entry
 *    or expert id outside [0, E), a per-token k outside [1, k]) cannot be seen
 *    without a sync: the affected slots get id -1 and weight 0, and, when
 *    `dev_err` is not NULL, the kernels add the number of such errors to the
 *    device int32 *dev_err (the caller zeroes it).
 *  - T == 0 is valid and enqueues nothing (moe_dispatch still writes zero
 *    counts and offsets).
 *  - Results do not depend on the kernel plan (tiling, K split, fused or
 *    separate selection) beyond fp32 summation order inside the gate, which
 *    is fixed per plan; plans are chosen from the shapes.  For tuning, these
 *    environment variables override the choice: MOE_GATE_TILE ("BMxBN", or
 *    "BMxBNw8" for eight wavefronts), MOE_GATE_SPLITS (1-8), MOE_GATE_RB
 *    (64/128/256/512-byte stages), MOE_GATE_NS (ring depth), MOE_GATE_NSW
 *    (0: one ring of x and W stages; 2: W two stages deep under three of x,
 *    where the tile fits that), MOE_GATE_NOPIPE
 *    (the register-staged gate kernel), MOE_SELECT_LPT (4/8/16/64 lanes per
 *    token), MOE_NO_FUSED_SELECT (selection in its own kernel),
 *    MOE_DISPATCH_UNFUSED (the three-kernel dispatch), MOE_DISPATCH_NO_SUPER
 *    (tile histograms without super-tile sums: the placement reads every
 *    tile's counts), MOE_SELECT_SUPER_WAVES (2/4/8 wavefronts per counted
 *    selection workgroup), MOE_NO_SMALL_DISPATCH (no one-workgroup
 *    selection + dispatch for small batches), MOE_HASH_DENSE (hash layers
 *    take the gate of every expert instead of k dot products per token),
 *    MOE_HASH_SLICE (64, up to 384 experts also 112/128/192 columns per
 *    dot-product slice), MOE_HASH_BESIDE (0: the hash layer's dispatch in
 *    its own placement kernel; 1: on the dot-product kernel's spare
 *    workgroups whenever possible), MOE_PLACE_GROUP (1/2/4/8 dispatch tiles
 *    per placement workgroup).  Values that do not fit the shapes are ignored;
 *    workspace sizes follow the same variables.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 11

/* return codes */
#define MOE_OK 0
#define MOE_EINVAL (-1)       /* bad shape, flag, pointer or workspace size */
#define MOE_EUNSUPPORTED (-2) /* valid but beyond the documented limits */
#define MOE_EDEVICE (-3)      /* HIP launch failure */

/* documented limits */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_K 32
#define MOE_MAX_GROUPS 64

/* dtype of x and W */
#define MOE_F32 0
#define MOE_BF16 1

/* score functions.
 * SOFTMAX        softmax over all E logits; select the top-k probabilities
 *                (ferrox_moe docs, route_top_k_softmax; DeepSeek-V3.2-Exp
 *                gate-forward excerpt, softmax branch).
 * SIGMOID        sigmoid(logit) per expert (DeepSeek-V3.2-Exp gate-forward
 *                excerpt; ferrox_moe route_top_k_sigmoid).
 * SQRT_SOFTPLUS  sqrt(softplus(logit)) per expert (ferrox_moe
 *                route_top_k_sqrtsoftplus; DeepSeek-V4 non-hash layers).
 * SOFTMAX_TOPK   select by raw logit, weights = softmax over just the k
 *                selected logits (ferrox_moe route_top_k_softmax_weight;
 *                gpt-oss). */
#define MOE_SCORE_SOFTMAX 0
#define MOE_SCORE_SIGMOID 1
#define MOE_SCORE_SQRT_SOFTPLUS 2
#define MOE_SCORE_SOFTMAX_TOPK 3

/* group score (DeepSeek-V3.2-Exp - Select experts, gate-forward excerpt): the
 * largest selection score of the group, or the sum of its two largest.  The
 * excerpt uses TOP2_SUM exactly when a selection bias exists. */
#define MOE_GROUP_MAX 0
#define MOE_GROUP_TOP2_SUM 1

typedef struct {
  int32_t T;            /* tokens */
  int32_t d;            /* hidden size */
  int32_t E;            /* routed experts, 1..MOE_MAX_EXPERTS */
  int32_t k;            /* experts per token; with k_per_token, k_max = the
                           row stride of ids/weights */
  int32_t dtype;        /* MOE_F32 or MOE_BF16: element type of x and W */
  int32_t score;        /* MOE_SCORE_* */
  int32_t n_groups;     /* contiguous expert groups; 1 = no group limit */
  int32_t topk_groups;  /* groups kept, 1..n_groups */
  int32_t group_score;  /* MOE_GROUP_* */
  int32_t renormalize;  /* 1: selected weights renormalised to sum to one
                           (norm_topk_prob, ferrox_moe route_top_k_softmax) */
  float route_scale;    /* weights multiplied by this after renormalising
                           (route_scale / routed_scaling_factor); 1 = none */
  int32_t k_per_group;  /* 0, or > 0 for grouped top-k with a quota (ferrox_moe
                           route_top_k_grouped): each of the n_groups groups
                           keeps its k_per_group largest q, and ids are the k
                           largest of those; needs topk_groups = n_groups and
                           k <= n_groups * min(k_per_group, E / n_groups) */
} moe_route_params;

/*
 * moe_route -- gate, scoring, selection and weights.
 *
 * Computes, for each token t (DeepSeek-V3.2-Exp - Select experts: formula,
 * "Explanation" and gate-forward excerpt; ferrox_moe route_top_k_* items;
 * per-request k: llama.cpp issue 13572 "dynamic number of experts"):
 *   l[t][e] = sum_i x[t][i] * W[e][i]  (+ logit_bias[e]),  fp32 accumulate;
 *   s = score(l);  q = s + select_bias  (the bias only chooses);
 *   with n_groups > 1: group score = max q or top-2 sum of q per group of
 *     E/n_groups contiguous experts; keep the topk_groups best groups, drop
 *     the experts of the others;
 *   ids[t][0..k_t-1] = the k_t largest q, larger first, equal q -> lower id;
 *   weights[t][j] = s[ids[t][j]] (unbiased; SOFTMAX_TOPK: softmax over the
 *     selected logits), renormalised when p->renormalize, times route_scale.
 * Slots j >= k_t hold id -1 and weight 0.
 *
 * Arguments:
 *   x            [T][d] MOE_F32 or MOE_BF16, or NULL (select-only mode)
 *   W            [E][d] same dtype as x, or NULL (select-only mode; x and W
 *                are both NULL or both set)
 *   logit_bias   [E] fp32 or NULL: added to every logit (moves selection and
 *                weights alike)
 *   select_bias  [E] fp32 or NULL: added to the selection score only
 *   k_per_token  [T] int32 in [1, k] or NULL (= k for every token)
 *   logits       [T][E] fp32 or NULL.  With x and W: if not NULL, the gate
 *                logits l (logit bias included) are written here.  Select-only
 *                mode: the input logits (required; logit_bias, if given, is
 *                added on read).
 *   ids          [T][k] int32 out
 *   weights      [T][k] fp32 out
 *   workspace    device scratch of workspace_bytes >=
 *                moe_route_workspace_size(p) bytes, or NULL/0.  It carries the
 *                gate's fp32 hand-off (split over K when that moves fewer
 *                bytes).  With logits given and too small a workspace the gate
 *                runs unsplit and hands off through logits; with neither it is
 *                MOE_EINVAL.  Contents need no initialisation and are
 *                clobbered.
 *   dev_err      [1] int32 or NULL: incremented per token whose k_per_token
 *                entry is outside [1, k]
 * Limits: k <= MOE_MAX_K, E <= MOE_MAX_EXPERTS, n_groups <= MOE_MAX_GROUPS,
 * k <= topk_groups * E / n_groups, TOP2_SUM needs groups of >= 2 experts,
 * T*d, T*E and T*k below 2^31.
 */
int32_t moe_route(const moe_route_params* p, const void* x, const void* W,
                  const float* logit_bias, const float* select_bias,
                  const int32_t* k_per_token, float* logits, int32_t* ids,
                  float* weights, void* workspace, size_t workspace_bytes,
                  int32_t* dev_err, void* stream);

/* Bytes of device workspace moe_route uses for these parameters (16-byte
 * aligned x and W assumed; 0 when none is needed). */
size_t moe_route_workspace_size(const moe_route_params* p);

/*
 * moe_route_hash -- hash routing (ferrox_moe docs, route_hash: a DeepSeek-V4
 * hash layer takes its expert ids from a fixed token-id -> expert-id table
 * instead of a learned selection, with no selection bias).
 *
 *   ids[t][j] = tid2eid[token_ids[t]][j]
 * tid2eid is row-major [vocab][k] int32 (row v = the k experts of token id
 * v).  A token id outside [0, vocab) empties its row (ids -1, weights 0,
 * one error); a table entry outside [0, E) empties its slot (one error).
 * When x and W are given, weights[t][j] = score(l[t][ids[t][j]]) with
 * l = x.W^T (+ logit_bias), renormalised over the row's valid slots when
 * p->renormalize, times route_scale; SOFTMAX needs renormalize = 1 (it then
 * equals SOFTMAX_TOPK).  With a workspace of at least
 * moe_route_hash_workspace_size(p) bytes: for bf16 x and W with k <= 8,
 * E <= 768, d a multiple of 8 and 16-byte aligned rows, only the k logits
 * a token needs are computed, as k dot products over slices of d with each
 * slice of W held on chip (x read once; the workspace holds the per-slice
 * partial sums, added in slice order); otherwise the logits of every expert
 * come from the tiled gate contraction (as in moe_route).  With no
 * workspace (NULL / 0) the k dot products are computed per token from W
 * in memory.  When x and W are NULL only ids are written (weights may be
 * NULL).  Uses p->T, d, E, k, dtype, score, renormalize, route_scale.
 */
int32_t moe_route_hash(const moe_route_params* p, const int32_t* token_ids,
                       const int32_t* tid2eid, int32_t vocab, const void* x,
                       const void* W, const float* logit_bias, int32_t* ids,
                       float* weights, void* workspace, size_t workspace_bytes,
                       int32_t* dev_err, void* stream);

/* Bytes of device workspace moe_route_hash uses for its logits hand-off
 * with these parameters (16-byte aligned x and W assumed). */
size_t moe_route_hash_workspace_size(const moe_route_params* p);

/*
 * moe_route_hash_dispatch -- moe_route_hash (with x and W and its
 * workspace hand-off) followed by moe_dispatch of its ids (k_stride =
 * p->k), with the results of the two calls (ferrox_moe docs, route_hash;
 * the dispatch as for moe_dispatch).  The hash kernel also counts each
 * tile's expert ids (tile histograms plus super-tile sums that the dot
 * product or gate kernel zeroes), so the dispatch is one placement kernel.
 *   arguments    as for moe_route_hash and moe_dispatch (x and W required)
 *   workspace    256-byte aligned, at least
 *                moe_route_hash_dispatch_workspace_size(p) bytes; contents
 *                need no initialisation and are clobbered
 */
int32_t moe_route_hash_dispatch(const moe_route_params* p, const int32_t* token_ids,
                                const int32_t* tid2eid, int32_t vocab, const void* x,
                                const void* W, const float* logit_bias, int32_t* ids,
                                float* weights, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* inv, double* maxvio, void* workspace,
                                size_t workspace_bytes, int32_t* dev_err, void* stream);
size_t moe_route_hash_dispatch_workspace_size(const moe_route_params* p);

/* Bytes of device workspace moe_dispatch needs for these sizes. */
size_t moe_dispatch_workspace_size(int32_t T, int32_t k_stride, int32_t E);

/*
 * moe_dispatch -- group routes by expert (the step that sends each token only
 * to its selected experts; under expert parallelism it feeds the all-to-all).
 * Passages: "I modelli MoE open hanno router opposti", the sentence on expert
 * parallelism (every routing choice becomes all-to-all traffic between GPUs);
 * "Feature Request: dynamic number of experts", Possible Implementation (only
 * the selected experts run, and their outputs are summed with the weights).
 * The pages fix no layout for the grouping; this is the plain stable
 * counting sort, counts -> exclusive offsets -> positions.
 *
 * Route r = t*k_stride + j is slot j of token t.  Routes with ids[r] < 0 are
 * empty and skipped; ids[r] >= E are errors (skipped, counted in *dev_err).
 *   counts[e]     number of routes to expert e                       [E]
 *   offsets[e]    exclusive prefix sum of counts; offsets[E] = R     [E+1]
 *   perm[p]       route index at position p: the routes of expert e
 *                 fill perm[offsets[e] .. offsets[e+1]) in ascending r
 *                 (a stable counting sort)          [T*k_stride], first R set
 *   inv[r]        position of route r in perm, -1 for skipped slots
 *                 [T*k_stride], may be NULL
 *   maxvio        [1] fp64, or NULL: the load statistic MaxVio =
 *                 max_e counts[e] / (R / E) - 1, R = offsets[E] (0 when
 *                 R = 0) -- "I modelli MoE open hanno router opposti", the
 *                 loss-free balancing paragraph (MaxVio 0.72 -> 0.04); written
 *                 by the kernel that writes counts, in IEEE fp64 in that order
 *   workspace     16-byte aligned device memory of at least
 *                 moe_dispatch_workspace_size(T, k_stride, E) bytes; its
 *                 contents need no initialisation and are clobbered
 * Limits: E <= MOE_MAX_EXPERTS, T*k_stride < 2^31.
 */
int32_t moe_dispatch(const int32_t* ids, int32_t T, int32_t k_stride, int32_t E,
                     int32_t* counts, int32_t* offsets, int32_t* perm,
                     int32_t* inv, double* maxvio, void* workspace, size_t workspace_bytes,
                     int32_t* dev_err, void* stream);

/*
 * moe_permute_rows -- the send buffer: each route's token row at the place
 * the dispatch gave the route, out[inv[r]] = x[r / k_stride] ("I modelli MoE
 * open hanno router opposti": under expert parallelism every routing choice
 * becomes all-to-all traffic; this buffer, in dispatch order, is what each
 * rank sends, and on one GPU the grouped input of the experts).
 *   x        [T][d] token rows (dtype MOE_F32 or MOE_BF16)
 *   inv      [T*k_stride] the place of route r: moe_dispatch's inv (rows
 *            0 .. offsets[E]-1 in dispatch order) or moe_dispatch_capacity's
 *            slot (expert-major rows e*capacity + rank); inv[r] < 0: not
 *            placed, skipped
 *   out      [out_rows][d]; rows no route is placed at are not written; the
 *            bytes of each row are copied unchanged.  Two routes placed at
 *            one row race (the dispatch and capacity inverses never do)
 *   dev_err  optional device counter: += places inv[r] >= out_rows (skipped)
 * Each token row is read once, whatever its number of routes.
 * Limits: T*k_stride < 2^31.  Returns MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED
 * or MOE_EDEVICE.
 */
int32_t moe_permute_rows(int32_t T, int32_t k_stride, int32_t d, int32_t dtype, const void* x,
                         const int32_t* inv, int32_t out_rows, void* out, int32_t* dev_err,
                         void* stream);

/*
 * moe_ep_layout -- per-rank send counts and offsets for expert parallelism
 * over n_ranks ranks owning E/n_ranks contiguous experts each (n_ranks
 * divides E): send_offsets[n] = offsets[n*E/n_ranks] (n <= n_ranks),
 * send_counts[n] = routes to rank n's experts.  The dispatch order is the
 * send order, so rank n's rows are send_offsets[n] .. send_offsets[n+1] of
 * moe_permute_rows' buffer.  offsets[E+1] from moe_dispatch; all device
 * memory.  The exchange itself needs more than one GPU and is not here.
 */
int32_t moe_ep_layout(const int32_t* offsets, int32_t E, int32_t n_ranks, int32_t* send_counts,
                      int32_t* send_offsets, void* stream);

/*
 * moe_dispatch_capacity -- a capacity limit on a dispatch: top-1 routing with
 * a capacity in the manner of the Switch Transformer ("I modelli MoE open
 * hanno router opposti"; the page gives no rule, the one taken here: each
 * expert keeps its first `capacity` routes in route order -- the order
 * moe_dispatch places them in -- and drops the rest).
 *   ids, offsets, inv  the ids given to moe_dispatch and its offsets[E+1]
 *                and inv[T*k_stride] for them
 *   slot     [T*k_stride] out: e*capacity + rank for a kept route of expert
 *            e (rank among e's routes), -1 for a dropped route and for slots
 *            that are not routes; it can serve as moe_combine's inv over
 *            expert rows [E*capacity][d]
 *   kept     [E] out: min(routes of e, capacity)
 *   dropped  [1] out (device): routes over capacity
 * Limits: E <= MOE_MAX_EXPERTS, E*capacity < 2^31, T*k_stride < 2^31.
 * Returns MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED or MOE_EDEVICE.
 */
int32_t moe_dispatch_capacity(const int32_t* ids, int32_t T, int32_t k_stride, int32_t E,
                              int32_t capacity, const int32_t* offsets, const int32_t* inv,
                              int32_t* slot, int32_t* kept, int32_t* dropped, void* stream);

/*
 * moe_route_dispatch -- moe_route followed by moe_dispatch of its ids
 * (k_stride = p->k): one pass of the router and the grouping of its routes,
 * with the results of the two calls (same arguments, same values, bit for
 * bit).  The routing kernels count their own picks per dispatch tile (the
 * routes of the tokens one workgroup selects), saving the dispatch's counting
 * kernel: after the gate kernel, the selection kernel writes each tile's
 * histogram and adds it into super-tile sums that the gate kernel zeroed, so
 * the one placement kernel reads about 2 sqrt(tiles) rows of counts; the gate
 * kernel with the selection fused (whole-row tiles) writes tile histograms
 * that the placement reads in full (tiles x E <= 32768 counts, E a multiple
 * of 8).  Other shapes use the dispatch's own kernels.
 *   workspace    256-byte aligned device memory of at least
 *                moe_route_dispatch_workspace_size(p) bytes (the gate
 *                hand-off, then the dispatch's tile data); contents need no
 *                initialisation and are clobbered
 *   counts, offsets, perm, inv, maxvio, dev_err: as for moe_dispatch (dev_err
 *                also as for moe_route)
 * Limits: those of moe_route and moe_dispatch.
 */
int32_t moe_route_dispatch(const moe_route_params* p, const void* x, const void* W,
                           const float* logit_bias, const float* select_bias,
                           const int32_t* k_per_token, float* logits, int32_t* ids,
                           float* weights, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv, double* maxvio, void* workspace,
                           size_t workspace_bytes, int32_t* dev_err, void* stream);

/* Bytes of device workspace moe_route_dispatch needs for these parameters
 * (16-byte aligned x and W assumed). */
size_t moe_route_dispatch_workspace_size(const moe_route_params* p);

/*
 * moe_route_dispatch_noalloc -- moe_route_dispatch with no workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The scratch the call needs (the gate's hand-off, the dispatch's tile
 * histograms) lives in a device array of MOE_NOALLOC_SCRATCH_BYTES inside
 * the library: one per GPU, held until the process ends, its address looked
 * up on the first call on that GPU (the device of `stream`).  The call
 * allocates nothing and creates no events; it enqueues the same kernels as
 * moe_route_dispatch and gives the same results, bit for bit.
 *   arguments    as for moe_route_dispatch, without workspace and its size;
 *                the caller still passes every input and output
 * Returns MOE_EUNSUPPORTED, with the bytes needed, when
 * moe_route_dispatch_workspace_size(p) exceeds MOE_NOALLOC_SCRATCH_BYTES.
 * Calls that overlap on one GPU (other streams or threads) share the array
 * and race: order them on one stream.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int32_t moe_route_dispatch_noalloc(const moe_route_params* p, const void* x, const void* W,
                                   const float* logit_bias, const float* select_bias,
                                   const int32_t* k_per_token, float* logits, int32_t* ids,
                                   float* weights, int32_t* counts, int32_t* offsets,
                                   int32_t* perm, int32_t* inv, double* maxvio,
                                   int32_t* dev_err, void* stream);

/*
 * How moe_route_dispatch runs for these parameters, with x and W given
 * (16-byte aligned when `aligned` is non-zero): host-side planning only,
 * nothing is enqueued.  For inspection and tests.  Returns MOE_OK, or the
 * error moe_route_dispatch would return for the parameters.
 */
#define MOE_PATH_SEPARATE 0    /* gate, select, then the dispatch's own kernels */
#define MOE_PATH_SELECT_HIST 1 /* the select kernel writes the dispatch's tile histograms */
#define MOE_PATH_FUSED 2       /* the gate kernel runs the selection on its tile's rows */
#define MOE_PATH_SMALL 3       /* one workgroup selects and performs the whole dispatch */
#define MOE_PATH_SELECT_SUPER 4 /* the select kernel writes tile histograms and super-tile
                                   sums (zeroed by the gate kernel): the placement reads
                                   about 2 sqrt(tiles) rows of counts, not every tile's */
typedef struct {
  int32_t path;                    /* MOE_PATH_* */
  int32_t gate_bm, gate_bn;        /* gate tile: tokens x experts */
  int32_t gate_waves;              /* wavefronts per gate workgroup (4 or 8) */
  int32_t gate_splits;             /* K split: partial sum arrays */
  int32_t gate_stage_bytes;        /* bytes of each tile row per stage; 0: register-staged */
  int32_t gate_ring_depth;         /* stages of x in the LDS ring (of W too, except for
                                      the largest tiles, whose W ring is one stage shorter) */
  int32_t gate_lds_bytes;          /* LDS of the ring */
  int32_t select_lanes;            /* lanes per token of the selection */
  int32_t select_experts_per_lane;
  int32_t hist_tokens;             /* tokens per dispatch tile the routing kernels count; 0: none */
  int32_t kernels;                 /* kernels enqueued per call */
} moe_plan_info;
int32_t moe_route_dispatch_plan(const moe_route_params* p, int32_t aligned, moe_plan_info* out);

/*
 * moe_combine -- a token's layer output from the outputs its experts
 * produced for it: the weighted sum over its selected experts, plus a
 * shared expert's output ("Feature Request: dynamic number of experts",
 * Possible Implementation: the selected experts' outputs combined with
 * their weights; "ferrox_moe", combine_expert_outputs: routed plus shared
 * expert outputs of one token).  Expert outputs come in dispatch order, so
 * slot j of token t reads row inv[t*k_stride + j] of Yp.
 *   Yp       [R][d] expert outputs; row p is the output for route perm[p]
 *            (R = offsets[E] of the dispatch; dtype MOE_F32 or MOE_BF16)
 *   inv      [T*k_stride] as written by moe_dispatch; < 0: empty slot
 *   weights  [T][k_stride] fp32 combine weights (as written by moe_route)
 *   shared   [T][d] a shared expert's output (weight 1), or NULL
 *   y        [T][d] out, dtype as Yp: sum over the valid slots, in slot
 *            order, of weights[t][j] * Yp[inv[t*k_stride+j]], then +
 *            shared[t]; accumulated in fp32, stored rounded to nearest (even)
 *   dev_err  [1] or NULL: += number of slots with inv >= R (left out)
 * All pointers are caller-owned device memory; y must not overlap the
 * inputs.  Asynchronous on `stream`.  Limits: k_stride <= MOE_MAX_K,
 * T*k_stride < 2^31.  Returns MOE_OK, MOE_EINVAL (bad sizes, dtype or a
 * required NULL pointer) or MOE_EDEVICE.
 */
int32_t moe_combine(int32_t T, int32_t k_stride, int32_t d, int32_t dtype, const void* Yp,
                    int32_t R, const int32_t* inv, const float* weights, const void* shared,
                    void* y, int32_t* dev_err, void* stream);

/*
 * Per-kernel timing, for benchmarks and profiling only.
 * moe_profile_enable(1) clears earlier records and, from then on, gives
 * every kernel the library launches a start and a stop HIP event that the
 * runtime sets when the kernel itself starts and ends (hipExtLaunchKernel;
 * the events are created on the host per launch); moe_profile_enable(0)
 * stops recording.  moe_profile_read waits for the
 * recorded events and fills ms[i] (summed kernel time, milliseconds) and
 * launches[i] for the kernels MOE_STAGE_* = i < n; it returns
 * MOE_NUM_STAGES.  Records are process-wide.
 */
#define MOE_STAGE_GATE 0         /* gate contraction */
#define MOE_STAGE_SELECT 1       /* score + select + weights */
#define MOE_STAGE_HASH 2         /* hash routing */
#define MOE_STAGE_DISP_HIST 3    /* dispatch: tile histograms */
#define MOE_STAGE_DISP_SCAN 4    /* dispatch: scans */
#define MOE_STAGE_DISP_SCATTER 5 /* dispatch: permutation */
#define MOE_STAGE_GATE_SELECT 6  /* gate contraction with the selection fused */
#define MOE_STAGE_SELECT_DISPATCH 7 /* selection + dispatch of a small batch */
#define MOE_STAGE_COMBINE 8      /* combine of expert outputs */
#define MOE_STAGE_CAPACITY 9     /* capacity limit on a dispatch */
#define MOE_STAGE_PERMUTE 10     /* send buffer rows */
#define MOE_STAGE_EP_LAYOUT 11   /* per-rank send layout */
#define MOE_STAGE_HASH_IDS 12    /* hash layer: the table's ids only */
#define MOE_STAGE_HASH_DOTS 13   /* hash layer: k dot products per token */
#define MOE_NUM_STAGES 14
int32_t moe_profile_enable(int32_t enable);
int32_t moe_profile_read(double* ms, int64_t* launches, int32_t n);

/* Text describing the last non-zero return of a call on this thread. */
const char* moe_last_error(void);

/* MOE_ABI_VERSION of the loaded library. */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
