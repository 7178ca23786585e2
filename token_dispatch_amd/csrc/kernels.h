// Host-side launchers of the gfx950 kernels (internal to the library).
// Each launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Kernel ids for the optional per-kernel event timing (MOE_STAGE_* values).
enum Stage : int32_t {
  kStageGate = 0,
  kStageSelect = 1,
  kStageHash = 2,
  kStageDispHist = 3,
  kStageDispScan = 4,
  kStageDispScatter = 5,
  kStageGateSelect = 6,
  kStageSelectDispatch = 7,
  kStageCombine = 8,
  kStageCapacity = 9,
  kStagePermute = 10,
  kStageEpLayout = 11,
  kStageHashIds = 12,
  kStageHashDots = 13,
  kNumStages = 14
};

// Per-kernel timing (moe_profile_enable): the start/stop events of the next
// launch of stage `st`, both null while timing is off.
void prof_events(Stage st, hipEvent_t* start, hipEvent_t* stop);

// Launch `kernel` on `stream`; while per-kernel timing is on, the launch
// carries start/stop events that the runtime sets when the kernel itself
// starts and ends (hipExtLaunchKernel), not when the stream reaches them.
template <typename... KArgs, typename... Args>
hipError_t launch(Stage st, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                  hipStream_t stream, Args... args) {
  hipEvent_t start = nullptr, stop = nullptr;
  prof_events(st, &start, &stop);
  hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, args...);
  return hipGetLastError();
}

// Flattened routing configuration handed to the select kernels.
struct RouteCfg {
  int32_t T, d, E, k;
  int32_t score;        // MOE_SCORE_*
  int32_t n_groups;     // 1 = no group limit
  int32_t topk_groups;
  int32_t group_score;  // MOE_GROUP_*
  int32_t renormalize;
  float route_scale;
  int32_t k_per_group = 0;  // > 0: grouped top-k, at most this many per group
};

// How the gate contraction is tiled: BM x BN tiles worked by wm x wn
// wavefronts, an NS-stage LDS ring of stages holding RB bytes of K per tile
// row, K split over `splits` workgroups (partial sums added by the select
// kernel), pipelined (buffer -> LDS copies) or the general register-staged
// kernel.
struct GatePlan {
  int bm, bn, ns, rb, splits;
  int wm = 2, wn = 2;
  bool pipe;
  int nsw = 0;  // stages of W in the ring when fewer than of x (0: ns, one ring)
};
GatePlan plan_gate(int32_t T, int32_t d, int32_t E, int32_t dtype, bool aligned,
                   bool allow_split);

// out[s][T][E] (s < g.splits) = partial x[T][d] . W[E][d]^T over the s-th K
// range (+ logit_bias in s = 0); dtype MOE_F32 / MOE_BF16.  zero (only with
// g.pipe): zero_words int32 set to 0 by the same kernel.
hipError_t launch_gate_gemm(const GatePlan& g, int32_t dtype, const void* x, const void* W,
                            const float* logit_bias, float* out, int32_t T, int32_t d,
                            int32_t E, hipStream_t stream, int32_t* zero = nullptr,
                            int32_t zero_words = 0);

// Count of one expert in one dispatch tile of the tile-major histograms
// that the routing kernels write for the placement kernel: at most the
// routes of a tile (<= 2048), so 16 bits; every placement workgroup reads
// all of them, half as many bytes as 32-bit counts.
using hist_t = uint16_t;

// Selection arguments of the gate kernel's fused epilogue (whole-row tiles:
// the selection runs on the tile's logits in LDS).  hist: per-M-tile expert
// histograms of the dispatch (tiles of BM tokens x k routes), or NULL;
// write_logits: also store the logits; vec: 16-byte select_bias loads.
struct SelectArgs {
  RouteCfg c;
  const float* select_bias;
  const int32_t* k_per_token;
  int32_t* ids;
  float* weights;
  int32_t* dev_err;
  hist_t* hist;
  int32_t write_logits;
  int32_t vec;
  // any gate kernel of the pipelined form: zero[0 .. zero_words) is set to
  // 0, each workgroup a slice (the super-tile sums the selection kernel that
  // follows adds into)
  int32_t* zero = nullptr;
  int32_t zero_words = 0;
};

// Tokens per tile (BM) when the gate kernel of plan g can run the selection
// of c in its epilogue (one workgroup holds whole rows of logits, no K
// split), else 0.
int gate_select_tokens(const GatePlan& g, int32_t dtype, const RouteCfg& c);
// Gate + selection in one kernel (gate_select_tokens(g, dtype, sa.c) > 0);
// logits (written when sa.write_logits) may be NULL otherwise.
hipError_t launch_gate_select(const GatePlan& g, int32_t dtype, const void* x, const void* W,
                              const float* logit_bias, float* logits, const SelectArgs& sa,
                              hipStream_t stream);

// Lanes per token and experts per lane of the select kernel for c.
void select_shape(const RouteCfg& c, int* lpt, int* vpl);

// Score + (grouped) top-k + weights.  The logits are the sum of `splits`
// fp32 partial arrays `split_stride` floats apart (summed in order); when
// logits_out is not NULL the summed logits are written there.  With `hist`
// the kernel also writes hist[b][e] = picks of expert e among tokens
// [b*n, (b+1)*n): the per-tile histograms of a dispatch whose tiles hold n*k
// routes, n = select_hist_tokens(c) (super_sum NULL: for the all-counts
// placement) or n = select_super_tokens(c) (super_sum [ceil(tiles / S)][E]
// int32, zeroed beforehand: each tile's counts are also added into row
// b / S, S = dispatch_super_size(T*k, n*k)).
hipError_t launch_select(const RouteCfg& c, const float* logits, int32_t splits,
                         int64_t split_stride, float* logits_out, const float* logit_bias,
                         const float* select_bias, const int32_t* k_per_token, int32_t* ids,
                         float* weights, int32_t* dev_err, hist_t* hist, int32_t* super_sum,
                         hipStream_t stream);
int select_hist_tokens(const RouteCfg& c);   // 0: no all-counts histogram option
int select_super_tokens(const RouteCfg& c);  // 0: no super-tile histogram option

// Selection and the whole dispatch of a small batch in one workgroup (when
// small_dispatch_ok(c)): the select kernel's outputs plus moe_dispatch's
// counts, offsets, perm and inv (inv may be NULL).
bool small_dispatch_ok(const RouteCfg& c);
hipError_t launch_route_dispatch_small(const RouteCfg& c, const float* logits, int32_t splits,
                                       int64_t split_stride, float* logits_out,
                                       const float* logit_bias, const float* select_bias,
                                       const int32_t* k_per_token, int32_t* ids,
                                       float* weights, int32_t* dev_err, int32_t* counts,
                                       int32_t* offsets, int32_t* perm, int32_t* inv,
                                       double* maxvio, hipStream_t stream);

// Hash routing: table gather (+ k gathered gate dot products and weights).
// With `logits` (the sum of `splits` arrays [T][E], split_stride floats
// apart, logit bias included) the weights come from those; otherwise, when
// weights is not NULL, from k dot products of x and W (+ logit_bias).
hipError_t launch_hash_route(const RouteCfg& c, int32_t dtype,
                             const int32_t* token_ids, const int32_t* tid2eid,
                             int32_t vocab, const void* x, const void* W,
                             const float* logit_bias, const float* logits, int32_t splits,
                             int64_t split_stride, int32_t* ids, float* weights,
                             int32_t* dev_err, hipStream_t stream);

// Hash routing with several tokens per wavefront.  Weights from the gate's
// logits (splits > 0: the sum of `splits` arrays [T][E], split_stride floats
// apart, logit bias included), or (splits == 0) from n_parts arrays of
// per-slot partial dot products [T*k] (split_stride = T*k floats apart,
// launch_hash_dots) plus logit_bias.  With hist (super_sum zeroed
// beforehand): each workgroup's hash_tile_tokens(k) tokens are one dispatch
// tile; the kernel writes the tile's histogram and adds it into super_sum
// (as launch_select does).
int hash_tile_tokens(int32_t k);
hipError_t launch_hash_tiles(const RouteCfg& c, const int32_t* token_ids,
                             const int32_t* tid2eid, int32_t vocab, const float* logits,
                             int32_t splits, int64_t split_stride, int32_t n_parts,
                             const float* logit_bias, int32_t* ids, float* weights,
                             int32_t* dev_err, hist_t* hist, int32_t* super_sum,
                             hipStream_t stream);

// The table's expert ids only (checked: -1 for a bad token id or entry; no
// error count), for launch_hash_dots.
hipError_t launch_hash_ids(const RouteCfg& c, const int32_t* token_ids, const int32_t* tid2eid,
                           int32_t vocab, int32_t* ids, hipStream_t stream);

// The k logits a hash layer needs, as k dot products per token over slices
// of d (bf16 x and W, k <= 8, E <= 768, d % 8 == 0, 16-byte aligned rows:
// hash_dot_slices > 0): part[s][t*k + j] = slice s's share of x[t] . W[ids[t*k
// + j]] (0 for ids < 0); zero[0 .. zero_words) is cleared.
int hash_dot_slices(const RouteCfg& c, int32_t dtype, bool aligned);
hipError_t launch_hash_dots(const RouteCfg& c, int32_t dtype, const void* x, const void* W,
                            const int32_t* ids, float* part, int32_t* zero, int32_t zero_words,
                            hipStream_t stream);

// The dispatch of a hash layer placed beside its dot products: the table
// ids are known before any logit, so the dot-product kernel's workgroups
// past the slices x chunks grid (the CUs that grid leaves idle) place the
// dispatch tiles of kBesideTile routes while the others stream x.
// launch_hash_ids_rows writes the ids and each tile's count of every expert
// (rows[tile][E], int32); the dot-product launch then takes `place`.
// hash_beside_places gives the number of placement workgroups, or 0 when
// this form does not apply (no free CU, tiles x E too large for the
// placements to finish inside the dot products, or MOE_HASH_BESIDE=0;
// MOE_HASH_BESIDE=1 takes it whenever it is possible at all).
constexpr int kBesideTile = 2048;
struct BesidePlace {
  const int32_t* ids;
  int64_t R;
  int32_t E, nt, n_place;
  int32_t n_dots;  // slice workgroups before the placement ones (set at launch)
  const int32_t* rows;
  int32_t *counts, *offsets, *perm, *inv;
  double* maxvio;
};
int hash_beside_places(const RouteCfg& c, int32_t dtype, bool aligned);
hipError_t launch_hash_ids_rows(const RouteCfg& c, const int32_t* token_ids,
                                const int32_t* tid2eid, int32_t vocab, int32_t* ids,
                                int32_t* rows, hipStream_t stream);
hipError_t launch_hash_dots_beside(const RouteCfg& c, int32_t dtype, const void* x,
                                   const void* W, float* part, const BesidePlace& place,
                                   hipStream_t stream);

// Dispatch placement from per-tile histograms already in tile_hist
// ([ceil(R / tile_routes)][E] hist_t, tile-major), when dispatch_hist_ok
// (E % 8 == 0: 16-byte rows).
bool dispatch_hist_ok(int64_t R, int32_t E, int32_t tile_routes);
hipError_t launch_dispatch_from_hist(const int32_t* ids, int64_t R, int32_t E,
                                     int32_t* counts, int32_t* offsets, int32_t* perm,
                                     int32_t* inv, double* maxvio, const hist_t* tile_hist,
                                     int32_t tile_routes, hipStream_t stream);

// Dispatch placement from tile histograms plus super-tile sums: the routing
// kernel of tile t (tile_routes routes each) wrote hist[t][E] and added it
// into super_sum[t / S][E], S = dispatch_super_size(R, tile_routes), the
// super sums zeroed beforehand (by the gate kernel of the same call).
bool dispatch_super_ok(int64_t R, int32_t E, int32_t tile_routes);
int dispatch_super_size(int64_t R, int32_t tile_routes);
hipError_t launch_dispatch_from_super(const int32_t* ids, int64_t R, int32_t E,
                                      int32_t* counts, int32_t* offsets, int32_t* perm,
                                      int32_t* inv, double* maxvio, const hist_t* tile_hist,
                                      const int32_t* super_sum, int32_t tile_routes,
                                      hipStream_t stream);

// Combine: y[t] = sum_j weights[t][j] * Yp[inv[t*k+j]] (+ shared[t]), fp32
// accumulation, dtype 0 = fp32 / 1 = bf16 for Yp, shared and y; slots with
// inv >= R are counted in *dev_err and left out.
hipError_t launch_combine(int32_t T, int32_t k, int32_t d, int32_t dtype, const void* Yp,
                          int32_t R, const int32_t* inv, const float* weights,
                          const void* shared, void* y, int32_t* dev_err, hipStream_t stream);

// Send buffer rows out[p] = x[perm[p] / k] for p < *count (device), out
// sized for T*k rows; dtype 0 = fp32 / 1 = bf16.
hipError_t launch_permute(int32_t T, int32_t k, int32_t d, int32_t dtype, const void* x,
                          const int32_t* inv, int32_t out_rows, void* out, int32_t* dev_err,
                          hipStream_t stream);
// Per-rank send counts[N] and offsets[N+1] for N ranks of E/N experts.
hipError_t launch_ep_layout(const int32_t* offsets, int32_t E, int32_t N, int32_t* send_counts,
                            int32_t* send_offsets, hipStream_t stream);

// Capacity limit on a dispatch: slot[r] = e*C + rank for the first C routes
// of each expert (route order), else -1; kept[E]; *dropped (device).
hipError_t launch_capacity(const int32_t* ids, int64_t R, int32_t E, int32_t C,
                           const int32_t* offsets, const int32_t* inv, int32_t* slot,
                           int32_t* kept, int32_t* dropped, hipStream_t stream);

// Dispatch: tile histograms -> scan -> stable scatter.  maxvio (or NULL):
// the load statistic max_e counts[e] / (R / E) - 1 in fp64 (0 when R = 0),
// written by the kernel that writes counts.
size_t dispatch_workspace_bytes(int64_t R, int32_t E);
int dispatch_kernels(int64_t R, int32_t E);  // kernels launch_dispatch enqueues
hipError_t launch_dispatch(const int32_t* ids, int64_t R, int32_t E,
                           int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv, double* maxvio, void* workspace, int32_t* dev_err,
                           hipStream_t stream);

}  // namespace moe
