// C ABI of the MoE router / dispatch library: argument validation on the
// host, thread-local error text, and kernel launches on the caller's stream.
// Every check here runs before anything is enqueued and touches no device
// state, so an invalid call never reaches the GPU.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "moe_route.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int32_t device_fail(hipError_t e, const char* what) {
  return fail(MOE_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kI32Max = 2147483647;

// Checks shared by moe_route and moe_route_hash.
int32_t check_common(const moe_route_params* p, bool need_d) {
  if (!p) return fail(MOE_EINVAL, "params is NULL");
  if (p->T < 0) return fail(MOE_EINVAL, "T=%d must be >= 0", p->T);
  if (need_d && p->d < 1) return fail(MOE_EINVAL, "d=%d must be >= 1", p->d);
  if (p->E < 1) return fail(MOE_EINVAL, "E=%d must be >= 1", p->E);
  if (p->E > MOE_MAX_EXPERTS)
    return fail(MOE_EUNSUPPORTED, "E=%d exceeds MOE_MAX_EXPERTS=%d", p->E, MOE_MAX_EXPERTS);
  if (p->k < 1) return fail(MOE_EINVAL, "k=%d must be >= 1", p->k);
  if (p->k > MOE_MAX_K) return fail(MOE_EUNSUPPORTED, "k=%d exceeds MOE_MAX_K=%d", p->k, MOE_MAX_K);
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16)
    return fail(MOE_EINVAL, "dtype=%d is not MOE_F32 or MOE_BF16", p->dtype);
  if (p->score < MOE_SCORE_SOFTMAX || p->score > MOE_SCORE_SOFTMAX_TOPK)
    return fail(MOE_EINVAL, "score=%d is not a MOE_SCORE_* value", p->score);
  if (p->renormalize != 0 && p->renormalize != 1)
    return fail(MOE_EINVAL, "renormalize=%d must be 0 or 1", p->renormalize);
  if (!std::isfinite(p->route_scale))
    return fail(MOE_EINVAL, "route_scale must be finite");
  if ((int64_t)p->T * p->k > kI32Max)
    return fail(MOE_EUNSUPPORTED, "T*k=%lld must be below 2^31", (long long)p->T * p->k);
  if (need_d && (int64_t)p->T * p->d > kI32Max)
    return fail(MOE_EUNSUPPORTED, "T*d must be below 2^31");
  return MOE_OK;
}

moe::RouteCfg to_cfg(const moe_route_params* p) {
  moe::RouteCfg c;
  c.T = p->T;
  c.d = p->d;
  c.E = p->E;
  c.k = p->k;
  c.score = p->score;
  c.n_groups = p->n_groups;
  c.topk_groups = p->topk_groups;
  c.group_score = p->group_score;
  c.renormalize = p->renormalize;
  c.route_scale = p->route_scale;
  c.k_per_group = p->k_per_group;
  return c;
}

// ---- optional per-kernel event timing --------------------------------------
struct ProfRecord {
  int32_t stage;
  hipEvent_t begin, end;
};
std::atomic<bool> g_prof_on{false};
std::mutex g_prof_mu;
std::vector<ProfRecord> g_prof_records;
// Set while moe_route_dispatch_noalloc runs on this thread: its launches
// carry no timing events (creating them would allocate).
thread_local bool g_no_events = false;

void prof_clear_locked() {
  for (auto& r : g_prof_records) {
    (void)hipEventDestroy(r.begin);
    (void)hipEventDestroy(r.end);
  }
  g_prof_records.clear();
}

// Every check of moe_route's parameters (shape, flags, limits).
int32_t check_route_params(const moe_route_params* p, bool need_d) {
  int32_t rc = check_common(p, need_d);
  if (rc != MOE_OK) return rc;
  if (p->k > p->E) return fail(MOE_EINVAL, "k=%d exceeds E=%d", p->k, p->E);
  if (p->n_groups < 1) return fail(MOE_EINVAL, "n_groups=%d must be >= 1", p->n_groups);
  if (p->n_groups > MOE_MAX_GROUPS)
    return fail(MOE_EUNSUPPORTED, "n_groups=%d exceeds MOE_MAX_GROUPS=%d", p->n_groups,
                MOE_MAX_GROUPS);
  if (p->E % p->n_groups != 0)
    return fail(MOE_EINVAL, "n_groups=%d does not divide E=%d", p->n_groups, p->E);
  if (p->topk_groups < 1 || p->topk_groups > p->n_groups)
    return fail(MOE_EINVAL, "topk_groups=%d must be in [1, n_groups=%d]", p->topk_groups,
                p->n_groups);
  if (p->group_score != MOE_GROUP_MAX && p->group_score != MOE_GROUP_TOP2_SUM)
    return fail(MOE_EINVAL, "group_score=%d is not a MOE_GROUP_* value", p->group_score);
  const int32_t gs = p->E / p->n_groups;
  if (p->k_per_group < 0) return fail(MOE_EINVAL, "k_per_group=%d must be >= 0", p->k_per_group);
  if (p->k_per_group > 0) {
    if (p->topk_groups != p->n_groups)
      return fail(MOE_EINVAL, "k_per_group > 0 takes no group limit (topk_groups = n_groups)");
    const int32_t keep = p->n_groups * std::min(p->k_per_group, gs);
    if (p->k > keep)
      return fail(MOE_EINVAL, "k=%d exceeds the %d experts the groups keep", p->k, keep);
  }
  if ((int64_t)p->k > (int64_t)p->topk_groups * gs)
    return fail(MOE_EINVAL, "k=%d exceeds the %d experts of the kept groups", p->k,
                p->topk_groups * gs);
  if (p->n_groups > 1 && p->group_score == MOE_GROUP_TOP2_SUM && gs < 2)
    return fail(MOE_EINVAL, "MOE_GROUP_TOP2_SUM needs groups of at least 2 experts");
  if ((int64_t)p->T * p->E > kI32Max) return fail(MOE_EUNSUPPORTED, "T*E must be below 2^31");
  return MOE_OK;
}

}  // namespace

namespace moe {

void prof_events(Stage st, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (g_no_events || !g_prof_on.load(std::memory_order_relaxed)) return;
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess) return;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return;
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_records.push_back({(int32_t)st, a, b});
  *start = a;
  *stop = b;
}

}  // namespace moe

extern "C" {

int32_t moe_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_clear_locked();
  g_prof_on.store(enable != 0);
  return MOE_OK;
}

int32_t moe_profile_read(double* ms, int64_t* launches, int32_t n) {
  if (!ms || !launches || n < 0) return fail(MOE_EINVAL, "ms and launches are required");
  for (int32_t i = 0; i < n; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof_records) {
    hipError_t e = hipEventSynchronize(r.end);
    if (e != hipSuccess) return device_fail(e, "event synchronize");
    float t = 0.f;
    e = hipEventElapsedTime(&t, r.begin, r.end);
    if (e != hipSuccess) return device_fail(e, "event elapsed time");
    if (r.stage < n) {
      ms[r.stage] += t;
      launches[r.stage] += 1;
    }
  }
  return moe::kNumStages;
}

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// Dispatch outputs when a small batch is routed and dispatched by one kernel.
struct SmallDispatch {
  int32_t *counts, *offsets, *perm, *inv;
  double* maxvio;
};

// Gate + select of moe_route on validated arguments (T > 0, ids and weights
// set, logits set in select-only mode).  `hist`: optional per-tile expert
// histograms for a fused dispatch (launch_select); `super_sum`: with hist
// and the gate, super-tile sums of super_words int32 that the gate kernel
// zeroes and the select kernel adds into.  `sd` (small_dispatch_ok batches
// only): the selection kernel also performs the dispatch.
int32_t route_core(const moe_route_params* p, const void* x, const void* W,
                   const float* logit_bias, const float* select_bias,
                   const int32_t* k_per_token, float* logits, int32_t* ids, float* weights,
                   void* workspace, size_t workspace_bytes, int32_t* dev_err, moe::hist_t* hist,
                   hipStream_t s, const SmallDispatch* sd = nullptr,
                   int32_t* super_sum = nullptr, int32_t super_words = 0) {
  const moe::RouteCfg c = to_cfg(p);
  hipError_t e;
  if (x == nullptr) {  // select-only
    if (sd)
      e = moe::launch_route_dispatch_small(c, logits, 1, 0, nullptr, logit_bias, select_bias,
                                           k_per_token, ids, weights, dev_err, sd->counts,
                                           sd->offsets, sd->perm, sd->inv, sd->maxvio, s);
    else if (super_sum)
      return fail(MOE_EINVAL, "super-tile sums need the gate kernel");
    else
      e = moe::launch_select(c, logits, 1, 0, nullptr, logit_bias, select_bias, k_per_token,
                             ids, weights, dev_err, hist, nullptr, s);
    if (e != hipSuccess) return device_fail(e, "select launch");
    return MOE_OK;
  }
  const bool aligned = reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(W) % 16 == 0;
  moe::GatePlan g = moe::plan_gate(p->T, p->d, p->E, p->dtype, aligned, true);
  if (!sd && moe::gate_select_tokens(g, p->dtype, c) > 0) {  // one kernel: logits stay in LDS
    moe::SelectArgs sa{};
    sa.c = c;
    sa.select_bias = select_bias;
    sa.k_per_token = k_per_token;
    sa.ids = ids;
    sa.weights = weights;
    sa.dev_err = dev_err;
    sa.hist = hist;
    sa.write_logits = logits != nullptr;
    sa.vec = p->E % 4 == 0 && (!select_bias || reinterpret_cast<uintptr_t>(select_bias) % 16 == 0);
    e = moe::launch_gate_select(g, p->dtype, x, W, logit_bias, logits, sa, s);
    if (e != hipSuccess) return device_fail(e, "gate + select launch");
    return MOE_OK;
  }
  const size_t te = (size_t)p->T * p->E * sizeof(float);
  float* hand_off = nullptr;
  if (workspace && workspace_bytes >= te * g.splits) {
    hand_off = static_cast<float*>(workspace);
    if (g.splits == 1 && logits) hand_off = logits;
  } else if (logits) {
    g = moe::plan_gate(p->T, p->d, p->E, p->dtype, aligned, false);
    hand_off = logits;  // no room for partial sums: unsplit, through logits
  } else {
    return fail(MOE_EINVAL, "workspace of %zu bytes is below the %zu needed (or pass logits)",
                workspace_bytes, te * g.splits);
  }
  e = moe::launch_gate_gemm(g, p->dtype, x, W, logit_bias, hand_off, p->T, p->d, p->E, s,
                            super_sum, super_sum ? super_words : 0);
  if (e != hipSuccess) return device_fail(e, "gate GEMM launch");
  if (sd)
    e = moe::launch_route_dispatch_small(c, hand_off, g.splits, (int64_t)p->T * p->E,
                                         g.splits > 1 ? logits : nullptr, nullptr, select_bias,
                                         k_per_token, ids, weights, dev_err, sd->counts,
                                         sd->offsets, sd->perm, sd->inv, sd->maxvio, s);
  else
    e = moe::launch_select(c, hand_off, g.splits, (int64_t)p->T * p->E,
                           g.splits > 1 ? logits : nullptr, nullptr, select_bias, k_per_token,
                           ids, weights, dev_err, hist, super_sum, s);
  if (e != hipSuccess) return device_fail(e, "select launch");
  return MOE_OK;
}

// Argument checks shared by moe_route and moe_route_dispatch.
int32_t check_route_call(const moe_route_params* p, const void* x, const void* W,
                         const float* logits, const int32_t* ids, const float* weights) {
  const bool select_only = (x == nullptr && W == nullptr);
  int32_t rc = check_route_params(p, !select_only);
  if (rc != MOE_OK) return rc;
  if (p->T > 0 && (x == nullptr) != (W == nullptr))
    return fail(MOE_EINVAL, "x and W must both be set or both be NULL");
  if (p->T == 0) return MOE_OK;
  if (!ids || !weights) return fail(MOE_EINVAL, "ids and weights are required");
  if (select_only && !logits)
    return fail(MOE_EINVAL, "select-only mode (x = W = NULL) needs logits");
  return MOE_OK;
}

size_t route_ws_bytes(const moe_route_params* p) {
  const moe::GatePlan g = moe::plan_gate(p->T, p->d, p->E, p->dtype, true, true);
  return (size_t)p->T * p->E * sizeof(float) * g.splits;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// The hash layer's hand-off: the per-slice partial dot products when the
// dot-product kernel applies (aligned rows assumed, as for route_ws_bytes),
// else the gate's logits of every expert.
size_t hash_ws_bytes(const moe_route_params* p) {
  const int ns = moe::hash_dot_slices(to_cfg(p), p->dtype, true);
  if (ns > 0) return (size_t)ns * p->T * p->k * sizeof(float);
  return route_ws_bytes(p);
}

// How moe_route_dispatch counts its routes for the dispatch.
//   kOwn:   the dispatch's own kernels (histogram, [scan,] placement);
//   kTiles: the routing kernels write each tile's histogram (tiles of
//           `tokens` tokens), the placement reads every tile's counts --
//           the gate kernel with the selection fused, or the select kernel
//           in select-only mode;
//   kSuper: the select kernel after the (pipelined) gate kernel also adds
//           each tile's counts into super-tile sums, which the gate kernel
//           zeroed; the placement reads about 2 sqrt(tiles) rows.
// `gate`: x and W are given; `aligned`: both are 16-byte aligned.
enum DispMode { kOwn = 0, kTiles = 1, kSuper = 2 };
struct DispPlan {
  int mode = kOwn;
  int tokens = 0;
  int64_t tiles = 0, supers = 0;
  size_t hist_bytes = 0, super_bytes = 0;
};

DispPlan disp_plan(const moe_route_params* p, bool gate, bool aligned) {
  const moe::RouteCfg c = to_cfg(p);
  const int64_t R = (int64_t)p->T * p->k;
  DispPlan d;
  int n = 0, mode = kOwn;
  if (gate) {
    const moe::GatePlan g = moe::plan_gate(p->T, p->d, p->E, p->dtype, aligned, true);
    const int nf = moe::gate_select_tokens(g, p->dtype, c);
    if (nf > 0) {
      if (!moe::dispatch_hist_ok(R, p->E, nf * p->k)) return d;
      n = nf;
      mode = kTiles;
    } else if (g.pipe && !std::getenv("MOE_DISPATCH_NO_SUPER")) {
      n = moe::select_super_tokens(c);
      mode = n > 0 ? kSuper : kOwn;
    }
  }
  if (mode == kOwn) {
    n = moe::select_hist_tokens(c);
    if (n <= 0 || !moe::dispatch_hist_ok(R, p->E, n * p->k)) return d;
    mode = kTiles;
  }
  d.mode = mode;
  d.tokens = n;
  d.tiles = (p->T + n - 1) / n;
  d.hist_bytes = (size_t)d.tiles * p->E * sizeof(moe::hist_t);
  if (mode == kSuper) {
    const int S = moe::dispatch_super_size(R, n * p->k);
    d.supers = (d.tiles + S - 1) / S;
    d.super_bytes = (size_t)d.supers * p->E * sizeof(int32_t);
  }
  return d;
}

// Dispatch part of the moe_route_dispatch workspace for a given plan.
size_t disp_ws_bytes(const moe_route_params* p, const DispPlan& d) {
  if (d.mode == kOwn) return moe::dispatch_workspace_bytes((int64_t)p->T * p->k, p->E);
  if (d.mode == kTiles) return d.hist_bytes;
  return align256(d.hist_bytes) + d.super_bytes;
}

}  // namespace

extern "C" {

int32_t moe_route(const moe_route_params* p, const void* x, const void* W,
                  const float* logit_bias, const float* select_bias,
                  const int32_t* k_per_token, float* logits, int32_t* ids,
                  float* weights, void* workspace, size_t workspace_bytes,
                  int32_t* dev_err, void* stream) {
  int32_t rc = check_route_call(p, x, W, logits, ids, weights);
  if (rc != MOE_OK || p->T == 0) return rc;
  return route_core(p, x, W, logit_bias, select_bias, k_per_token, logits, ids, weights,
                    workspace, workspace_bytes, dev_err, nullptr,
                    static_cast<hipStream_t>(stream));
}

size_t moe_route_dispatch_workspace_size(const moe_route_params* p) {
  if (check_route_params(p, true) != MOE_OK) return 0;
  const int64_t R = (int64_t)p->T * p->k;
  if (R > kI32Max) return 0;
  if (p->T == 0) return moe::dispatch_workspace_bytes(R, p->E);
  // enough for every path the call may take (aligned or not, gate or not)
  size_t disp = 0;
  for (int path = 0; path < 3; ++path)
    disp = std::max(disp, disp_ws_bytes(p, disp_plan(p, path < 2, path == 0)));
  return align256(route_ws_bytes(p)) + disp;
}

int32_t moe_route_dispatch(const moe_route_params* p, const void* x, const void* W,
                           const float* logit_bias, const float* select_bias,
                           const int32_t* k_per_token, float* logits, int32_t* ids,
                           float* weights, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv, double* maxvio, void* workspace,
                           size_t workspace_bytes, int32_t* dev_err, void* stream) {
  int32_t rc = check_route_call(p, x, W, logits, ids, weights);
  if (rc != MOE_OK) return rc;
  const int64_t R = (int64_t)p->T * p->k;
  if (R > kI32Max) return fail(MOE_EUNSUPPORTED, "T*k must be below 2^31");
  if (!counts || !offsets) return fail(MOE_EINVAL, "counts and offsets are required");
  if (R > 0 && !perm) return fail(MOE_EINVAL, "perm is required");
  const size_t need = moe_route_dispatch_workspace_size(p);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MOE_EINVAL, "workspace of %zu bytes is below the %zu needed", workspace_bytes,
                need);
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(MOE_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (p->T == 0) {  // zero counts and offsets only
    e = moe::launch_dispatch(ids, 0, p->E, counts, offsets, perm, inv, maxvio, nullptr, dev_err,
                             s);
    if (e != hipSuccess) return device_fail(e, "dispatch launch");
    return MOE_OK;
  }
  const size_t route = align256(route_ws_bytes(p));
  if (moe::small_dispatch_ok(to_cfg(p)) && !std::getenv("MOE_NO_SMALL_DISPATCH")) {
    const SmallDispatch sd{counts, offsets, perm, inv, maxvio};
    return route_core(p, x, W, logit_bias, select_bias, k_per_token, logits, ids, weights,
                      workspace, route, dev_err, nullptr, s, &sd);
  }
  void* disp_ws = static_cast<char*>(workspace) + route;
  const bool gate = x != nullptr;
  const bool aligned = reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(W) % 16 == 0;
  const DispPlan dp = disp_plan(p, gate, aligned);
  moe::hist_t* hist = dp.mode != kOwn ? static_cast<moe::hist_t*>(disp_ws) : nullptr;
  int32_t* super_sum =
      dp.mode == kSuper
          ? reinterpret_cast<int32_t*>(static_cast<char*>(disp_ws) + align256(dp.hist_bytes))
          : nullptr;
  rc = route_core(p, x, W, logit_bias, select_bias, k_per_token, logits, ids, weights,
                  workspace, route, dev_err, hist, s, nullptr, super_sum,
                  (int32_t)(dp.supers * p->E));
  if (rc != MOE_OK) return rc;
  if (dp.mode == kSuper)
    e = moe::launch_dispatch_from_super(ids, R, p->E, counts, offsets, perm, inv, maxvio, hist,
                                        super_sum, dp.tokens * p->k, s);
  else if (dp.mode == kTiles)
    e = moe::launch_dispatch_from_hist(ids, R, p->E, counts, offsets, perm, inv, maxvio, hist,
                                       dp.tokens * p->k, s);
  else
    e = moe::launch_dispatch(ids, R, p->E, counts, offsets, perm, inv, maxvio, disp_ws, dev_err,
                             s);
  if (e != hipSuccess) return device_fail(e, "dispatch launch");
  return MOE_OK;
}

int32_t moe_route_dispatch_plan(const moe_route_params* p, int32_t aligned,
                                moe_plan_info* out) {
  if (!out) return fail(MOE_EINVAL, "out is required");
  int32_t rc = check_route_params(p, true);
  if (rc != MOE_OK) return rc;
  const int64_t R = (int64_t)p->T * p->k;
  if (R > kI32Max) return fail(MOE_EUNSUPPORTED, "T*k must be below 2^31");
  *out = moe_plan_info{};
  const moe::RouteCfg c = to_cfg(p);
  const moe::GatePlan g = moe::plan_gate(p->T, p->d, p->E, p->dtype, aligned != 0, true);
  out->gate_bm = g.bm;
  out->gate_bn = g.bn;
  out->gate_waves = g.wm * g.wn;
  out->gate_splits = g.pipe ? g.splits : 1;
  out->gate_stage_bytes = g.pipe ? g.rb : 0;
  out->gate_ring_depth = g.pipe ? g.ns : 2;
  out->gate_lds_bytes = g.pipe ? (g.ns * g.bm + (g.nsw > 0 ? g.nsw : g.ns) * g.bn) * g.rb : 0;
  moe::select_shape(c, &out->select_lanes, &out->select_experts_per_lane);
  if (p->T == 0) {
    out->path = MOE_PATH_SEPARATE;
    out->kernels = 1;  // the dispatch writes zero counts and offsets
    return MOE_OK;
  }
  if (moe::small_dispatch_ok(c) && !std::getenv("MOE_NO_SMALL_DISPATCH")) {
    out->path = MOE_PATH_SMALL;
    out->kernels = 2;
    return MOE_OK;
  }
  const DispPlan dp = disp_plan(p, true, aligned != 0);
  out->hist_tokens = dp.tokens;
  const bool fused = moe::gate_select_tokens(g, p->dtype, c) > 0;
  out->path = fused ? MOE_PATH_FUSED
                    : dp.mode == kSuper ? MOE_PATH_SELECT_SUPER
                                        : dp.mode == kTiles ? MOE_PATH_SELECT_HIST
                                                            : MOE_PATH_SEPARATE;
  out->kernels = (fused ? 1 : 2) + (dp.mode != kOwn ? 1 : moe::dispatch_kernels(R, p->E));
  return MOE_OK;
}

size_t moe_route_workspace_size(const moe_route_params* p) {
  if (check_route_params(p, true) != MOE_OK || p->T == 0) return 0;
  return route_ws_bytes(p);
}

}  // extern "C"

namespace {

// Argument checks of moe_route_hash (and of moe_route_hash_dispatch).
int32_t check_hash_call(const moe_route_params* p, const int32_t* token_ids,
                        const int32_t* tid2eid, int32_t vocab, const void* x, const void* W,
                        const int32_t* ids, const float* weights) {
  const bool ids_only = (x == nullptr && W == nullptr);
  int32_t rc = check_common(p, !ids_only);
  if (rc != MOE_OK) return rc;
  if (p->T > 0 && (x == nullptr) != (W == nullptr))
    return fail(MOE_EINVAL, "x and W must both be set or both be NULL");
  if (vocab < 1) return fail(MOE_EINVAL, "vocab=%d must be >= 1", vocab);
  if (!ids_only && p->score == MOE_SCORE_SOFTMAX && !p->renormalize)
    return fail(MOE_EUNSUPPORTED,
                "hash routing with MOE_SCORE_SOFTMAX needs renormalize=1 (the full-softmax "
                "denominator needs every expert's logit)");
  if ((int64_t)p->T * p->E > kI32Max) return fail(MOE_EUNSUPPORTED, "T*E must be below 2^31");
  if (p->T > 0) {
    if (!token_ids || !tid2eid || !ids)
      return fail(MOE_EINVAL, "token_ids, tid2eid and ids are required");
    if (!ids_only && !weights) return fail(MOE_EINVAL, "weights are required with x and W");
  }
  return MOE_OK;
}

// Hash routing on validated arguments, T > 0.  With a workspace: when the
// shapes allow (hash_dot_slices > 0) the method's own work -- the table's
// ids, k dot products per token over slices of d (partials in the
// workspace), then the multi-token hash kernel adding them; otherwise the
// tiled gate contraction of every expert into the workspace, then the
// multi-token hash kernel (with `hist`: also the dispatch's tile histograms
// and the super-tile sums the dots or gate kernel zeroes).  With no
// workspace: the one-token-per-wavefront kernel (k dot products per token,
// or ids only).  Sets *used_tiles when the tile histograms were written.
int32_t hash_core(const moe_route_params* p, const int32_t* token_ids, const int32_t* tid2eid,
                  int32_t vocab, const void* x, const void* W, const float* logit_bias,
                  int32_t* ids, float* weights, void* workspace, size_t workspace_bytes,
                  int32_t* dev_err, hipStream_t s, moe::hist_t* hist = nullptr,
                  int32_t* super_sum = nullptr, int32_t super_words = 0,
                  bool* used_tiles = nullptr, const moe::BesidePlace* beside = nullptr,
                  bool* used_beside = nullptr) {
  const bool ids_only = (x == nullptr && W == nullptr);
  hipError_t e;
  if (used_tiles) *used_tiles = false;
  if (used_beside) *used_beside = false;
  if (!ids_only && workspace) {
    const bool aligned = reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                         reinterpret_cast<uintptr_t>(W) % 16 == 0;
    const moe::RouteCfg c = to_cfg(p);
    const int ns = moe::hash_dot_slices(c, p->dtype, aligned);
    const int64_t Rk = (int64_t)p->T * p->k;
    if (ns > 0 && workspace_bytes >= (size_t)ns * Rk * sizeof(float)) {
      float* part = static_cast<float*>(workspace);
      if (beside) {  // the dispatch placed by the dot-product kernel's free workgroups
        e = moe::launch_hash_ids_rows(c, token_ids, tid2eid, vocab, ids,
                                      const_cast<int32_t*>(beside->rows), s);
        if (e != hipSuccess) return device_fail(e, "hash ids launch");
        e = moe::launch_hash_dots_beside(c, p->dtype, x, W, part, *beside, s);
        if (e != hipSuccess) return device_fail(e, "hash dot products launch");
        e = moe::launch_hash_tiles(c, token_ids, tid2eid, vocab, part, 0, Rk, ns, logit_bias,
                                   ids, weights, dev_err, nullptr, nullptr, s);
        if (e != hipSuccess) return device_fail(e, "hash route launch");
        if (used_beside) *used_beside = true;
        return MOE_OK;
      }
      const bool tiles = hist && super_sum;
      e = moe::launch_hash_ids(c, token_ids, tid2eid, vocab, ids, s);
      if (e != hipSuccess) return device_fail(e, "hash ids launch");
      e = moe::launch_hash_dots(c, p->dtype, x, W, ids, part, tiles ? super_sum : nullptr,
                                tiles ? super_words : 0, s);
      if (e != hipSuccess) return device_fail(e, "hash dot products launch");
      e = moe::launch_hash_tiles(c, token_ids, tid2eid, vocab, part, 0, Rk, ns, logit_bias,
                                 ids, weights, dev_err, tiles ? hist : nullptr,
                                 tiles ? super_sum : nullptr, s);
      if (e != hipSuccess) return device_fail(e, "hash route launch");
      if (used_tiles) *used_tiles = tiles;
      return MOE_OK;
    }
    const size_t te = (size_t)p->T * p->E * sizeof(float);
    moe::GatePlan g = moe::plan_gate(p->T, p->d, p->E, p->dtype, aligned, true);
    if (workspace_bytes < te * g.splits)
      g = moe::plan_gate(p->T, p->d, p->E, p->dtype, aligned, false);
    if (workspace_bytes >= te * g.splits) {
      float* lg = static_cast<float*>(workspace);
      const bool tiles = hist && super_sum && g.pipe;
      e = moe::launch_gate_gemm(g, p->dtype, x, W, logit_bias, lg, p->T, p->d, p->E, s,
                                tiles ? super_sum : nullptr, tiles ? super_words : 0);
      if (e != hipSuccess) return device_fail(e, "gate GEMM launch");
      e = moe::launch_hash_tiles(c, token_ids, tid2eid, vocab, lg, g.splits,
                                 (int64_t)p->T * p->E, 0, nullptr, ids, weights, dev_err,
                                 tiles ? hist : nullptr, tiles ? super_sum : nullptr, s);
      if (e != hipSuccess) return device_fail(e, "hash route launch");
      if (used_tiles) *used_tiles = tiles;
      return MOE_OK;
    }
  }
  // logits of the k table experts only: k dot products per token
  e = moe::launch_hash_route(to_cfg(p), p->dtype, token_ids, tid2eid, vocab, x, W, logit_bias,
                             nullptr, 1, (int64_t)p->T * p->E, ids,
                             ids_only ? nullptr : weights, dev_err, s);
  if (e != hipSuccess) return device_fail(e, "hash route launch");
  return MOE_OK;
}

// Rows of counts for the dispatch placed beside the hash layer's dot
// products (0 when that form does not apply to these shapes).
size_t beside_rows_bytes(const moe_route_params* p) {
  if (moe::hash_beside_places(to_cfg(p), p->dtype, true) < 1) return 0;
  const int64_t R = (int64_t)p->T * p->k;
  return (size_t)((R + moe::kBesideTile - 1) / moe::kBesideTile) * p->E * sizeof(int32_t);
}

// Tile histograms plus super-tile sums of moe_route_hash_dispatch.
DispPlan hash_disp_plan(const moe_route_params* p) {
  DispPlan d;
  const int64_t R = (int64_t)p->T * p->k;
  const int n = moe::hash_tile_tokens(p->k);
  if (p->T == 0 || !moe::dispatch_super_ok(R, p->E, n * p->k)) return d;
  d.mode = kSuper;
  d.tokens = n;
  d.tiles = (p->T + n - 1) / n;
  d.hist_bytes = (size_t)d.tiles * p->E * sizeof(moe::hist_t);
  const int S = moe::dispatch_super_size(R, n * p->k);
  d.supers = (d.tiles + S - 1) / S;
  d.super_bytes = (size_t)d.supers * p->E * sizeof(int32_t);
  return d;
}

}  // namespace

extern "C" {

int32_t moe_route_hash(const moe_route_params* p, const int32_t* token_ids,
                       const int32_t* tid2eid, int32_t vocab, const void* x,
                       const void* W, const float* logit_bias, int32_t* ids,
                       float* weights, void* workspace, size_t workspace_bytes,
                       int32_t* dev_err, void* stream) {
  int32_t rc = check_hash_call(p, token_ids, tid2eid, vocab, x, W, ids, weights);
  if (rc != MOE_OK || p->T == 0) return rc;
  return hash_core(p, token_ids, tid2eid, vocab, x, W, logit_bias, ids, weights, workspace,
                   workspace_bytes, dev_err, static_cast<hipStream_t>(stream));
}

size_t moe_route_hash_dispatch_workspace_size(const moe_route_params* p) {
  if (check_common(p, true) != MOE_OK) return 0;
  const int64_t R = (int64_t)p->T * p->k;
  if ((int64_t)p->T * p->E > kI32Max) return 0;
  if (p->T == 0) return 0;
  const DispPlan d = hash_disp_plan(p);
  const size_t disp = std::max({disp_ws_bytes(p, d), moe::dispatch_workspace_bytes(R, p->E),
                                beside_rows_bytes(p)});
  return align256(hash_ws_bytes(p)) + disp;
}

int32_t moe_route_hash_dispatch(const moe_route_params* p, const int32_t* token_ids,
                                const int32_t* tid2eid, int32_t vocab, const void* x,
                                const void* W, const float* logit_bias, int32_t* ids,
                                float* weights, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* inv, double* maxvio, void* workspace,
                                size_t workspace_bytes, int32_t* dev_err, void* stream) {
  if (x == nullptr || W == nullptr) return fail(MOE_EINVAL, "x and W are required");
  int32_t rc = check_hash_call(p, token_ids, tid2eid, vocab, x, W, ids, weights);
  if (rc != MOE_OK) return rc;
  if (!counts || !offsets) return fail(MOE_EINVAL, "counts and offsets are required");
  const int64_t R = (int64_t)p->T * p->k;
  if (R > 0 && !perm) return fail(MOE_EINVAL, "perm is required");
  if (p->E > MOE_MAX_EXPERTS)
    return fail(MOE_EUNSUPPORTED, "E=%d exceeds MOE_MAX_EXPERTS=%d", p->E, MOE_MAX_EXPERTS);
  const size_t need = moe_route_hash_dispatch_workspace_size(p);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MOE_EINVAL, "workspace of %zu bytes is below the %zu needed", workspace_bytes,
                need);
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(MOE_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (p->T == 0) {  // zero counts and offsets only
    e = moe::launch_dispatch(ids, 0, p->E, counts, offsets, perm, inv, maxvio, nullptr, dev_err,
                             s);
    if (e != hipSuccess) return device_fail(e, "dispatch launch");
    return MOE_OK;
  }
  const size_t route = align256(hash_ws_bytes(p));
  void* disp_ws = static_cast<char*>(workspace) + route;
  const bool aligned = reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(W) % 16 == 0;
  const int n_place = moe::hash_beside_places(to_cfg(p), p->dtype, aligned);
  if (n_place > 0 && beside_rows_bytes(p) > 0) {
    // every tile's row of counts in the dispatch part of the workspace
    moe::BesidePlace bp;
    bp.ids = ids;
    bp.R = R;
    bp.E = p->E;
    bp.nt = (int32_t)((R + moe::kBesideTile - 1) / moe::kBesideTile);
    bp.n_place = n_place;
    bp.rows = static_cast<const int32_t*>(disp_ws);
    bp.counts = counts;
    bp.offsets = offsets;
    bp.perm = perm;
    bp.inv = inv;
    bp.maxvio = maxvio;
    bp.n_dots = 0;
    bool placed = false;
    rc = hash_core(p, token_ids, tid2eid, vocab, x, W, logit_bias, ids, weights, workspace,
                   route, dev_err, s, nullptr, nullptr, 0, nullptr, &bp, &placed);
    if (rc != MOE_OK || placed) return rc;
    // routed by another kernel (no dot products): the plain dispatch of its ids
    e = moe::launch_dispatch(ids, R, p->E, counts, offsets, perm, inv, maxvio, disp_ws, dev_err,
                             s);
    if (e != hipSuccess) return device_fail(e, "dispatch launch");
    return MOE_OK;
  }
  const DispPlan dp = hash_disp_plan(p);
  moe::hist_t* hist = dp.mode == kSuper ? static_cast<moe::hist_t*>(disp_ws) : nullptr;
  int32_t* super_sum =
      dp.mode == kSuper
          ? reinterpret_cast<int32_t*>(static_cast<char*>(disp_ws) + align256(dp.hist_bytes))
          : nullptr;
  bool tiles = false;
  rc = hash_core(p, token_ids, tid2eid, vocab, x, W, logit_bias, ids, weights, workspace,
                 route, dev_err, s, hist, super_sum, (int32_t)(dp.supers * p->E), &tiles);
  if (rc != MOE_OK) return rc;
  if (tiles)
    e = moe::launch_dispatch_from_super(ids, R, p->E, counts, offsets, perm, inv, maxvio, hist,
                                        super_sum, dp.tokens * p->k, s);
  else
    e = moe::launch_dispatch(ids, R, p->E, counts, offsets, perm, inv, maxvio, disp_ws, dev_err,
                             s);
  if (e != hipSuccess) return device_fail(e, "dispatch launch");
  return MOE_OK;
}

size_t moe_route_hash_workspace_size(const moe_route_params* p) {
  if (check_common(p, true) != MOE_OK || p->T == 0) return 0;
  if ((int64_t)p->T * p->E > kI32Max) return 0;
  return hash_ws_bytes(p);
}

size_t moe_dispatch_workspace_size(int32_t T, int32_t k_stride, int32_t E) {
  if (T < 0 || k_stride < 1 || E < 1) return 0;
  return moe::dispatch_workspace_bytes((int64_t)T * k_stride, E);
}

int32_t moe_dispatch(const int32_t* ids, int32_t T, int32_t k_stride, int32_t E,
                     int32_t* counts, int32_t* offsets, int32_t* perm,
                     int32_t* inv, double* maxvio, void* workspace, size_t workspace_bytes,
                     int32_t* dev_err, void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T=%d must be >= 0", T);
  if (k_stride < 1) return fail(MOE_EINVAL, "k_stride=%d must be >= 1", k_stride);
  if (E < 1) return fail(MOE_EINVAL, "E=%d must be >= 1", E);
  if (E > MOE_MAX_EXPERTS)
    return fail(MOE_EUNSUPPORTED, "E=%d exceeds MOE_MAX_EXPERTS=%d", E, MOE_MAX_EXPERTS);
  const int64_t R = (int64_t)T * k_stride;
  if (R > kI32Max) return fail(MOE_EUNSUPPORTED, "T*k_stride must be below 2^31");
  if (!counts || !offsets) return fail(MOE_EINVAL, "counts and offsets are required");
  if (R > 0 && (!ids || !perm)) return fail(MOE_EINVAL, "ids and perm are required");
  const size_t need = moe::dispatch_workspace_bytes(R, E);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MOE_EINVAL, "workspace of %zu bytes is below the %zu needed", workspace_bytes,
                need);
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(MOE_EINVAL, "workspace must be 16-byte aligned");
  hipError_t e = moe::launch_dispatch(ids, R, E, counts, offsets, perm, inv, maxvio, workspace,
                                      dev_err, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "dispatch launch");
  return MOE_OK;
}

int32_t moe_combine(int32_t T, int32_t k_stride, int32_t d, int32_t dtype, const void* Yp,
                    int32_t R, const int32_t* inv, const float* weights, const void* shared,
                    void* y, int32_t* dev_err, void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T=%d must be >= 0", T);
  if (d < 0) return fail(MOE_EINVAL, "d=%d must be >= 0", d);
  if (R < 0) return fail(MOE_EINVAL, "R=%d must be >= 0", R);
  if (k_stride < 1) return fail(MOE_EINVAL, "k_stride=%d must be >= 1", k_stride);
  if (k_stride > MOE_MAX_K)
    return fail(MOE_EUNSUPPORTED, "k_stride=%d exceeds MOE_MAX_K=%d", k_stride, MOE_MAX_K);
  if (dtype != MOE_F32 && dtype != MOE_BF16)
    return fail(MOE_EINVAL, "dtype=%d is not MOE_F32 or MOE_BF16", dtype);
  if ((int64_t)T * k_stride > kI32Max)
    return fail(MOE_EUNSUPPORTED, "T*k_stride must be below 2^31");
  if (T == 0 || d == 0) return MOE_OK;
  if (!inv || !weights || !y) return fail(MOE_EINVAL, "inv, weights and y are required");
  if (R > 0 && !Yp) return fail(MOE_EINVAL, "Yp is required when R > 0");
  hipError_t e = moe::launch_combine(T, k_stride, d, dtype, Yp, R, inv, weights, shared, y,
                                     dev_err, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "combine launch");
  return MOE_OK;
}

int32_t moe_dispatch_capacity(const int32_t* ids, int32_t T, int32_t k_stride, int32_t E,
                              int32_t capacity, const int32_t* offsets, const int32_t* inv,
                              int32_t* slot, int32_t* kept, int32_t* dropped, void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T=%d must be >= 0", T);
  if (k_stride < 1) return fail(MOE_EINVAL, "k_stride=%d must be >= 1", k_stride);
  if (E < 1) return fail(MOE_EINVAL, "E=%d must be >= 1", E);
  if (E > MOE_MAX_EXPERTS)
    return fail(MOE_EUNSUPPORTED, "E=%d exceeds MOE_MAX_EXPERTS=%d", E, MOE_MAX_EXPERTS);
  if (capacity < 0) return fail(MOE_EINVAL, "capacity=%d must be >= 0", capacity);
  if ((int64_t)E * capacity > kI32Max)
    return fail(MOE_EUNSUPPORTED, "E*capacity must be below 2^31");
  const int64_t R = (int64_t)T * k_stride;
  if (R > kI32Max) return fail(MOE_EUNSUPPORTED, "T*k_stride must be below 2^31");
  if (!offsets || !kept || !dropped) return fail(MOE_EINVAL, "offsets, kept and dropped are required");
  if (R > 0 && (!ids || !inv || !slot)) return fail(MOE_EINVAL, "ids, inv and slot are required");
  hipError_t e = moe::launch_capacity(ids, R, E, capacity, offsets, inv, slot, kept, dropped,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "capacity launch");
  return MOE_OK;
}

int32_t moe_permute_rows(int32_t T, int32_t k_stride, int32_t d, int32_t dtype, const void* x,
                         const int32_t* inv, int32_t out_rows, void* out, int32_t* dev_err,
                         void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T=%d must be >= 0", T);
  if (k_stride < 1) return fail(MOE_EINVAL, "k_stride=%d must be >= 1", k_stride);
  if (d < 0) return fail(MOE_EINVAL, "d=%d must be >= 0", d);
  if (out_rows < 0) return fail(MOE_EINVAL, "out_rows=%d must be >= 0", out_rows);
  if (dtype != MOE_F32 && dtype != MOE_BF16)
    return fail(MOE_EINVAL, "dtype=%d is not MOE_F32 or MOE_BF16", dtype);
  if ((int64_t)T * k_stride > kI32Max)
    return fail(MOE_EUNSUPPORTED, "T*k_stride must be below 2^31");
  if (T == 0 || d == 0) return MOE_OK;
  if (!x || !inv) return fail(MOE_EINVAL, "x and inv are required");
  if (out_rows > 0 && !out) return fail(MOE_EINVAL, "out is required when out_rows > 0");
  hipError_t e = moe::launch_permute(T, k_stride, d, dtype, x, inv, out_rows, out, dev_err,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "permute launch");
  return MOE_OK;
}

int32_t moe_ep_layout(const int32_t* offsets, int32_t E, int32_t n_ranks, int32_t* send_counts,
                      int32_t* send_offsets, void* stream) {
  if (E < 1) return fail(MOE_EINVAL, "E=%d must be >= 1", E);
  if (n_ranks < 1 || E % n_ranks != 0)
    return fail(MOE_EINVAL, "n_ranks=%d must divide E=%d", n_ranks, E);
  if (!offsets || !send_counts || !send_offsets)
    return fail(MOE_EINVAL, "offsets, send_counts and send_offsets are required");
  hipError_t e = moe::launch_ep_layout(offsets, E, n_ranks, send_counts, send_offsets,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "ep layout launch");
  return MOE_OK;
}

}  // extern "C"

// ---- moe_route_dispatch without a caller workspace ----------------------------
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops): the gate's K-split hand-off and the
// dispatch's tile histograms live in this file-scope device array instead of
// a workspace.  Every GPU the library runs on holds its own copy until the
// process ends.  No kernel needs it zeroed: each call writes every byte it
// later reads.  Calls that overlap on one GPU (two streams, or two threads)
// share the array and race.
namespace {

constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device of `stream` (looked up once
// per device, with that device current).
int32_t scratch_for_stream(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return device_fail(e, "get device");
  int dev = cur;
  if (stream) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return device_fail(e, "stream device");
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_EUNSUPPORTED, "device %d is beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return device_fail(e, "set device");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess) return device_fail(e, "scratch symbol address");
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256 != 0)
      return fail(MOE_EDEVICE, "scratch symbol address is not 256-byte aligned");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int32_t moe_route_dispatch_noalloc(
    const moe_route_params* p, const void* x, const void* W, const float* logit_bias,
    const float* select_bias, const int32_t* k_per_token, float* logits, int32_t* ids,
    float* weights, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
    double* maxvio, int32_t* dev_err, void* stream) {
  int32_t rc = check_route_call(p, x, W, logits, ids, weights);
  if (rc != MOE_OK) return rc;
  const size_t need = moe_route_dispatch_workspace_size(p);
  if (need > kScratchBytes)
    return fail(MOE_EUNSUPPORTED,
                "these shapes need %zu bytes of scratch; moe_route_dispatch_noalloc holds %zu "
                "(use moe_route_dispatch with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  rc = scratch_for_stream(static_cast<hipStream_t>(stream), &ws);
  if (rc != MOE_OK) return rc;
  g_no_events = true;
  rc = moe_route_dispatch(p, x, W, logit_bias, select_bias, k_per_token, logits, ids, weights,
                          counts, offsets, perm, inv, maxvio, ws, kScratchBytes, dev_err, stream);
  g_no_events = false;
  return rc;
}
