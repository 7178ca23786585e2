// Scoring, selection-only bias, group limit, top-k and weights on gfx950.
//
// Sources: "DeepSeek-V3.2-Exp - Select experts" (formula, "Explanation",
// gate-forward excerpt); ferrox_moe crate docs (route_top_k_softmax,
// _sigmoid(_with_bias), _sqrtsoftplus, _softmax_weight); llama.cpp issue
// 13572 (a per-request k over the same scores).
//
// A segment of LPT lanes (4, 8, 16 or 64) routes one token; lane i of a
// segment holds experts [i*VPL, (i+1)*VPL) in registers (about 16 per lane,
// so a segment is as narrow as E allows: the work of a top-k round is
// VALU-bound and shrinks with fewer lanes per token).  Every expert carries
// a 32-bit order-preserving key of its selection quantity.  One round of the
// top-k: each lane takes its best key (lowest slot on equal keys), the
// segment maximum comes from DPP lane permutations (VALU, no LDS), and among
// the lanes holding it the lowest lane wins (one ballot) -- so equal scores
// go to the lower expert id.  The winner clears that key and records the
// expert as the round's pick in LDS.  After k_t rounds lane j of the segment
// takes picks j, j + LPT, ..., reads their logits back from the token's LDS
// row, computes only those weights and writes ids[t][j] / weights[t][j]
// (consecutive lanes, consecutive addresses).
//
// With no selection bias and no group limit (MONO) every score function is
// strictly increasing in the logit, so the keys are the logits themselves
// (the same choice, without evaluating or saturating scores).  Otherwise the
// key is q = score + bias in fp32.  Group scores (largest q, or sum of the
// two largest) come from a butterfly over the group's lanes when a group is
// a power-of-two run of whole lanes, else from one segment reduction per
// group.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"
#include "select_core.h"

namespace moe {
namespace {

using sel::kHistMaxE;
using sel::kMaxK;
using sel::load_vals;

// Requires n_groups <= LPT (one lane per group for the ranking).  The
// logits are the sum of NSPLIT partial arrays `split_stride` floats apart (a
// K split of the gate), added in a fixed order.  `vec`: the logits, their
// split stride and the bias arrays allow 16-byte loads (E % 4 == 0).
// HIST (E <= kHistMaxE): also hist[block][e] = number of picks of expert e
// among the workgroup's TPB tokens -- the routes t*k + j of those tokens are
// one tile of the dispatch (counted with ballot peer masks, no atomics).
template <int LPT, int VPL, int NSPLIT, bool MONO, int WPB, bool HIST>
__global__ __launch_bounds__(WPB * kWave) void select_kernel(
    RouteCfg c, const float* __restrict__ logits, int64_t split_stride,
    float* __restrict__ logits_out, const float* __restrict__ logit_bias,
    const float* __restrict__ select_bias, const int32_t* __restrict__ k_per_token,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ dev_err,
    int vec, int32_t* __restrict__ hist) {
  constexpr int TPW = kWave / LPT;               // tokens per wavefront
  constexpr int TPB = WPB * TPW;                 // tokens per workgroup
  constexpr int ROW = LPT * VPL;                 // >= E
  constexpr int KPL = (kMaxK + LPT - 1) / LPT;   // output slots per lane
  __shared__ __attribute__((aligned(16))) float lrow[TPB][ROW];  // logits (+ logit_bias)
  __shared__ int32_t pick[TPB][kMaxK];                          // expert of each rank
  __shared__ int32_t whist[HIST ? WPB : 1][HIST ? kHistMaxE : 1];  // per-wave pick counts

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int seg = lane / LPT;  // token slot in the wavefront
  const int sl = lane % LPT;   // lane inside the segment
  const int tb = wave * TPW + seg;
  const int64_t t0 = ((int64_t)blockIdx.x * WPB + wave) * TPW;
  // a whole wavefront past the end leaves at once, unless HIST (block syncs)
  if (!HIST && t0 >= c.T) return;
  const int64_t t = t0 + seg;
  const bool tok_ok = t < c.T;
  const int E = c.E;
  const int e0 = sl * VPL;
  const int nval = min(max(E - e0, 0), VPL);  // this lane's experts
  const bool lvec = vec && nval == VPL;

  // logits (NSPLIT partial sums added in order), + logit_bias
  const int64_t trow = tok_ok ? t : (t0 < c.T ? t0 : (int64_t)c.T - 1);
  float lv[VPL];
  {
    float pv[NSPLIT][VPL];
#pragma unroll
    for (int sp = 0; sp < NSPLIT; ++sp)
      load_vals<VPL>(logits + sp * split_stride + trow * E, e0, E, lvec, 0.f, pv[sp]);
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      lv[j] = pv[0][j];
#pragma unroll
      for (int sp = 1; sp < NSPLIT; ++sp) lv[j] += pv[sp][j];
    }
  }
  if (NSPLIT > 1 && logits_out && tok_ok) {
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (j < nval) logits_out[t * E + e0 + j] = lv[j];
  }
  if (logit_bias) {
    float lb[VPL];
    load_vals<VPL>(logit_bias, e0, E, lvec, 0.f, lb);
#pragma unroll
    for (int j = 0; j < VPL; ++j) lv[j] += lb[j];
  }
#pragma unroll
  for (int j = 0; j < VPL; ++j)
    if (!tok_ok || j >= nval) lv[j] = -INFINITY;
#pragma unroll
  for (int j = 0; j < VPL; ++j) lrow[tb][e0 + j] = lv[j];

  int pid[KPL];
  sel::select_token<LPT, VPL, MONO>(c, sl, seg, tok_ok, t, trow, lv, nval, lvec, lrow[tb],
                                    pick[tb], select_bias, k_per_token, ids, weights, dev_err,
                                    pid);
  if constexpr (HIST) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    for (int e = lane; e < E; e += kWave) whist[wave][e] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    sel::count_picks<LPT>(pid, sl, c.k, nbits, whist[wave]);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += WPB * kWave) {
      int n = 0;
#pragma unroll
      for (int w8 = 0; w8 < WPB; ++w8) n += whist[w8][e];
      hist[(int64_t)blockIdx.x * E + e] = n;
    }
  }
}

// Waves of a workgroup that also counts its picks for the dispatch: 4, or
// 16 for one-token wavefronts (16 tokens, so that 16 tokens x k routes make
// a whole dispatch tile at k = 16).
constexpr int hist_waves(int lpt) { return lpt == kWave ? 16 : 4; }

template <int LPT, int VPL, int NS, bool MONO>
hipError_t launch_vpl(const RouteCfg& c, const float* logits, int64_t stride, float* logits_out,
                      const float* logit_bias, const float* select_bias,
                      const int32_t* k_per_token, int32_t* ids, float* weights, int32_t* dev_err,
                      int vec, int32_t* hist, hipStream_t s) {
  constexpr int tpb = 4 * (kWave / LPT);
  const int64_t blocks = ((int64_t)c.T + tpb - 1) / tpb;
  if constexpr (LPT * VPL <= kHistMaxE) {
    if (hist) {  // one dispatch tile per workgroup: hist_waves(LPT) waves
      constexpr int HW = hist_waves(LPT);
      constexpr int htpb = HW * (kWave / LPT);
      const int64_t hblocks = ((int64_t)c.T + htpb - 1) / htpb;
      return launch(kStageSelect, select_kernel<LPT, VPL, NS, MONO, HW, true>,
                    dim3((uint32_t)hblocks), dim3(HW * kWave), s, c, logits, stride, logits_out,
                    logit_bias, select_bias, k_per_token, ids, weights, dev_err, vec, hist);
    }
  }
  if (hist) return hipErrorInvalidValue;
  return launch(kStageSelect, select_kernel<LPT, VPL, NS, MONO, 4, false>, dim3((uint32_t)blocks),
                dim3(4 * kWave), s, c, logits, stride, logits_out, logit_bias, select_bias,
                k_per_token, ids, weights, dev_err, vec, (int32_t*)nullptr);
}

template <int LPT, int VPL, bool MONO>
hipError_t launch_splits(const RouteCfg& c, const float* logits, int splits, int64_t stride,
                         float* logits_out, const float* logit_bias, const float* select_bias,
                         const int32_t* k_per_token, int32_t* ids, float* weights,
                         int32_t* dev_err, int vec, int32_t* hist, hipStream_t s) {
#define MOE_S(S_)                                                                        \
  return launch_vpl<LPT, VPL, S_, MONO>(c, logits, stride, logits_out, logit_bias,       \
                                        select_bias, k_per_token, ids, weights, dev_err, \
                                        vec, hist, s)
  if (splits == 2) MOE_S(2);
  if (splits == 4) MOE_S(4);
  if (splits == 8) MOE_S(8);
  if (splits != 1) return hipErrorInvalidValue;
  MOE_S(1);
#undef MOE_S
}

template <int LPT, int VPL>
hipError_t launch_mono(const RouteCfg& c, bool mono, const float* logits, int splits,
                       int64_t stride, float* logits_out, const float* logit_bias,
                       const float* select_bias, const int32_t* k_per_token, int32_t* ids,
                       float* weights, int32_t* dev_err, int vec, int32_t* hist,
                       hipStream_t s) {
  if (mono)
    return launch_splits<LPT, VPL, true>(c, logits, splits, stride, logits_out, logit_bias,
                                         select_bias, k_per_token, ids, weights, dev_err, vec,
                                         hist, s);
  return launch_splits<LPT, VPL, false>(c, logits, splits, stride, logits_out, logit_bias,
                                        select_bias, k_per_token, ids, weights, dev_err, vec,
                                        hist, s);
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

// Segment width (lanes per token) and experts per lane for these routing
// parameters: the narrowest segment (about 16 experts per lane) that still
// ranks the groups with one lane per group -- unless that leaves fewer than
// 8 wavefronts per CU (2048 on the chip): then 16-lane segments, whose
// shorter per-lane scans cut the serial latency of each round.
void select_shape(const RouteCfg& c, int* lpt, int* vpl) {
  const int E = c.E;
  const bool grouped = c.n_groups > 1 && c.topk_groups < c.n_groups;
  const int G = grouped ? c.n_groups : 1;
  const bool few = (int64_t)c.T * 8 < 2048 * kWave;  // 8-lane segments: T / 8 wavefronts
  int l = 64, v = 16;
  if (few && G <= 16 && E <= 128) {
    l = 16;
    v = E <= 16 ? 1 : E <= 32 ? 2 : E <= 64 ? 4 : 8;
  } else if (E <= 16 && G <= 4) {
    l = 4, v = 4;
  } else if (E <= 32 && G <= 4) {
    l = 4, v = 8;
  } else if (E <= 64 && G <= 8) {
    l = 8, v = 8;
  } else if (E <= 128 && G <= 8) {
    l = 8, v = 16;
  } else if (E <= 256 && G <= 16) {
    l = 16, v = 16;
  } else if (E <= 384 && G <= 16) {
    l = 16, v = 24;
  } else {
    v = E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16;
  }
  // MOE_SELECT_LPT=4|8|16|64 forces the segment width (tuning sweeps)
  if (const char* env = std::getenv("MOE_SELECT_LPT")) {
    const int want = std::atoi(env);
    const int vw = (E + want - 1) / want;
    if (want == 64 && vw <= 16) {
      l = 64;
      v = vw <= 1 ? 1 : vw <= 2 ? 2 : vw <= 4 ? 4 : vw <= 8 ? 8 : 16;
    } else if (want == 16 && G <= 16 && vw <= 24) {
      l = 16;
      v = vw <= 1 ? 1 : vw <= 2 ? 2 : vw <= 4 ? 4 : vw <= 8 ? 8 : vw <= 16 ? 16 : 24;
    } else if (want == 8 && G <= 8 && vw <= 16) {
      l = 8;
      v = vw <= 8 ? 8 : 16;
    } else if (want == 4 && G <= 4 && vw <= 8) {
      l = 4;
      v = vw <= 4 ? 4 : 8;
    }
  }
  *lpt = l;
  *vpl = v;
}

int select_hist_tokens(const RouteCfg& c) {
  int lpt, vpl;
  select_shape(c, &lpt, &vpl);
  if (lpt * vpl > kHistMaxE) return 0;
  return hist_waves(lpt) * (kWave / lpt);
}

hipError_t launch_select(const RouteCfg& c, const float* logits, int32_t splits,
                         int64_t split_stride, float* logits_out, const float* logit_bias,
                         const float* select_bias, const int32_t* k_per_token, int32_t* ids,
                         float* weights, int32_t* dev_err, int32_t* hist, hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  const int E = c.E;
  const bool grouped = c.n_groups > 1 && c.topk_groups < c.n_groups;
  const bool mono = select_bias == nullptr && !grouped;
  const int vec = E % 4 == 0 && aligned16(logits) && split_stride % 4 == 0 &&
                  (!logit_bias || aligned16(logit_bias)) &&
                  (!select_bias || aligned16(select_bias));
  int lpt, vpl;
  select_shape(c, &lpt, &vpl);
#define MOE_SEL(LPT_, VPL_)                                                                  \
  if (lpt == LPT_ && vpl == VPL_)                                                            \
    return launch_mono<LPT_, VPL_>(c, mono, logits, splits, split_stride, logits_out,        \
                                   logit_bias, select_bias, k_per_token, ids, weights, dev_err, \
                                   vec, hist, stream);
  MOE_SEL(16, 1)
  MOE_SEL(16, 2)
  MOE_SEL(16, 4)
  MOE_SEL(16, 8)
  MOE_SEL(4, 4)
  MOE_SEL(4, 8)
  MOE_SEL(8, 8)
  MOE_SEL(8, 16)
  MOE_SEL(16, 16)
  MOE_SEL(16, 24)
  MOE_SEL(64, 1)
  MOE_SEL(64, 2)
  MOE_SEL(64, 4)
  MOE_SEL(64, 8)
  MOE_SEL(64, 16)
#undef MOE_SEL
  return hipErrorInvalidValue;
}

}  // namespace moe
