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
//
// The per-token code lives in select_core.h and serves three kernels: the
// select kernel here (optionally also counting its picks into the
// dispatch's tile histograms), the gate kernel's fused epilogue, and the
// one-workgroup kernel below that also performs the whole dispatch of a
// small batch.
#include <cstdlib>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "select_core.h"

namespace moe {
namespace {

using sel::kMaxK;
using sel::load_vals;

// Requires n_groups <= LPT (one lane per group for the ranking).  The
// logits are the sum of NSPLIT partial arrays `split_stride` floats apart (a
// K split of the gate), added in a fixed order.  `vec`: the logits, their
// split stride and the bias arrays allow 16-byte loads (E % 4 == 0).
// HIST: also hist[block][e] = number of picks of expert e among the
// workgroup's TPB tokens -- the routes t*k + j of those tokens are one tile
// of the dispatch (counted with ballot peer masks, no atomics) -- and, with
// super_sum, the same counts added into super_sum[block / super_S][e]
// (integer atomics; the placement kernel then reads super rows instead of
// every tile's row).
template <int LPT, int VPL, int NSPLIT, bool MONO, int WPB, bool HIST>
__global__ __launch_bounds__(WPB * kWave) void select_kernel(
    RouteCfg c, const float* __restrict__ logits, int64_t split_stride,
    float* __restrict__ logits_out, const float* __restrict__ logit_bias,
    const float* __restrict__ select_bias, const int32_t* __restrict__ k_per_token,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ dev_err,
    int vec, hist_t* __restrict__ hist, int32_t* __restrict__ super_sum, int super_S) {
  constexpr int TPW = kWave / LPT;               // tokens per wavefront
  constexpr int TPB = WPB * TPW;                 // tokens per workgroup
  constexpr int ROW = LPT * VPL;                 // >= E
  constexpr int KPL = (kMaxK + LPT - 1) / LPT;   // output slots per lane
  __shared__ __attribute__((aligned(16))) float lrow[TPB][ROW];  // logits (+ logit_bias)
  __shared__ int32_t pick[TPB][kMaxK];                          // expert of each rank
  __shared__ int32_t whist[HIST ? WPB : 1][HIST ? ROW : 1];  // per-wave pick counts

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
  float sb[VPL];
  int kraw;
  {
    float pv[NSPLIT][VPL];
#pragma unroll
    for (int sp = 0; sp < NSPLIT; ++sp)
      load_vals<VPL>(logits + sp * split_stride + trow * E, e0, E, lvec, 0.f, pv[sp]);
    sel::load_sbias<VPL, MONO>(select_bias, e0, E, lvec, sb);
    kraw = k_per_token ? k_per_token[trow] : c.k;
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
  sel::select_token<LPT, VPL, MONO>(c, sl, seg, tok_ok, t, lv, nval, sb, kraw, lrow[tb],
                                    pick[tb], ids, weights, dev_err, pid);
  if constexpr (HIST) {
    for (int e = lane; e < E; e += kWave) whist[wave][e] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    sel::count_picks<LPT, sel::id_bits_for(ROW)>(pid, sl, c.k, whist[wave]);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += WPB * kWave) {
      int n = 0;
#pragma unroll
      for (int w8 = 0; w8 < WPB; ++w8) n += whist[w8][e];
      hist[(int64_t)blockIdx.x * E + e] = (hist_t)n;
      if (super_sum && n) atomicAdd(&super_sum[(int64_t)(blockIdx.x / super_S) * E + e], n);
    }
  }
}

// Routing and dispatch of a small batch in one workgroup (T * k <=
// kSmallRoutes routes, E <= kSmallE): the selection as in select_kernel,
// pass by pass over the tokens, each route's expert kept in LDS; then the
// dispatch of moe_dispatch in LDS -- per-chunk (64 routes) counts from
// ballot peer masks, per-expert exclusive scans over the chunks (one
// wavefront per expert), the scan over experts, and the stable placement
// (position = expert offset + earlier chunks + peers below in the chunk).
// One launch instead of three for decode-sized batches.
// Wavefronts per small workgroup: 16 where a lane's experts and the
// double-buffered logits of a pass (2 x NSPLIT x VPL registers) leave room
// under the 128 VGPRs of a 1024-lane workgroup -- one selection pass for 256
// 4-lane tokens (Mixtral-like: 10.3 -> 9.0 us) --, else 8 (8 experts per
// lane spill at 16 wavefronts).
constexpr int small_waves(int vpl, int nsplit) { return vpl <= 4 && vpl * nsplit <= 16 ? 16 : 8; }
constexpr int kSmallRoutes = 2048;
constexpr int kSmallE = 128;
constexpr int kSmallIdBits = 7;  // bits of an expert id below kSmallE

template <int LPT, int VPL, int NSPLIT, bool MONO>
__global__ __launch_bounds__(small_waves(VPL, NSPLIT) * kWave) void route_dispatch_small_kernel(
    RouteCfg c, const float* __restrict__ logits, int64_t split_stride,
    float* __restrict__ logits_out, const float* __restrict__ logit_bias,
    const float* __restrict__ select_bias, const int32_t* __restrict__ k_per_token,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ dev_err,
    int vec, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, double* __restrict__ maxvio) {
  constexpr int kSmallWaves = small_waves(VPL, NSPLIT);
  constexpr int TPW = kWave / LPT;               // tokens per wavefront and pass
  constexpr int TPP = kSmallWaves * TPW;         // tokens per pass
  constexpr int ROW = LPT * VPL;
  constexpr int KPL = (kMaxK + LPT - 1) / LPT;
  constexpr int NCH = kSmallRoutes / kWave;      // chunks of 64 routes, at most
  __shared__ __attribute__((aligned(16))) float lrow[TPP][ROW];
  __shared__ int32_t pick[TPP][kMaxK];
  __shared__ int32_t rid[kSmallRoutes];          // expert of each route, -1: none
  __shared__ int32_t cbase[NCH][kSmallE];        // per-chunk counts, then bases
  __shared__ int32_t off[kSmallE + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = lane / LPT, sl = lane % LPT;
  const int E = c.E, K = c.k;
  const int e0 = sl * VPL;
  const int nval = min(max(E - e0, 0), VPL);
  const bool lvec = vec && nval == VPL;
  const int T = c.T;

  // Pass by pass; the logits and per-token k of the next pass are loaded
  // while this one is selected (two register buffers, alternating passes).
  float sb[VPL], lb[VPL];
  sel::load_sbias<VPL, MONO>(select_bias, e0, E, lvec, sb);
  if (logit_bias) {
    load_vals<VPL>(logit_bias, e0, E, lvec, 0.f, lb);
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) lb[j] = 0.f;
  }
  float pv[2][NSPLIT][VPL];
  int kr[2];
  auto fetch = [&](int pass, auto bc) {
    constexpr int B = decltype(bc)::value;
    const int tw = pass * TPP + wave * TPW;
    const int64_t t = tw + seg;
    const int64_t trow = t < T ? t : (tw < T ? tw : T - 1);  // a row inside the batch
#pragma unroll
    for (int sp = 0; sp < NSPLIT; ++sp)
      load_vals<VPL>(logits + sp * split_stride + trow * E, e0, E, lvec, 0.f, pv[B][sp]);
    kr[B] = k_per_token ? k_per_token[trow] : K;
  };
  auto run = [&](int pass, auto bc) {
    constexpr int B = decltype(bc)::value;
    const int tw = pass * TPP + wave * TPW;
    if ((pass + 1) * TPP < T) fetch(pass + 1, std::integral_constant<int, 1 - B>());
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // lrow / pick rows reused
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int tb = wave * TPW + seg;
    const int64_t t = tw + seg;
    const bool tok_ok = t < T;
    float lv[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      lv[j] = pv[B][0][j];
#pragma unroll
      for (int sp = 1; sp < NSPLIT; ++sp) lv[j] += pv[B][sp][j];
    }
    if (NSPLIT > 1 && logits_out && tok_ok) {
#pragma unroll
      for (int j = 0; j < VPL; ++j)
        if (j < nval) logits_out[t * E + e0 + j] = lv[j];
    }
    if (logit_bias) {
#pragma unroll
      for (int j = 0; j < VPL; ++j) lv[j] += lb[j];
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (!tok_ok || j >= nval) lv[j] = -INFINITY;
#pragma unroll
    for (int j = 0; j < VPL; ++j) lrow[tb][e0 + j] = lv[j];
    int pid[KPL];
    sel::select_token<LPT, VPL, MONO>(c, sl, seg, tok_ok, t, lv, nval, sb, kr[B], lrow[tb],
                                      pick[tb], ids, weights, dev_err, pid);
    if (tok_ok) {
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const int r = sl + i * LPT;
        if (r < K) rid[t * K + r] = pid[i];
      }
    }
  };
  fetch(0, std::integral_constant<int, 0>());
  for (int pass = 0; pass * TPP + wave * TPW < T; pass += 2) {  // wave-uniform
    run(pass, std::integral_constant<int, 0>());
    if ((pass + 1) * TPP + wave * TPW >= T) break;
    run(pass + 1, std::integral_constant<int, 1>());
  }
  __syncthreads();

  // dispatch of the R routes held in rid
  const int R = T * K;
  const int nch = (R + kWave - 1) / kWave;
  for (int i = tid; i < nch * kSmallE; i += kSmallWaves * kWave) cbase[i / kSmallE][i % kSmallE] = 0;
  __syncthreads();
  const uint64_t below = lanemask_lt();
  for (int ch = wave; ch < nch; ch += kSmallWaves) {
    const int r = ch * kWave + lane;
    const int e = r < R ? rid[r] : -1;
    const uint64_t p = peer_mask<kSmallIdBits>(e);
    if (e >= 0 && (p & below) == 0) cbase[ch][e] = __popcll(p);  // one leader per expert
  }
  __syncthreads();
  // wavefront w: experts w, w + kSmallWaves, ...: exclusive scan over the chunks
  for (int e = wave; e < E; e += kSmallWaves) {
    const int v = lane < nch ? cbase[lane][e] : 0;
    const int inc = wave_incl_scan_i32(v);
    if (lane < nch) cbase[lane][e] = inc - v;
    if (lane == 63) off[e] = inc;  // the expert's total, for now
  }
  __syncthreads();
  if (wave == 0) {  // totals -> exclusive offsets over the experts (two per lane)
    const int a = 2 * lane < E ? off[2 * lane] : 0;
    const int b = 2 * lane + 1 < E ? off[2 * lane + 1] : 0;
    const int inc = wave_incl_scan_i32(a + b);
    __builtin_amdgcn_wave_barrier();
    if (2 * lane < E) {
      counts[2 * lane] = a;
      offsets[2 * lane] = off[2 * lane] = inc - a - b;
    }
    if (2 * lane + 1 < E) {
      counts[2 * lane + 1] = b;
      offsets[2 * lane + 1] = off[2 * lane + 1] = inc - b;
    }
    if (lane == 63) offsets[E] = off[E] = inc;
    if (maxvio) {  // MaxVio = max_e count_e / (R / E) - 1, 0 without routes
      const int mx = (int)wave_max_u32((uint32_t)max(a, b));
      if (lane == 63) *maxvio = inc > 0 ? (double)mx / ((double)inc / (double)E) - 1.0 : 0.0;
    }
  }
  __syncthreads();
  for (int ch = wave; ch < nch; ch += kSmallWaves) {
    const int r = ch * kWave + lane;
    const int e = r < R ? rid[r] : -1;
    const uint64_t p = peer_mask<kSmallIdBits>(e);
    const int pos = e >= 0 ? off[e] + cbase[ch][e] + __popcll(p & below) : -1;
    if (r < R) {
      if (inv) inv[r] = pos;
      if (pos >= 0) perm[pos] = r;
    }
  }
}

// Waves of a workgroup that also counts its picks for the dispatch: the
// fewer of 4 or 8 (16 for one-token wavefronts) whose tokens x k_stride
// routes make a dispatch tile the placement kernel takes (256-2048 routes,
// tiles x E within its count limit), or 0 -- Qwen3-like 4 (16 tokens x 16),
// OLMoE-like 8 (32 x 8; step 21.7 -> 18.6 us without the histogram
// kernel).  16 waves of multi-lane segments measured slower: DeepSeek-V3-
// like tiles of 64 tokens leave 128 workgroups for 256 CUs on a VALU-heavy
// selection (select 14 -> 19 us, more than the histogram kernel saves).
int hist_waves(const RouteCfg& c, int lpt) {
  const int ws[2] = {lpt == kWave ? 16 : 4, lpt == kWave ? 16 : 8};
  for (int w : ws) {
    const int tile = w * (kWave / lpt) * c.k;
    if (dispatch_hist_ok((int64_t)c.T * c.k, c.E, tile)) return w;
  }
  return 0;
}

// Waves of a workgroup that counts its picks into tile histograms and
// super-tile sums (the placement then reads about 2 sqrt(tiles) rows, so any
// tile size works): 8 when that still gives at least 256 workgroups (larger
// tiles, fewer placement workgroups), else 4; 16 for one-token wavefronts;
// tiles of at most 2048 routes.  MOE_SELECT_SUPER_WAVES (2, 4 or 8)
// overrides the choice for sweeps: 2-wave tiles (twice the placement
// workgroups) measured slower on every shape (Qwen3-like step 23.0 ->
// 25.8 us, DeepSeek-V4-like 119.4 -> 146.7 us).
int super_waves(const RouteCfg& c, int lpt) {
  const int tpw = kWave / lpt;
  if (lpt == kWave) return 16 * c.k <= 2048 ? 16 : 0;
  auto wgs = [&](int w) { return ((int64_t)c.T + w * tpw - 1) / (w * tpw); };
  if (const char* env = std::getenv("MOE_SELECT_SUPER_WAVES")) {
    const int w = std::atoi(env);
    if ((w == 2 || w == 4 || w == 8) && w * tpw * c.k <= 2048) return w;
  }
  if (wgs(8) >= 256 && 8 * tpw * c.k <= 2048) return 8;
  return 4 * tpw * c.k <= 2048 ? 4 : 0;
}

template <int LPT, int VPL, int NS, bool MONO>
hipError_t launch_vpl(const RouteCfg& c, const float* logits, int64_t stride, float* logits_out,
                      const float* logit_bias, const float* select_bias,
                      const int32_t* k_per_token, int32_t* ids, float* weights, int32_t* dev_err,
                      int vec, hist_t* hist, int32_t* super_sum, hipStream_t s) {
  constexpr int tpb = 4 * (kWave / LPT);
  const int64_t blocks = ((int64_t)c.T + tpb - 1) / tpb;
  if (hist) {  // one dispatch tile per workgroup
    const int hw = super_sum ? super_waves(c, LPT) : hist_waves(c, LPT);
    const int64_t R = (int64_t)c.T * c.k;
#define MOE_H(HW_)                                                                            \
  if (hw == HW_) {                                                                            \
    constexpr int htpb = HW_ * (kWave / LPT);                                                 \
    const int64_t hblocks = ((int64_t)c.T + htpb - 1) / htpb;                                 \
    const int S = super_sum ? dispatch_super_size(R, htpb * c.k) : 1;                         \
    return launch(kStageSelect, select_kernel<LPT, VPL, NS, MONO, HW_, true>,                 \
                  dim3((uint32_t)hblocks), dim3(HW_ * kWave), s, c, logits, stride,          \
                  logits_out, logit_bias, select_bias, k_per_token, ids, weights, dev_err,   \
                  vec, hist, super_sum, S);                                                   \
  }
    if constexpr (LPT == kWave) {
      MOE_H(16)
    } else {
      MOE_H(2)
      MOE_H(4)
      MOE_H(8)
    }
#undef MOE_H
    return hipErrorInvalidValue;
  }
  return launch(kStageSelect, select_kernel<LPT, VPL, NS, MONO, 4, false>, dim3((uint32_t)blocks),
                dim3(4 * kWave), s, c, logits, stride, logits_out, logit_bias, select_bias,
                k_per_token, ids, weights, dev_err, vec, (hist_t*)nullptr, (int32_t*)nullptr, 1);
}

template <int LPT, int VPL, bool MONO>
hipError_t launch_splits(const RouteCfg& c, const float* logits, int splits, int64_t stride,
                         float* logits_out, const float* logit_bias, const float* select_bias,
                         const int32_t* k_per_token, int32_t* ids, float* weights,
                         int32_t* dev_err, int vec, hist_t* hist, int32_t* super_sum,
                         hipStream_t s) {
#define MOE_S(S_)                                                                        \
  return launch_vpl<LPT, VPL, S_, MONO>(c, logits, stride, logits_out, logit_bias,       \
                                        select_bias, k_per_token, ids, weights, dev_err, \
                                        vec, hist, super_sum, s)
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
                       float* weights, int32_t* dev_err, int vec, hist_t* hist,
                       int32_t* super_sum, hipStream_t s) {
  if (mono)
    return launch_splits<LPT, VPL, true>(c, logits, splits, stride, logits_out, logit_bias,
                                         select_bias, k_per_token, ids, weights, dev_err, vec,
                                         hist, super_sum, s);
  return launch_splits<LPT, VPL, false>(c, logits, splits, stride, logits_out, logit_bias,
                                        select_bias, k_per_token, ids, weights, dev_err, vec,
                                        hist, super_sum, s);
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
  const bool grouped = c.n_groups > 1 && (c.topk_groups < c.n_groups || c.k_per_group > 0);
  const int G = grouped ? c.n_groups : 1;  // segments hold a lane per group
  const bool few = (int64_t)c.T * 8 < 2048 * kWave;  // 8-lane segments: T / 8 wavefronts
  // a batch small enough for one workgroup: the narrowest segment holding
  // at most 8 experts per lane (more tokens per wavefront, fewer passes)
  const bool tiny = (int64_t)c.T * c.k <= kSmallRoutes;
  int l = 64, v = 16;
  if (tiny && E <= 32 && G <= 4) {
    l = 4;
    v = E <= 4 ? 1 : E <= 8 ? 2 : E <= 16 ? 4 : 8;
  } else if (tiny && E <= 64 && G <= 8) {
    l = 8, v = 8;
  } else if (few && G <= 16 && E <= 128) {
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
  return hist_waves(c, lpt) * (kWave / lpt);
}

int select_super_tokens(const RouteCfg& c) {
  int lpt, vpl;
  select_shape(c, &lpt, &vpl);
  const int w = super_waves(c, lpt);
  if (w == 0 || !dispatch_super_ok((int64_t)c.T * c.k, c.E, w * (kWave / lpt) * c.k)) return 0;
  return w * (kWave / lpt);
}

bool small_dispatch_ok(const RouteCfg& c) {
  if ((int64_t)c.T * c.k > kSmallRoutes || c.E > kSmallE || c.T == 0) return false;
  int lpt, vpl;
  select_shape(c, &lpt, &vpl);
  return lpt <= 16 && vpl <= 8;
}

hipError_t launch_route_dispatch_small(const RouteCfg& c, const float* logits, int32_t splits,
                                       int64_t split_stride, float* logits_out,
                                       const float* logit_bias, const float* select_bias,
                                       const int32_t* k_per_token, int32_t* ids,
                                       float* weights, int32_t* dev_err, int32_t* counts,
                                       int32_t* offsets, int32_t* perm, int32_t* inv,
                                       double* maxvio, hipStream_t stream) {
  if (!small_dispatch_ok(c)) return hipErrorInvalidValue;
  const bool grouped = c.n_groups > 1 && c.topk_groups < c.n_groups;
  const bool mono = select_bias == nullptr && !grouped && c.k_per_group == 0;
  const int vec = c.E % 4 == 0 && aligned16(logits) && split_stride % 4 == 0 &&
                  (!logit_bias || aligned16(logit_bias)) &&
                  (!select_bias || aligned16(select_bias));
  int lpt, vpl;
  select_shape(c, &lpt, &vpl);
#define MOE_SD(L_, V_, S_, M_)                                                                \
  if (lpt == L_ && vpl == V_ && splits == S_ && mono == M_)                                   \
    return launch(kStageSelectDispatch, route_dispatch_small_kernel<L_, V_, S_, M_>, dim3(1),  \
                  dim3(small_waves(V_, S_) * kWave), stream, c, logits, split_stride,        \
                  logits_out,                                                                  \
                  logit_bias, select_bias, k_per_token, ids, weights, dev_err, vec, counts,  \
                  offsets, perm, inv, maxvio);
#define MOE_SDV(L_, V_)   \
  MOE_SD(L_, V_, 1, true) \
  MOE_SD(L_, V_, 1, false) \
  MOE_SD(L_, V_, 2, true) \
  MOE_SD(L_, V_, 2, false) \
  MOE_SD(L_, V_, 4, true) \
  MOE_SD(L_, V_, 4, false) \
  MOE_SD(L_, V_, 8, true) \
  MOE_SD(L_, V_, 8, false)
  MOE_SDV(4, 1)
  MOE_SDV(4, 2)
  MOE_SDV(4, 4)
  MOE_SDV(4, 8)
  MOE_SDV(8, 8)
  MOE_SDV(16, 1)
  MOE_SDV(16, 2)
  MOE_SDV(16, 4)
  MOE_SDV(16, 8)
#undef MOE_SDV
#undef MOE_SD
  return hipErrorInvalidValue;
}

hipError_t launch_select(const RouteCfg& c, const float* logits, int32_t splits,
                         int64_t split_stride, float* logits_out, const float* logit_bias,
                         const float* select_bias, const int32_t* k_per_token, int32_t* ids,
                         float* weights, int32_t* dev_err, hist_t* hist, int32_t* super_sum,
                         hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  const int E = c.E;
  const bool grouped = c.n_groups > 1 && c.topk_groups < c.n_groups;
  const bool mono = select_bias == nullptr && !grouped && c.k_per_group == 0;
  const int vec = E % 4 == 0 && aligned16(logits) && split_stride % 4 == 0 &&
                  (!logit_bias || aligned16(logit_bias)) &&
                  (!select_bias || aligned16(select_bias));
  int lpt, vpl;
  select_shape(c, &lpt, &vpl);
#define MOE_SEL(LPT_, VPL_)                                                                  \
  if (lpt == LPT_ && vpl == VPL_)                                                            \
    return launch_mono<LPT_, VPL_>(c, mono, logits, splits, split_stride, logits_out,        \
                                   logit_bias, select_bias, k_per_token, ids, weights, dev_err, \
                                   vec, hist, super_sum, stream);
  MOE_SEL(16, 1)
  MOE_SEL(16, 2)
  MOE_SEL(16, 4)
  MOE_SEL(16, 8)
  MOE_SEL(4, 1)
  MOE_SEL(4, 2)
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
