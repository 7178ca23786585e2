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

namespace moe {
namespace {

constexpr int kMaxK = 32;  // MOE_MAX_K
constexpr int kHistMaxE = 256;  // experts of the per-block histogram option

// ---- DPP helpers ------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Partner lanes: quad_perm [1,0,3,2] and [2,3,0,1] pair lanes within a quad;
// row_half_mirror pairs the two quads of 8 lanes, row_mirror the two halves
// of a 16-lane row.  After the steps up to width W every lane of an aligned
// W-lane group holds the group's reduction (bitwise the same in every lane:
// each step combines two equal-width partial results, a+b == b+a).
constexpr int kQuad1 = 0xB1, kQuad2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

template <int W>
__device__ __forceinline__ uint32_t grp_max_u32(uint32_t v) {
  uint32_t o = dpp_u32<kQuad1>(v);
  v = v > o ? v : o;
  o = dpp_u32<kQuad2>(v);
  v = v > o ? v : o;
  if constexpr (W >= 8) {
    o = dpp_u32<kHalfMirror>(v);
    v = v > o ? v : o;
  }
  if constexpr (W >= 16) {
    o = dpp_u32<kMirror>(v);
    v = v > o ? v : o;
  }
  return v;
}
template <int W>
__device__ __forceinline__ float grp_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kQuad1>(v));
  v = fmaxf(v, dpp_f32<kQuad2>(v));
  if constexpr (W >= 8) v = fmaxf(v, dpp_f32<kHalfMirror>(v));
  if constexpr (W >= 16) v = fmaxf(v, dpp_f32<kMirror>(v));
  return v;
}
template <int W>
__device__ __forceinline__ float grp_sum_f32(float v) {
  v += dpp_f32<kQuad1>(v);
  v += dpp_f32<kQuad2>(v);
  if constexpr (W >= 8) v += dpp_f32<kHalfMirror>(v);
  if constexpr (W >= 16) v += dpp_f32<kMirror>(v);
  return v;
}

// Segment-wide operations for LPT = 4, 8, 16 (within a DPP row) and 64
// (rows, then the four row results through scalar registers).
template <int LPT>
struct Seg {
  __device__ static uint32_t max_u32(uint32_t v) { return grp_max_u32<LPT>(v); }
  __device__ static float max_f32(float v) { return grp_max_f32<LPT>(v); }
  __device__ static float sum_f32(float v) { return grp_sum_f32<LPT>(v); }
  // lowest lane of this segment whose bit is set in `b`, or -1
  __device__ static int first(uint64_t b, int seg) {
    const uint32_t bits = (uint32_t)(b >> (seg * LPT)) & ((1u << LPT) - 1u);
    return bits ? __builtin_ctz(bits) : -1;
  }
  // value of segment lane i (every lane must take part)
  __device__ static float bcast_f32(float v, int seg, int i) {
    return __shfl(v, seg * LPT + i, kWave);
  }
};

template <>
struct Seg<64> {
  __device__ static uint32_t max_u32(uint32_t v) {
    v = grp_max_u32<16>(v);
    uint32_t a = (uint32_t)readlane_i32((int)v, 0), b = (uint32_t)readlane_i32((int)v, 16);
    uint32_t c = (uint32_t)readlane_i32((int)v, 32), d = (uint32_t)readlane_i32((int)v, 48);
    a = a > b ? a : b;
    c = c > d ? c : d;
    return a > c ? a : c;
  }
  __device__ static float max_f32(float v) {
    v = grp_max_f32<16>(v);
    return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
                 fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
  }
  __device__ static float sum_f32(float v) {
    v = grp_sum_f32<16>(v);
    return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
  }
  __device__ static int first(uint64_t b, int) { return b ? __builtin_ctzll(b) : -1; }
  __device__ static float bcast_f32(float v, int, int i) { return readlane_f32(v, i); }
};

// (first, second) largest of a set, combined pairwise.
struct Top2 {
  float a, b;  // a >= b
};
__device__ __forceinline__ Top2 top2_merge(Top2 x, Top2 y) {
  Top2 r;
  if (x.a >= y.a) {
    r.a = x.a;
    r.b = fmaxf(x.b, y.a);
  } else {
    r.a = y.a;
    r.b = fmaxf(y.b, x.a);
  }
  return r;
}
__device__ __forceinline__ Top2 top2_push(Top2 x, float v) {
  if (v > x.a) {
    x.b = x.a;
    x.a = v;
  } else if (v > x.b) {
    x.b = v;
  }
  return x;
}
__device__ __forceinline__ Top2 shfl_xor_top2(Top2 x, int off) {
  Top2 r;
  r.a = __shfl_xor(x.a, off, kWave);
  r.b = __shfl_xor(x.b, off, kWave);
  return r;
}

// row[e0 .. e0 + VPL) of a row of E floats (entries past E read as `fill`):
// 16-byte loads when `vec` (row + e0 16-byte aligned and e0 + VPL <= E),
// else scalar loads of row[min(e0 + j, E - 1)], never past the row; every
// load is issued before any value is used.
template <int VPL>
__device__ __forceinline__ void load_vals(const float* __restrict__ row, int e0, int E, bool vec,
                                          float fill, float (&v)[VPL]) {
  if constexpr (VPL % 4 == 0) {
    if (vec) {
      typedef float f32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int q = 0; q < VPL / 4; ++q) {
        const f32x4 x = reinterpret_cast<const f32x4*>(row + e0)[q];
        v[4 * q] = x[0];
        v[4 * q + 1] = x[1];
        v[4 * q + 2] = x[2];
        v[4 * q + 3] = x[3];
      }
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < VPL; ++j) v[j] = row[min(e0 + j, E - 1)];
#pragma unroll
  for (int j = 0; j < VPL; ++j)
    if (e0 + j >= E) v[j] = fill;
}

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
  using S = Seg<LPT>;
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
  const int E = c.E, K = c.k;
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

  const bool need_full_softmax = c.score == kSoftmax && (!MONO || !c.renormalize);

  // softmax over all experts (only when a probability itself is needed)
  float m_all = 0.f, inv_sum_all = 0.f;
  if (need_full_softmax) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < VPL; ++j) m = fmaxf(m, lv[j]);
    m_all = S::max_f32(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) s += (j < nval) ? expf(lv[j] - m_all) : 0.f;
    inv_sum_all = 1.0f / S::sum_f32(s);
  }

  uint32_t key[VPL];
  if constexpr (MONO) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) key[j] = (j < nval) ? ordered_key(lv[j]) : 0u;
  } else {
    float q[VPL], b[VPL];
    if (select_bias) {
      load_vals<VPL>(select_bias, e0, E, lvec, 0.f, b);
    } else {
#pragma unroll
      for (int j = 0; j < VPL; ++j) b[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const float s = (c.score == kSoftmax) ? expf(lv[j] - m_all) * inv_sum_all
                                            : elementwise_score(c.score, lv[j]);
      q[j] = (j < nval) ? s + b[j] : -INFINITY;
    }
    const bool grouped = c.n_groups > 1 && c.topk_groups < c.n_groups;
    if (grouped) {
      const int G = c.n_groups;
      const int gs = E / G;
      const bool top2 = c.group_score == kGroupTop2Sum;
      const int lpg = gs / VPL;  // lanes per group on the fast path
      const bool fast = (gs % VPL == 0) && lpg >= 1 && lpg <= LPT && (lpg & (lpg - 1)) == 0;
      float my_g = -INFINITY;    // fast path: score of this lane's group
      float lane_g = -INFINITY;  // slow path: segment lane gamma holds g_gamma
      if (fast) {
        Top2 p = {-INFINITY, -INFINITY};
#pragma unroll
        for (int j = 0; j < VPL; ++j) p = top2_push(p, q[j]);
        for (int off = 1; off < lpg; off <<= 1) p = top2_merge(p, shfl_xor_top2(p, off));
        my_g = top2 ? p.a + p.b : p.a;
      } else {
        for (int g = 0; g < G; ++g) {
          Top2 p = {-INFINITY, -INFINITY};
#pragma unroll
          for (int j = 0; j < VPL; ++j)
            if (j < nval && (e0 + j) / gs == g) p = top2_push(p, q[j]);
          for (int off = LPT / 2; off >= 1; off >>= 1) p = top2_merge(p, shfl_xor_top2(p, off));
          if (sl == g) lane_g = top2 ? p.a + p.b : p.a;
        }
      }
      // rank of group `sl` (for sl < G) by (g desc, group id asc); every lane
      // takes part in the shuffles (a shuffle from an inactive lane is undefined)
      const float g_fast = __shfl(my_g, seg * LPT + (fast && sl < G ? sl * lpg : 0), kWave);
      const float g_me = fast ? g_fast : lane_g;
      int rank = 0;
      for (int g = 0; g < G; ++g) {
        const float gg = fast ? S::bcast_f32(my_g, seg, g * lpg) : S::bcast_f32(lane_g, seg, g);
        rank += (gg > g_me) || (gg == g_me && g < sl);
      }
      const uint64_t kept_all = __ballot(sl < G && rank < c.topk_groups);
      const uint64_t kept = (LPT == 64) ? kept_all
                                        : ((kept_all >> (seg * LPT)) & ((1ull << LPT) - 1ull));
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int e = e0 + j;
        key[j] = (j < nval && ((kept >> (e / gs)) & 1ull)) ? ordered_key(q[j]) : 0u;
      }
    } else {
#pragma unroll
      for (int j = 0; j < VPL; ++j) key[j] = (j < nval) ? ordered_key(q[j]) : 0u;
    }
  }

  int kt = k_per_token ? k_per_token[trow] : K;
  if (!tok_ok) kt = 0;
  if (tok_ok && (kt < 1 || kt > K)) {
    if (sl == 0 && dev_err) atomicAdd(dev_err, 1);
    kt = 0;
  }
  // rounds: the largest k_t of the wavefront (every lane runs them)
  int k_rounds = kt;
  if constexpr (LPT < 64) {
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1)
      k_rounds = max(k_rounds, __shfl_xor(k_rounds, off, kWave));
  }

  for (int r = 0; r < k_rounds; ++r) {
    uint32_t head = key[0];
    int hs = 0;
#pragma unroll
    for (int j = 1; j < VPL; ++j)
      if (key[j] > head) {
        head = key[j];
        hs = j;
      }
    const uint32_t smax = S::max_u32(head);
    const int win = S::first(__ballot(head == smax && r < kt), seg);
    if (sl == win) {
#pragma unroll
      for (int j = 0; j < VPL; ++j)
        if (j == hs) key[j] = 0u;
      pick[tb][r] = e0 + hs;
    }
  }
  // the picks and the logit row were written by lanes of this wavefront
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // weights of the picks this lane writes: ranks sl, sl + LPT, ...
  int pid[KPL];
  float pl[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int r = sl + i * LPT;
    pid[i] = r < kt ? pick[tb][r] : -1;
    pl[i] = pid[i] >= 0 ? lrow[tb][pid[i]] : -INFINITY;
  }
  float w[KPL];
  if (c.score == kSoftmax && need_full_softmax) {
#pragma unroll
    for (int i = 0; i < KPL; ++i) w[i] = pid[i] >= 0 ? expf(pl[i] - m_all) * inv_sum_all : 0.f;
  } else if (c.score == kSoftmax || c.score == kSoftmaxTopk) {
    // softmax restricted to the picked logits; for SOFTMAX it equals the
    // renormalised full softmax because the full denominator cancels
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < KPL; ++i) m = fmaxf(m, pl[i]);
    const float m_sel = S::max_f32(m);
#pragma unroll
    for (int i = 0; i < KPL; ++i) w[i] = pid[i] >= 0 ? expf(pl[i] - m_sel) : 0.f;
  } else {
#pragma unroll
    for (int i = 0; i < KPL; ++i) w[i] = pid[i] >= 0 ? elementwise_score(c.score, pl[i]) : 0.f;
  }
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < KPL; ++i) part += w[i];
  const bool normalize = c.score == kSoftmaxTopk ||
                         (c.score == kSoftmax && !need_full_softmax) || c.renormalize;
  const float total = S::sum_f32(part);
  const float scale = normalize ? c.route_scale / total : c.route_scale;
  if (tok_ok) {
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int r = sl + i * LPT;
      if (r < K) {
        ids[t * K + r] = pid[i];
        weights[t * K + r] = pid[i] >= 0 ? w[i] * scale : 0.f;
      }
    }
  }
  if constexpr (HIST) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    for (int e = lane; e < E; e += kWave) whist[wave][e] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint64_t below = lanemask_lt();
#pragma unroll
    for (int i = 0; i < KPL; ++i) {  // chunk i: every lane's i-th pick
      const int e = (sl + i * LPT < K) ? pid[i] : -1;
      const uint64_t p = peer_mask(e, nbits);
      if (e >= 0 && (p & below) == 0) whist[wave][e] += __popcll(p);
    }
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

}  // namespace

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
