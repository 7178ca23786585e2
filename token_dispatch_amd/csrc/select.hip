// Scoring, selection-only bias, group limit, top-k and weights on gfx950.
//
// Sources: "DeepSeek-V3.2-Exp - Select experts" (formula, "Explanation",
// gate-forward excerpt); ferrox_moe crate docs (route_top_k_softmax,
// _sigmoid(_with_bias), _sqrtsoftplus, _softmax_weight); llama.cpp issue
// 13572 (a per-request k over the same scores).
//
// A segment of LPT lanes routes one token: 16 lanes (4 tokens per wavefront)
// when E <= 128, else the whole 64-lane wavefront.  Lane i of a segment
// holds experts [i*VPL, (i+1)*VPL) in registers.  Every expert carries a
// 32-bit order-preserving key of its selection quantity.  One round of the
// top-k: each lane takes its best key (lowest slot on equal keys), the
// segment maximum comes from DPP row rotations (VALU, no LDS), and among the
// lanes holding it the lowest lane wins (one ballot) -- so equal scores go to
// the lower expert id.  The winner records the round number as that slot's
// rank and clears the key.  After k_t rounds each lane turns its picked slots
// into weights and writes them straight to ids[t][rank] / weights[t][rank].
//
// With no selection bias and no group limit every score function is strictly
// increasing in the logit, so the keys are the logits themselves (the same
// choice, without evaluating or saturating scores).  Otherwise the key is
// q = score + bias in fp32.  Group scores (largest q, or sum of the two
// largest) come from a butterfly over the group's lanes when a group is a
// power-of-two run of whole lanes, else from one segment reduction per group.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

// ---- DPP helpers ------------------------------------------------------------
// row_ror:n rotates values right by n lanes inside each row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kRor8 = 0x128, kRor4 = 0x124, kRor2 = 0x122, kRor1 = 0x121;

__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  uint32_t o;
  o = dpp_u32<kRor8>(v);
  v = v > o ? v : o;
  o = dpp_u32<kRor4>(v);
  v = v > o ? v : o;
  o = dpp_u32<kRor2>(v);
  v = v > o ? v : o;
  o = dpp_u32<kRor1>(v);
  v = v > o ? v : o;
  return v;
}
__device__ __forceinline__ float row_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kRor8>(v));
  v = fmaxf(v, dpp_f32<kRor4>(v));
  v = fmaxf(v, dpp_f32<kRor2>(v));
  v = fmaxf(v, dpp_f32<kRor1>(v));
  return v;
}
__device__ __forceinline__ float row_sum_f32(float v) {
  v += dpp_f32<kRor8>(v);
  v += dpp_f32<kRor4>(v);
  v += dpp_f32<kRor2>(v);
  v += dpp_f32<kRor1>(v);
  return v;
}

// Segment-wide reductions for LPT = 16 (rows) and LPT = 64 (rows, then the
// four row results through scalar registers).
template <int LPT>
struct Seg;

template <>
struct Seg<16> {
  __device__ static uint32_t max_u32(uint32_t v) { return row_max_u32(v); }
  __device__ static float max_f32(float v) { return row_max_f32(v); }
  __device__ static float sum_f32(float v) { return row_sum_f32(v); }
  // lowest lane of this segment whose bit is set in `b`, or -1
  __device__ static int first(uint64_t b, int seg) {
    const uint32_t bits = (uint32_t)(b >> (seg * 16)) & 0xFFFFu;
    return bits ? __builtin_ctz(bits) : -1;
  }
  // value of segment lane i (every lane must take part)
  __device__ static float bcast_f32(float v, int seg, int i) {
    return __shfl(v, seg * 16 + i, kWave);
  }
};

template <>
struct Seg<64> {
  __device__ static uint32_t max_u32(uint32_t v) {
    v = row_max_u32(v);
    uint32_t a = (uint32_t)readlane_i32((int)v, 0), b = (uint32_t)readlane_i32((int)v, 16);
    uint32_t c = (uint32_t)readlane_i32((int)v, 32), d = (uint32_t)readlane_i32((int)v, 48);
    a = a > b ? a : b;
    c = c > d ? c : d;
    return a > c ? a : c;
  }
  __device__ static float max_f32(float v) {
    v = row_max_f32(v);
    return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
                 fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
  }
  __device__ static float sum_f32(float v) {
    v = row_sum_f32(v);
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

// Requires n_groups <= LPT (one lane per group for the ranking).  The
// logits are the sum of NSPLIT partial arrays `split_stride` floats apart (a K
// split of the gate), added in a fixed order.
template <int LPT, int VPL, int NSPLIT>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void select_kernel(
    RouteCfg c, const float* __restrict__ logits, int64_t split_stride,
    float* __restrict__ logits_out, const float* __restrict__ logit_bias,
    const float* __restrict__ select_bias, const int32_t* __restrict__ k_per_token,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ dev_err) {
  using S = Seg<LPT>;
  constexpr int TPW = kWave / LPT;  // tokens per wavefront
  const int lane = threadIdx.x & 63;
  const int seg = lane / LPT;  // token slot in the wavefront
  const int sl = lane % LPT;   // lane inside the segment
  const int64_t t0 = ((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)) * TPW;
  if (t0 >= c.T) return;  // whole wavefront past the end; no block sync below
  const int64_t t = t0 + seg;
  const bool tok_ok = t < c.T;
  const int E = c.E, K = c.k;
  const int e0 = sl * VPL;

  // Unconditional loads from clamped addresses, masked afterwards: a load
  // under a per-slot condition would be waited on before the next one.
  const int64_t trow = tok_ok ? t : t0;
  float pv[NSPLIT][VPL];
#pragma unroll
  for (int sp = 0; sp < NSPLIT; ++sp)
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      pv[sp][j] = logits[sp * split_stride + trow * E + min(e0 + j, E - 1)];
  float lv[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    lv[j] = pv[0][j];
#pragma unroll
    for (int sp = 1; sp < NSPLIT; ++sp) lv[j] += pv[sp][j];
  }
  if (NSPLIT > 1 && logits_out && tok_ok) {
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (e0 + j < E) logits_out[t * E + e0 + j] = lv[j];
  }
  if (logit_bias) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) lv[j] += logit_bias[min(e0 + j, E - 1)];
  }
#pragma unroll
  for (int j = 0; j < VPL; ++j)
    if (!tok_ok || e0 + j >= E) lv[j] = -INFINITY;

  const bool grouped = c.n_groups > 1 && c.topk_groups < c.n_groups;
  const bool monotone = select_bias == nullptr && !grouped;
  const bool need_full_softmax = c.score == kSoftmax && (!monotone || !c.renormalize);

  // softmax over all experts (only when a probability itself is needed)
  float m_all = 0.f, inv_sum_all = 0.f;
  if (need_full_softmax) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < VPL; ++j) m = fmaxf(m, lv[j]);
    m_all = S::max_f32(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) s += (e0 + j < E) ? expf(lv[j] - m_all) : 0.f;
    inv_sum_all = 1.0f / S::sum_f32(s);
  }

  uint32_t key[VPL];
  if (monotone) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) key[j] = (e0 + j < E) ? ordered_key(lv[j]) : 0u;
  } else {
    float q[VPL], b[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) b[j] = select_bias ? select_bias[min(e0 + j, E - 1)] : 0.0f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const float s = (c.score == kSoftmax) ? expf(lv[j] - m_all) * inv_sum_all
                                            : elementwise_score(c.score, lv[j]);
      q[j] = (e0 + j < E) ? s + b[j] : -INFINITY;
    }
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
            if (e0 + j < E && (e0 + j) / gs == g) p = top2_push(p, q[j]);
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
      const uint64_t kept = (LPT == 64) ? kept_all : ((kept_all >> (seg * LPT)) & 0xFFFFull);
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int e = e0 + j;
        key[j] = (e < E && ((kept >> (e / gs)) & 1ull)) ? ordered_key(q[j]) : 0u;
      }
    } else {
#pragma unroll
      for (int j = 0; j < VPL; ++j) key[j] = (e0 + j < E) ? ordered_key(q[j]) : 0u;
    }
  }

  int kt = k_per_token ? k_per_token[trow] : K;
  if (!tok_ok) kt = 0;
  if (tok_ok && (kt < 1 || kt > K)) {
    if (sl == 0 && dev_err) atomicAdd(dev_err, 1);
    kt = 0;
  }
  int k_rounds = kt;
  if (LPT < 64)
    k_rounds = max(max(readlane_i32(kt, 0), readlane_i32(kt, 16)),
                   max(readlane_i32(kt, 32), readlane_i32(kt, 48)));

  int rank[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) rank[j] = -1;
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
        if (j == hs) {
          rank[j] = r;
          key[j] = 0u;
        }
    }
  }

  // weights of the picked slots
  float w[VPL];
  float part = 0.f;
  if (c.score == kSoftmax && need_full_softmax) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      w[j] = rank[j] >= 0 ? expf(lv[j] - m_all) * inv_sum_all : 0.f;
      part += w[j];
    }
  } else if (c.score == kSoftmax || c.score == kSoftmaxTopk) {
    // softmax restricted to the picked logits; for SOFTMAX it equals the
    // renormalised full softmax because the full denominator cancels
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (rank[j] >= 0) m = fmaxf(m, lv[j]);
    const float m_sel = S::max_f32(m);
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      w[j] = rank[j] >= 0 ? expf(lv[j] - m_sel) : 0.f;
      part += w[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      w[j] = rank[j] >= 0 ? elementwise_score(c.score, lv[j]) : 0.f;
      part += w[j];
    }
  }
  const bool normalize = c.score == kSoftmaxTopk ||
                         (c.score == kSoftmax && !need_full_softmax) || c.renormalize;
  const float total = S::sum_f32(part);
  const float scale = normalize ? c.route_scale / total : c.route_scale;
  if (tok_ok) {
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (rank[j] >= 0) {
        ids[t * K + rank[j]] = e0 + j;
        weights[t * K + rank[j]] = w[j] * scale;
      }
    for (int r = kt + sl; r < K; r += LPT) {  // unused slots
      ids[t * K + r] = -1;
      weights[t * K + r] = 0.f;
    }
  }
}

template <int LPT, int VPL, int S>
hipError_t launch_vpl(const RouteCfg& c, const float* logits, int64_t stride, float* logits_out,
                      const float* logit_bias, const float* select_bias,
                      const int32_t* k_per_token, int32_t* ids, float* weights, int32_t* dev_err,
                      hipStream_t s) {
  constexpr int tokens_per_block = kWavesPerBlock * (kWave / LPT);
  const int64_t blocks = ((int64_t)c.T + tokens_per_block - 1) / tokens_per_block;
  prof_begin(kStageSelect, s);
  hipLaunchKernelGGL((select_kernel<LPT, VPL, S>), dim3((uint32_t)blocks),
                     dim3(kWavesPerBlock * kWave), 0, s, c, logits, stride, logits_out,
                     logit_bias, select_bias, k_per_token, ids, weights, dev_err);
  prof_end(kStageSelect, s);
  return hipGetLastError();
}

template <int LPT, int VPL>
hipError_t launch_splits(const RouteCfg& c, const float* logits, int splits, int64_t stride,
                         float* logits_out, const float* logit_bias, const float* select_bias,
                         const int32_t* k_per_token, int32_t* ids, float* weights,
                         int32_t* dev_err, hipStream_t s) {
#define MOE_S(S_)                                                                              \
  return launch_vpl<LPT, VPL, S_>(c, logits, stride, logits_out, logit_bias, select_bias,      \
                                  k_per_token, ids, weights, dev_err, s)
  if constexpr (VPL <= 8) {
    if (splits == 2) MOE_S(2);
    if (splits == 4) MOE_S(4);
    if (splits == 8) MOE_S(8);
  }
  if (splits != 1) return hipErrorInvalidValue;
  MOE_S(1);
#undef MOE_S
}

}  // namespace

hipError_t launch_select(const RouteCfg& c, const float* logits, int32_t splits,
                         int64_t split_stride, float* logits_out, const float* logit_bias,
                         const float* select_bias, const int32_t* k_per_token, int32_t* ids,
                         float* weights, int32_t* dev_err, hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  const int E = c.E;
  const bool few_groups = c.n_groups <= 16 || c.topk_groups >= c.n_groups;
#define MOE_SEL(LPT_, VPL_)                                                                  \
  return launch_splits<LPT_, VPL_>(c, logits, splits, split_stride, logits_out, logit_bias, \
                                   select_bias, k_per_token, ids, weights, dev_err, stream)
  if (few_groups) {  // 16-lane segments rank at most 16 groups
    if (E <= 16) MOE_SEL(16, 1);
    if (E <= 32) MOE_SEL(16, 2);
    if (E <= 64) MOE_SEL(16, 4);
    if (E <= 128) MOE_SEL(16, 8);
  }
  if (E <= 64) MOE_SEL(64, 1);
  if (E <= 128) MOE_SEL(64, 2);
  if (E <= 256) MOE_SEL(64, 4);
  if (E <= 384) MOE_SEL(64, 6);
  if (E <= 512) MOE_SEL(64, 8);
  MOE_SEL(64, 16);
#undef MOE_SEL
}

}  // namespace moe
