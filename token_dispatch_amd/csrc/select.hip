// Scoring, selection-only bias, group limit, top-k and weights on gfx950.
//
// One wavefront routes one token (sources: "DeepSeek-V3.2-Exp - Select
// experts": formula, "Explanation", gate-forward excerpt; ferrox_moe crate
// docs: route_top_k_softmax / _sigmoid(_with_bias) / _sqrtsoftplus /
// _softmax_weight; llama.cpp issue 13572 for a per-request k).
//
// Lane L holds experts [L*VPL, (L+1)*VPL) in registers.  Each expert carries
// a 32-bit order-preserving key of its selection quantity; a round of the
// top-k takes the wave maximum of the lanes' best keys and, among lanes that
// hold it, the lowest lane (a ballot), whose lowest slot wins -- so equal
// scores go to the lower expert id.  The winner clears its key and lane j
// keeps the j-th pick, so after k rounds lanes 0..k-1 hold the row's slots in
// order and write it with one coalesced store.
//
// When neither a selection bias nor a group limit is present, every score
// function is strictly increasing in the logit, so the kernel selects on the
// logit itself (the same choice without evaluating or saturating scores).
// Otherwise the key is q = score + bias in fp32.  Group scores (largest q, or
// sum of the two largest) come from a segmented butterfly when a group is a
// power-of-two run of whole lanes, else from a per-group wave reduction.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

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

template <int VPL>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void select_kernel(
    RouteCfg c, const float* __restrict__ logits,
    const float* __restrict__ logit_bias, const float* __restrict__ select_bias,
    const int32_t* __restrict__ k_per_token, int32_t* __restrict__ ids,
    float* __restrict__ weights, int32_t* __restrict__ dev_err) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= c.T) return;  // uniform per wave; no block-level sync below
  const int E = c.E;
  const int e0 = lane * VPL;

  float lv[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = e0 + j;
    lv[j] = (e < E) ? logits[t * E + e] + (logit_bias ? logit_bias[e] : 0.0f) : -INFINITY;
  }

  const bool grouped = c.n_groups > 1 && c.topk_groups < c.n_groups;
  const bool monotone = select_bias == nullptr && !grouped;
  const bool need_full_softmax =
      c.score == kSoftmax && (!monotone || !c.renormalize);

  // softmax over all experts (only when a probability itself is needed)
  float m_all = 0.f, inv_sum_all = 0.f;
  if (need_full_softmax) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < VPL; ++j) m = fmaxf(m, lv[j]);
    m_all = wave_max_f32(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) s += (e0 + j < E) ? expf(lv[j] - m_all) : 0.f;
    inv_sum_all = 1.0f / wave_sum_f32(s);
  }

  uint32_t key[VPL];
  if (monotone) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) key[j] = (e0 + j < E) ? ordered_key(lv[j]) : 0u;
  } else {
    float q[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = e0 + j;
      float s = (c.score == kSoftmax) ? expf(lv[j] - m_all) * inv_sum_all
                                      : elementwise_score(c.score, lv[j]);
      q[j] = (e < E) ? s + (select_bias ? select_bias[e] : 0.0f) : -INFINITY;
    }
    if (grouped) {
      const int G = c.n_groups;
      const int gs = E / G;
      const bool top2 = c.group_score == kGroupTop2Sum;
      const int lpg = gs / VPL;  // lanes per group on the fast path
      const bool fast = (gs % VPL == 0) && lpg >= 1 && lpg <= kWave && (lpg & (lpg - 1)) == 0;
      float my_g = -INFINITY;  // fast path: score of this lane's group
      float lane_g = -INFINITY;  // slow path: lane gamma holds g_gamma
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
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) p = top2_merge(p, shfl_xor_top2(p, off));
          if (lane == g) lane_g = top2 ? p.a + p.b : p.a;
        }
      }
      // group gamma's score, for gamma < G, on every lane
      auto group_score = [&](int g) -> float {
        return fast ? readlane_f32(my_g, g * lpg) : readlane_f32(lane_g, g);
      };
      // rank of each lane's own value g_me among the groups: (g desc, id asc)
      // Lane L ranks group L here; kept groups become a 64-bit mask.
      int rank = 0;
      // every lane shuffles (a shuffle from an inactive lane is undefined)
      const float g_fast = __shfl(my_g, (lane < G ? lane : 0) * (fast ? lpg : 0), kWave);
      const float g_me = fast ? g_fast : lane_g;
      for (int g = 0; g < G; ++g) {
        const float gg = group_score(g);
        rank += (gg > g_me) || (gg == g_me && g < lane);
      }
      const uint64_t kept = __ballot(lane < G && rank < c.topk_groups);
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int e = e0 + j;
        if (e < E && !((kept >> (e / gs)) & 1ull)) q[j] = -INFINITY;
      }
#pragma unroll
      for (int j = 0; j < VPL; ++j)
        key[j] = (e0 + j < E && q[j] != -INFINITY) ? ordered_key(q[j]) : 0u;
    } else {
#pragma unroll
      for (int j = 0; j < VPL; ++j) key[j] = (e0 + j < E) ? ordered_key(q[j]) : 0u;
    }
  }

  int kt = k_per_token ? k_per_token[t] : c.k;
  if (kt < 1 || kt > c.k) {
    if (lane == 0 && dev_err) atomicAdd(dev_err, 1);
    kt = 0;
  }

  int my_id = -1;
  float my_l = 0.f;
  for (int r = 0; r < kt; ++r) {
    uint32_t head = key[0];
    int hs = 0;
#pragma unroll
    for (int j = 1; j < VPL; ++j)
      if (key[j] > head) {
        head = key[j];
        hs = j;
      }
    const uint32_t gmax = wave_max_u32(head);
    const uint64_t cand = __ballot(head == gmax);
    const int wl = __ffsll((unsigned long long)cand) - 1;
    const bool win = lane == wl;
    float lh = lv[0];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      if (j == hs) lh = lv[j];
      if (win && j == hs) key[j] = 0u;
    }
    const int sel_slot = readlane_i32(hs, wl);
    const float sel_l = readlane_f32(lh, wl);
    if (lane == r) {
      my_id = wl * VPL + sel_slot;
      my_l = sel_l;
    }
  }

  const bool sel = lane < kt;
  float w = 0.f;
  if (c.score == kSoftmax || c.score == kSoftmaxTopk) {
    if (need_full_softmax && c.score == kSoftmax) {
      w = sel ? expf(my_l - m_all) * inv_sum_all : 0.f;
      if (c.renormalize) {
        const float tot = wave_sum_f32(w);
        w = sel ? w / tot : 0.f;
      }
    } else {
      // softmax restricted to the selected logits; equals the renormalised
      // full softmax because the full denominator cancels
      const float m_sel = wave_max_f32(sel ? my_l : -INFINITY);
      const float ex = sel ? expf(my_l - m_sel) : 0.f;
      const float tot = wave_sum_f32(ex);
      w = sel ? ex / tot : 0.f;
    }
  } else {
    w = sel ? elementwise_score(c.score, my_l) : 0.f;
    if (c.renormalize) {
      const float tot = wave_sum_f32(w);
      w = sel ? w / tot : 0.f;
    }
  }
  w *= c.route_scale;
  if (lane < c.k) {
    ids[t * c.k + lane] = sel ? my_id : -1;
    weights[t * c.k + lane] = sel ? w : 0.f;
  }
}

template <int VPL>
hipError_t launch_vpl(const RouteCfg& c, const float* logits, const float* logit_bias,
                      const float* select_bias, const int32_t* k_per_token,
                      int32_t* ids, float* weights, int32_t* dev_err, hipStream_t s) {
  const int64_t blocks = ((int64_t)c.T + kWavesPerBlock - 1) / kWavesPerBlock;
  prof_begin(kStageSelect, s);
  hipLaunchKernelGGL(select_kernel<VPL>, dim3((uint32_t)blocks), dim3(kWavesPerBlock * kWave),
                     0, s, c, logits, logit_bias, select_bias, k_per_token, ids, weights,
                     dev_err);
  prof_end(kStageSelect, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const RouteCfg& c, const float* logits,
                         const float* logit_bias, const float* select_bias,
                         const int32_t* k_per_token, int32_t* ids,
                         float* weights, int32_t* dev_err, hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  const int E = c.E;
  if (E <= 64) return launch_vpl<1>(c, logits, logit_bias, select_bias, k_per_token, ids, weights, dev_err, stream);
  if (E <= 128) return launch_vpl<2>(c, logits, logit_bias, select_bias, k_per_token, ids, weights, dev_err, stream);
  if (E <= 256) return launch_vpl<4>(c, logits, logit_bias, select_bias, k_per_token, ids, weights, dev_err, stream);
  if (E <= 384) return launch_vpl<6>(c, logits, logit_bias, select_bias, k_per_token, ids, weights, dev_err, stream);
  if (E <= 512) return launch_vpl<8>(c, logits, logit_bias, select_bias, k_per_token, ids, weights, dev_err, stream);
  return launch_vpl<16>(c, logits, logit_bias, select_bias, k_per_token, ids, weights, dev_err, stream);
}

}  // namespace moe
