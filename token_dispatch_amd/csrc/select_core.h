// Per-token selection shared by the select kernel and the gate kernel's
// fused epilogue (device code; included by both sources).  The method and
// its sources are described in select.hip.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace sel {

constexpr int kMaxK = 32;        // MOE_MAX_K

// Ballots per peer mask for expert ids below `row` (a row of LPT * VPL
// experts): the bits of the largest id.
constexpr int id_bits_for(int row) { return row <= 128 ? 7 : row <= 256 ? 8 : 10; }

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

// Selection bias of a lane's experts (zeros without one; not read when MONO).
template <int VPL, bool MONO>
__device__ __forceinline__ void load_sbias(const float* __restrict__ select_bias, int e0, int E,
                                           bool vec, float (&sb)[VPL]) {
  if (!MONO && select_bias) {
    load_vals<VPL>(select_bias, e0, E, vec, 0.f, sb);
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) sb[j] = 0.f;
  }
}

// One token's selection by a segment of LPT lanes of a wavefront.  Lane sl
// holds experts [e0, e0 + nval), e0 = sl * VPL, in lv: logits (+ logit
// bias), -inf past E and for a missing token (tok_ok false), and in sb their
// selection bias (zeros without one; unused when MONO).  kraw: the token's
// requested k (its per-token k, or k).  lrow: the token's row of lv in LDS
// (the picks' logits are read back from it); pick: kMaxK ints of LDS for the
// token.  Writes ids[t][*] and weights[t][*] and leaves in pid the experts
// this lane wrote (ranks sl, sl + LPT, ...; -1: none).  Every lane of the
// wavefront takes part.  KC > 0: k == KC, known when compiling -- the rounds
// are unrolled and the weights' slot loops fold (the fused gate + selection
// at k = 4: selection 11.4 -> 8.8 us of its 74-77 us); a token whose k_t is
// below KC gets no pick in its later rounds (r < k_t fails there).
template <int LPT, int VPL, bool MONO, int KC = 0>
__device__ __forceinline__ void select_token(
    const RouteCfg& c, int sl, int seg, bool tok_ok, int64_t t, const float (&lv)[VPL],
    int nval, const float (&sb)[VPL], int kraw, const float* lrow, int32_t* pick,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ dev_err,
    int (&pid)[(kMaxK + LPT - 1) / LPT]) {
  using S = Seg<LPT>;
  constexpr int KPL = (kMaxK + LPT - 1) / LPT;  // output slots per lane
  const int E = c.E, K = KC > 0 ? KC : c.k;
  const int e0 = sl * VPL;
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
    for (int j = 0; j < VPL; ++j) s += (j < nval) ? exp_fast(lv[j] - m_all) : 0.f;
    inv_sum_all = 1.0f / S::sum_f32(s);
  }

  uint32_t key[VPL];
  if constexpr (MONO) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) key[j] = (j < nval) ? ordered_key(lv[j]) : 0u;
  } else {
    // the score of every expert: one loop per score function (the
    // wave-uniform branch is taken once, not per expert)
    float q[VPL];
    switch (c.score) {
      case kSoftmax:
#pragma unroll
        for (int j = 0; j < VPL; ++j) q[j] = exp_fast(lv[j] - m_all) * inv_sum_all;
        break;
      case kSigmoid:
#pragma unroll
        for (int j = 0; j < VPL; ++j) q[j] = sigmoid_f32(lv[j]);
        break;
      case kSqrtSoftplus:
#pragma unroll
        for (int j = 0; j < VPL; ++j) q[j] = __builtin_amdgcn_sqrtf(softplus_f32(lv[j]));
        break;
      default:
#pragma unroll
        for (int j = 0; j < VPL; ++j) q[j] = lv[j];
        break;
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) q[j] = (j < nval) ? q[j] + sb[j] : -INFINITY;
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

  int kt = kraw;
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

  // grouped top-k with a quota of k_per_group picks per group (the rounds
  // take the largest key left, so a group's picks are its best; once a group
  // has its quota its other experts leave the race, which gives the top-k of
  // the groups' best).  Segment lane g (g < n_groups) counts group g's picks.
  const int kpg = c.k_per_group;
  const int gsz = kpg > 0 ? E / c.n_groups : 1;
  const int g_lo = sl * gsz;  // this lane's group: experts [g_lo, g_lo + gsz)
  int gcount = 0;

  // KC == 0: k_rounds rounds, the loop as it was compiled before the
  // compile-time case existed (unrolling or outlining it slowed the select
  // kernel); KC > 0: KC rounds, unrolled.
  constexpr int kUnroll = KC > 0 ? KC : 1;
  const int n_rounds = KC > 0 ? KC : k_rounds;
#pragma unroll kUnroll
  for (int r = 0; r < n_rounds; ++r) {
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
      pick[r] = e0 + hs;
    }
    if (kpg > 0) {  // uniform
      const int e_win = __shfl(e0 + hs, seg * LPT + max(win, 0), kWave);
      const bool mine = r < kt && sl < c.n_groups && e_win >= g_lo && e_win < g_lo + gsz;
      gcount += mine;
      const uint64_t filled = __ballot(mine && gcount == kpg);
      if (filled) {  // some segment's group reached its quota this round
        const int gl = S::first(filled, seg);
        if (gl >= 0) {
          const int lo = gl * gsz - e0, hi = lo + gsz;  // that group, in this lane's slots
#pragma unroll
          for (int j = 0; j < VPL; ++j)
            if (j >= lo && j < hi) key[j] = 0u;
        }
      }
    }
  }
  // the picks and the logit row were written by lanes of this wavefront
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // weights of the picks this lane writes: ranks sl, sl + LPT, ...; slots
  // whose ranks are all >= K are skipped (wave-uniform), they hold no pick
  const int nslots = (K + LPT - 1) / LPT;
  float pl[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int r = sl + i * LPT;
    pid[i] = (i < nslots && r < kt) ? pick[r] : -1;
    pl[i] = pid[i] >= 0 ? lrow[pid[i]] : -INFINITY;
  }
  float w[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) w[i] = 0.f;
  if (c.score == kSoftmax && need_full_softmax) {
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (i < nslots) w[i] = pid[i] >= 0 ? exp_fast(pl[i] - m_all) * inv_sum_all : 0.f;
  } else if (c.score == kSoftmax || c.score == kSoftmaxTopk) {
    // softmax restricted to the picked logits; for SOFTMAX it equals the
    // renormalised full softmax because the full denominator cancels
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < KPL; ++i) m = fmaxf(m, pl[i]);
    const float m_sel = S::max_f32(m);
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (i < nslots) w[i] = pid[i] >= 0 ? expf(pl[i] - m_sel) : 0.f;
  } else {
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (i < nslots) w[i] = pid[i] >= 0 ? elementwise_score(c.score, pl[i]) : 0.f;
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
}

// Adds a wavefront's picks (pid of each lane, ranks below K, ids < 2^NB) to whist_w[e]:
// ballot peer masks give one leader per expert and chunk, so no two lanes
// update one entry at once (no atomics).
template <int LPT, int NB>
__device__ __forceinline__ void count_picks(const int (&pid)[(kMaxK + LPT - 1) / LPT], int sl,
                                            int K, int32_t* whist_w) {
  constexpr int KPL = (kMaxK + LPT - 1) / LPT;
  const uint64_t below = lanemask_lt();
#pragma unroll
  for (int i = 0; i < KPL; ++i) {  // chunk i: every lane's i-th pick
    if (i * LPT >= K) break;      // wave-uniform: no rank below K in this chunk
    const int e = (sl + i * LPT < K) ? pid[i] : -1;
    const uint64_t p = peer_mask<NB>(e);
    if (e >= 0 && (p & below) == 0) whist_w[e] += __popcll(p);
  }
}

}  // namespace sel
}  // namespace moe
