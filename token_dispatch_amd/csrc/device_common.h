// Device helpers for the gfx950 routing kernels: wave64 reductions, ordered
// keys and score functions.  Internal to the HIP library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// Score function ids (same values as MOE_SCORE_* / MOE_GROUP_* in the ABI).
enum : int32_t { kSoftmax = 0, kSigmoid = 1, kSqrtSoftplus = 2, kSoftmaxTopk = 3 };
enum : int32_t { kGroupMax = 0, kGroupTop2Sum = 1 };

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Order-preserving map float -> uint32: a < b (as floats, no NaN) iff
// key(a) < key(b) (as unsigned).  Key 0 is below every float, -inf included,
// and marks an empty / removed candidate.
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, kWave);
    v = v > o ? v : o;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ int readlane_i32(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Lanes below this one, as a 64-bit mask.
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Mask of the lanes whose id (0 <= id < 2^NB) equals this lane's id,
// without atomics: one ballot per bit of the id narrows the set (meaningless
// for a lane whose id is < 0; callers test that).  A fixed bit count keeps
// the code straight-line: bits above an id's width are 0 in every valid id
// and leave the mask unchanged.
template <int NB>
__device__ __forceinline__ uint64_t peer_mask(int e) {
  uint64_t p = __ballot(e >= 0);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(bit);
    p &= bit ? m : ~m;
  }
  return p;
}

// Score functions from the hardware base-2 exponential and logarithm,
// reciprocal and square root (v_exp_f32, v_log_f32, v_rcp_f32, v_sqrt_f32,
// about 1 ulp each) -- a selection bias or a group limit needs the score of
// every expert of a token, and the library forms cost several times more:
//   exp(x)      = 2^(x log2 e)  (the product adds about |x| 2^-24 relative)
//   sigmoid(x)  = 1 / (1 + exp(-x))
//   softplus(x) = max(x, 0) + log(1 + e),  e = exp(-|x|) in (0, 1]:
//                 log(1 + e) = log2(1 + e) ln 2, or below e = 2^-7 the series
//                 e - e^2/2 + e^3/3 (next term < 2^-30), where the rounding
//                 of 1 + e would cost too much of the small result.
// The error, a few 1e-7 relative, is far below the 1e-4 bar of scores and
// weights.
__device__ __forceinline__ float exp_fast(float x) {
  return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}

__device__ __forceinline__ float sigmoid_f32(float l) {
  return __builtin_amdgcn_rcpf(1.0f + exp_fast(-l));
}

__device__ __forceinline__ float softplus_f32(float l) {
  const float e = exp_fast(-fabsf(l));
  const float lp = e < 0.0078125f ? e * (1.0f - e * (0.5f - e * (1.0f / 3.0f)))
                                  : __builtin_amdgcn_logf(1.0f + e) * 0.693147180559945309f;
  return fmaxf(l, 0.0f) + lp;
}

// Per-expert score for the element-wise score functions.  SOFTMAX needs the
// whole row and is handled by the callers.
__device__ __forceinline__ float elementwise_score(int32_t score, float l) {
  switch (score) {
    case kSigmoid: return sigmoid_f32(l);
    case kSqrtSoftplus: return __builtin_amdgcn_sqrtf(softplus_f32(l));
    default: return l;
  }
}

}  // namespace moe
