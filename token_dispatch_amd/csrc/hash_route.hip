// Hash routing on gfx950 (ferrox_moe crate docs, route_hash: in a
// DeepSeek-V4 hash layer the expert ids are the token id's row of a fixed
// token-id -> expert-id table, with no learned selection and no selection
// bias).
//
// Lanes j < k of a token's segment gather the table row (validating the
// token id and every entry), then, when weights are wanted, lane j takes the
// logit of slot j and the segment turns the k logits into weights with the
// layer's score function.  The logits come either from the gate contraction
// of every expert (the tiled matrix-core kernel, into a workspace; NSPLIT
// K-split partial arrays added in order; several tokens per wavefront, and
// optionally the dispatch's tile histograms) -- the k dot products alone
// would re-read k rows of W from L2 for every token, about 64 times the
// gate's L2 traffic at E = 384, k = 6 -- or, with no workspace, from k dot
// products of length d computed here (one wavefront per token, the lanes
// striding over d with 16-byte loads).
#include "device_common.h"
#include "kernels.h"
#include "select_core.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

template <typename In>
__device__ __forceinline__ float to_f32(In v);
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }

// Partial dot product of x row and W row held by this lane.
template <typename In, bool VEC>
__device__ __forceinline__ float lane_dot(const In* __restrict__ xr, const In* __restrict__ wr,
                                          int d, int lane) {
  float acc = 0.f;
  if (VEC) {
    constexpr int P = 16 / sizeof(In);
    for (int i = lane * P; i < d; i += kWave * P) {
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(xr + i);
      const u32x4_t b = *reinterpret_cast<const u32x4_t*>(wr + i);
      if constexpr (sizeof(In) == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc = fmaf(bf16_lo(a[q]), bf16_lo(b[q]), acc);
          acc = fmaf(bf16_hi(a[q]), bf16_hi(b[q]), acc);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = fmaf(__uint_as_float(a[q]), __uint_as_float(b[q]), acc);
      }
    }
  } else {
    for (int i = lane; i < d; i += kWave) acc = fmaf(to_f32<In>(xr[i]), to_f32<In>(wr[i]), acc);
  }
  return acc;
}

// NSPLIT == 0: dot products from x and W (+ logit_bias); NSPLIT > 0: the
// logits (bias included) are the sum of NSPLIT arrays [T][E], split_stride
// floats apart.
template <typename In, bool VEC, int NSPLIT>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void hash_route_kernel(
    RouteCfg c, const int32_t* __restrict__ token_ids,
    const int32_t* __restrict__ tid2eid, int32_t vocab, const In* __restrict__ x,
    const In* __restrict__ W, const float* __restrict__ logit_bias,
    const float* __restrict__ logits, int64_t split_stride,
    int32_t* __restrict__ ids, float* __restrict__ weights,
    int32_t* __restrict__ dev_err) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= c.T) return;
  const int k = c.k;

  const int v = token_ids[t];
  const bool tok_ok = v >= 0 && v < vocab;
  int e = -1;
  bool bad_slot = false;
  if (lane < k && tok_ok) {
    e = tid2eid[(int64_t)v * k + lane];
    if (e < 0 || e >= c.E) {
      bad_slot = true;
      e = -1;
    }
  }
  const int nerr = tok_ok ? __popcll(__ballot(bad_slot)) : 1;
  if (lane == 0 && nerr && dev_err) atomicAdd(dev_err, nerr);
  if (lane < k) ids[t * k + lane] = e;
  if (weights == nullptr) return;

  float my_l = 0.f;
  if constexpr (NSPLIT > 0) {
    if (e >= 0) {
      float pv[NSPLIT];
#pragma unroll
      for (int sp = 0; sp < NSPLIT; ++sp) pv[sp] = logits[sp * split_stride + t * c.E + e];
      my_l = pv[0];
#pragma unroll
      for (int sp = 1; sp < NSPLIT; ++sp) my_l += pv[sp];
    }
  } else {
    const In* xr = x + t * (int64_t)c.d;
    for (int j = 0; j < k; ++j) {
      const int ej = readlane_i32(e, j);
      if (ej < 0) continue;
      float acc = wave_sum_f32(lane_dot<In, VEC>(xr, W + (int64_t)ej * c.d, c.d, lane));
      if (logit_bias) acc += logit_bias[ej];
      if (lane == j) my_l = acc;
    }
  }

  const bool sel = lane < k && e >= 0;
  float w;
  if (c.score == kSoftmax || c.score == kSoftmaxTopk) {
    const float m = wave_max_f32(sel ? my_l : -INFINITY);
    const float ex = sel ? expf(my_l - m) : 0.f;
    const float tot = wave_sum_f32(ex);
    w = sel ? ex / tot : 0.f;
  } else {
    w = sel ? elementwise_score(c.score, my_l) : 0.f;
    if (c.renormalize) {
      const float tot = wave_sum_f32(w);
      w = sel ? w / tot : 0.f;
    }
  }
  if (lane < k) weights[t * k + lane] = sel ? w * c.route_scale : 0.f;
}

// Hash routing from the gate's logits with several tokens per wavefront: a
// segment of SEG lanes (SEG = 4, 8, 16 or 64, the smallest >= k) routes one
// token, lane j < k taking slot j; WPB wavefronts per workgroup.  The
// token's k logits are gathered from the gate's NSPLIT partial arrays
// (added in order) and turned into weights with segment-wide DPP
// reductions.  HIST: the workgroup's tokens x k routes are one dispatch tile;
// their expert ids are counted with ballot peer masks into hist[block][E]
// and added into super_sum[block / super_S][E] (zeroed by the gate kernel
// of the same call) -- the dispatch then needs only its placement kernel.
template <int SEG, int NSPLIT, int WPB, bool HIST, int NB>
__global__ __launch_bounds__(WPB * kWave) void hash_route_tiles_kernel(
    RouteCfg c, const int32_t* __restrict__ token_ids, const int32_t* __restrict__ tid2eid,
    int32_t vocab, const float* __restrict__ logits, int64_t split_stride,
    int32_t* __restrict__ ids, float* __restrict__ weights, int32_t* __restrict__ dev_err,
    hist_t* __restrict__ hist, int32_t* __restrict__ super_sum, int super_S) {
  constexpr int TPW = kWave / SEG;
  using S = sel::Seg<SEG>;
  __shared__ int32_t whist[HIST ? WPB : 1][HIST ? 1024 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seg = lane / SEG, sl = lane % SEG;
  const int k = c.k, E = c.E;
  const int64_t t = ((int64_t)blockIdx.x * WPB + wave) * TPW + seg;
  const bool tok_in = t < c.T;
  const int v = tok_in ? token_ids[t] : 0;
  const bool tok_ok = tok_in && v >= 0 && v < vocab;
  int e = -1;
  bool bad_slot = false;
  if (sl < k && tok_ok) {
    e = tid2eid[(int64_t)v * k + sl];
    if (e < 0 || e >= E) {
      bad_slot = true;
      e = -1;
    }
  }
  float my_l = 0.f;
  if (e >= 0) {
    float pv[NSPLIT];
#pragma unroll
    for (int sp = 0; sp < NSPLIT; ++sp) pv[sp] = logits[sp * split_stride + t * E + e];
    my_l = pv[0];
#pragma unroll
    for (int sp = 1; sp < NSPLIT; ++sp) my_l += pv[sp];
  }
  // errors: bad table entries, and a bad token id once per token
  const int nerr = __popcll(__ballot(bad_slot)) + __popcll(__ballot(tok_in && !tok_ok && sl == 0));
  if (lane == 0 && nerr && dev_err) atomicAdd(dev_err, nerr);
  const bool valid = e >= 0;
  float w;
  if (c.score == kSoftmax || c.score == kSoftmaxTopk) {
    const float m = S::max_f32(valid ? my_l : -INFINITY);
    const float ex = valid ? expf(my_l - m) : 0.f;
    const float tot = S::sum_f32(ex);
    w = valid ? ex / tot : 0.f;
  } else {
    w = valid ? elementwise_score(c.score, my_l) : 0.f;
    if (c.renormalize) {
      const float tot = S::sum_f32(w);
      w = valid ? w / tot : 0.f;
    }
  }
  if (tok_in && sl < k) {
    ids[t * k + sl] = e;
    weights[t * k + sl] = valid ? w * c.route_scale : 0.f;
  }
  if constexpr (HIST) {
    for (int x = lane; x < E; x += kWave) whist[wave][x] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint64_t p = peer_mask<NB>(e);
    if (e >= 0 && (p & lanemask_lt()) == 0) whist[wave][e] += __popcll(p);
    __syncthreads();
    for (int x = threadIdx.x; x < E; x += WPB * kWave) {
      int n = 0;
#pragma unroll
      for (int w8 = 0; w8 < WPB; ++w8) n += whist[w8][x];
      hist[(int64_t)blockIdx.x * E + x] = (hist_t)n;
      if (super_sum && n) atomicAdd(&super_sum[(int64_t)(blockIdx.x / super_S) * E + x], n);
    }
  }
}

// Lanes per token of the multi-token hash kernel (k <= 32).
int hash_seg(int k) { return k <= 4 ? 4 : k <= 8 ? 8 : k <= 16 ? 16 : 64; }
constexpr int kHashTileWaves = 4;

template <int SEG, int NS, bool HIST>
hipError_t launch_tiles_nb(const RouteCfg& c, const int32_t* tok, const int32_t* tab,
                           int32_t vocab, const float* logits, int64_t stride, int32_t* ids,
                           float* w, int32_t* err, hist_t* hist, int32_t* super_sum, int S,
                           hipStream_t s) {
  constexpr int tpb = kHashTileWaves * (kWave / SEG);
  const dim3 grid((uint32_t)(((int64_t)c.T + tpb - 1) / tpb));
  const dim3 block(kHashTileWaves * kWave);
  auto go = [&](auto kernel) {
    return launch(kStageHash, kernel, grid, block, s, c, tok, tab, vocab, logits, stride, ids,
                  w, err, hist, super_sum, S);
  };
  if (c.E <= 128) return go(hash_route_tiles_kernel<SEG, NS, kHashTileWaves, HIST, 7>);
  if (c.E <= 256) return go(hash_route_tiles_kernel<SEG, NS, kHashTileWaves, HIST, 8>);
  return go(hash_route_tiles_kernel<SEG, NS, kHashTileWaves, HIST, 10>);
}

template <int SEG>
hipError_t launch_tiles_seg(const RouteCfg& c, const int32_t* tok, const int32_t* tab,
                            int32_t vocab, const float* logits, int32_t splits, int64_t stride,
                            int32_t* ids, float* w, int32_t* err, hist_t* hist,
                            int32_t* super_sum, int S, hipStream_t s) {
#define MOE_HT(NS_)                                                                           \
  if (splits == NS_)                                                                          \
    return hist ? launch_tiles_nb<SEG, NS_, true>(c, tok, tab, vocab, logits, stride, ids, w,  \
                                                  err, hist, super_sum, S, s)                 \
                : launch_tiles_nb<SEG, NS_, false>(c, tok, tab, vocab, logits, stride, ids, w, \
                                                   err, hist, super_sum, S, s);
  MOE_HT(1)
  MOE_HT(2)
  MOE_HT(4)
  MOE_HT(8)
#undef MOE_HT
  return hipErrorInvalidValue;
}

template <typename In>
hipError_t launch_typed(const RouteCfg& c, const int32_t* tok, const int32_t* tab, int32_t vocab,
                        const void* x, const void* W, const float* lb, const float* logits,
                        int32_t splits, int64_t split_stride, int32_t* ids, float* w,
                        int32_t* err, hipStream_t s) {
  const dim3 grid((uint32_t)(((int64_t)c.T + kWavesPerBlock - 1) / kWavesPerBlock));
  const dim3 block(kWavesPerBlock * kWave);
  const In* xi = (const In*)x;
  const In* Wi = (const In*)W;
  if (logits) {
#define MOE_H(S_)                                                                              \
  if (splits == S_)                                                                            \
    return launch(kStageHash, hash_route_kernel<In, false, S_>, grid, block, s, c, tok, tab,  \
                  vocab, xi, Wi, lb, logits, split_stride, ids, w, err);
    MOE_H(1)
    MOE_H(2)
    MOE_H(4)
    MOE_H(8)
#undef MOE_H
    return hipErrorInvalidValue;
  }
  const bool vec = x != nullptr && (c.d % (16 / sizeof(In)) == 0) &&
                   reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(W) % 16 == 0;
  if (vec)
    return launch(kStageHash, hash_route_kernel<In, true, 0>, grid, block, s, c, tok, tab, vocab,
                  xi, Wi, lb, (const float*)nullptr, (int64_t)0, ids, w, err);
  return launch(kStageHash, hash_route_kernel<In, false, 0>, grid, block, s, c, tok, tab, vocab,
                xi, Wi, lb, (const float*)nullptr, (int64_t)0, ids, w, err);
}

}  // namespace

hipError_t launch_hash_route(const RouteCfg& c, int32_t dtype,
                             const int32_t* token_ids, const int32_t* tid2eid,
                             int32_t vocab, const void* x, const void* W,
                             const float* logit_bias, const float* logits, int32_t splits,
                             int64_t split_stride, int32_t* ids, float* weights,
                             int32_t* dev_err, hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  if (dtype == 1)
    return launch_typed<uint16_t>(c, token_ids, tid2eid, vocab, x, W, logit_bias, logits, splits,
                                  split_stride, ids, weights, dev_err, stream);
  return launch_typed<float>(c, token_ids, tid2eid, vocab, x, W, logit_bias, logits, splits,
                             split_stride, ids, weights, dev_err, stream);
}

int hash_tile_tokens(int32_t k) { return kHashTileWaves * (kWave / hash_seg(k)); }

hipError_t launch_hash_tiles(const RouteCfg& c, const int32_t* token_ids,
                             const int32_t* tid2eid, int32_t vocab, const float* logits,
                             int32_t splits, int64_t split_stride, int32_t* ids, float* weights,
                             int32_t* dev_err, hist_t* hist, int32_t* super_sum,
                             hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  if (c.E > 1024 || c.k > 32) return hipErrorInvalidValue;
  int S = 1;
  if (hist) {
    const int64_t R = (int64_t)c.T * c.k;
    const int tr = hash_tile_tokens(c.k) * c.k;
    if (!dispatch_super_ok(R, c.E, tr)) return hipErrorInvalidValue;
    S = dispatch_super_size(R, tr);
  }
  switch (hash_seg(c.k)) {
    case 4: return launch_tiles_seg<4>(c, token_ids, tid2eid, vocab, logits, splits, split_stride,
                                       ids, weights, dev_err, hist, super_sum, S, stream);
    case 8: return launch_tiles_seg<8>(c, token_ids, tid2eid, vocab, logits, splits, split_stride,
                                       ids, weights, dev_err, hist, super_sum, S, stream);
    case 16: return launch_tiles_seg<16>(c, token_ids, tid2eid, vocab, logits, splits,
                                         split_stride, ids, weights, dev_err, hist, super_sum,
                                         S, stream);
    default: return launch_tiles_seg<64>(c, token_ids, tid2eid, vocab, logits, splits,
                                         split_stride, ids, weights, dev_err, hist, super_sum,
                                         S, stream);
  }
}

}  // namespace moe
