// Row movement around the experts on gfx950: the send buffer (token rows in
// dispatch order) and its per-rank layout, and the combine.
//
// Combine: the output row of each token is the weighted sum of the
// outputs its selected experts produced for it, plus a shared expert's
// output.  Sources: "Feature Request: dynamic number of experts (hyperparam
// per request)" (llama.cpp issue 13572), "Possible Implementation" -- the
// selected experts' outputs are combined with their weights; "ferrox_moe"
// crate documentation, function combine_expert_outputs -- routed plus shared
// expert outputs of one token.
//
// The expert outputs arrive in dispatch order: row p of Yp belongs to route
// perm[p], so slot j of token t reads row inv[t*k + j] (the inverse the
// dispatch wrote).  The work is a gather and a short reduction, HBM-bound:
// every valid slot reads one row of d elements, every token writes one.
//
// One wavefront per (token, chunk of 64 x UPL 16-byte units of its row).
// Lanes 0..k-1 read the token's inv and weights; each valid slot's row index
// and weight then come to every lane with readlane (scalar registers), in
// slot order.  The loads of up to 16 row pieces per lane (16 / UPL slots)
// are issued together with the shared row's (one memory round trip for a
// token's slots, not one per slot), then added in fp32 with one fma per
// element per slot: sum_j w_j * Y_j, slots in order, then + shared.
// The result is stored in the input type (bf16: round to nearest even).
// Expert rows are read once and outputs written once, so 16-byte units go
// through non-temporal loads and stores (Qwen3-like rows: 5.5 -> 6.2 TB/s;
// DeepSeek-V3-like: 5.2 -> 6.5 TB/s); the shared rows keep the default
// policy.
// Rows whose length is not a whole number of 16-byte units, or unaligned
// pointers, take the same loop with one element per unit.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kCombineWaves = 4;
constexpr int kSlotsInFlight = 16;  // slots whose rows are loaded together

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest even on the upper 16 bits (quiet NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One unit of a row: N = 8 (bf16) or 4 (fp32) elements from 16 bytes, or a
// single element (N = 1).  raw() and raw_cached() load it as it is in memory
// (so that many units can be in flight in few registers; raw() is
// non-temporal), at() reads element i of it.
template <class Elem, int N>
struct Unit {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  using Raw = std::conditional_t<(N > 1), u32x4, Elem>;
  __device__ static Raw raw(const Elem* row, int64_t u) {
    if constexpr (N > 1)  // read once: non-temporal
      return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + u);
    else
      return row[u];
  }
  __device__ static Raw raw_cached(const Elem* row, int64_t u) {
    if constexpr (N > 1)
      return reinterpret_cast<const u32x4*>(row)[u];
    else
      return row[u];
  }
  __device__ static float at(const Raw& q, int i) {
    if constexpr (N == 1) {
      if constexpr (sizeof(Elem) == 2)
        return bf16_to_f32(q);
      else
        return q;
    } else if constexpr (sizeof(Elem) == 2) {
      return __uint_as_float(i % 2 ? q[i / 2] & 0xFFFF0000u : q[i / 2] << 16);
    } else {
      return __uint_as_float(q[i]);
    }
  }
  __device__ static void store(Elem* row, int64_t u, const float (&v)[N]) {
    if constexpr (N == 1) {
      if constexpr (sizeof(Elem) == 2)
        row[u] = (Elem)f32_to_bf16(v[0]);
      else
        row[u] = v[0];
    } else {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      u32x4 q;
      if constexpr (sizeof(Elem) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = f32_to_bf16(v[2 * i]) | (f32_to_bf16(v[2 * i + 1]) << 16);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = __float_as_uint(v[i]);
      }
      __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(row) + u);  // written once
    }
  }
};

// Elem: float or uint16_t (bf16 bits); N elements per unit (N * sizeof(Elem)
// = 16, or 1); UPL units per lane, so wavefront g handles chunk
// c = g % nchunks (UPL * 64 units) of the row of token t = g / nchunks.
// Slots are loaded kSlotsInFlight / UPL at a time: the row pieces in flight
// per wavefront stay at 16 (registers), and few slots (k = 1, 2) still
// keep several pieces in flight.
template <class Elem, int N, int UPL>
__global__ __launch_bounds__(kCombineWaves * kWave) void combine_kernel(
    int32_t T, int32_t k, int32_t d, int32_t nchunks, const Elem* __restrict__ Yp, int32_t R,
    const int32_t* __restrict__ inv, const float* __restrict__ weights,
    const Elem* __restrict__ shared, Elem* __restrict__ y, int32_t* __restrict__ dev_err) {
  using U = Unit<Elem, N>;
  constexpr int kSIF = kSlotsInFlight / UPL;
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  const int64_t t = g / nchunks;
  const int c = (int)(g - t * nchunks);
  if (t >= T) return;  // whole wavefronts leave together

  // the token's slots: lane j < k holds slot j
  int32_t p = -1;
  float w = 0.f;
  if (lane < k) {
    p = inv[t * k + lane];
    w = weights[t * k + lane];
  }
  if (c == 0) {  // one chunk of the token counts its bad slots
    const uint64_t bad = __ballot(lane < k && p >= R);
    if (bad && lane == 0 && dev_err) atomicAdd(dev_err, (int)__popcll(bad));
  }
  uint64_t rest = __ballot(lane < k && p >= 0 && p < R);  // valid slots, in order

  const int64_t units = d / N;  // N divides d
  int64_t uc[UPL];  // clamped: loads stay in the row
#pragma unroll
  for (int a = 0; a < UPL; ++a) {
    const int64_t u = ((int64_t)c * UPL + a) * kWave + lane;
    uc[a] = u < units ? u : units - 1;
  }
  // the shared row's loads go out first, with the first slots', through the
  // cache (non-temporal loads of the shared rows measured 8-15% slower)
  typename U::Raw sh[UPL];
  if (shared) {
#pragma unroll
    for (int a = 0; a < UPL; ++a) sh[a] = U::raw_cached(shared + t * d, uc[a]);
  }
  float acc[UPL][N];
#pragma unroll
  for (int a = 0; a < UPL; ++a)
#pragma unroll
    for (int i = 0; i < N; ++i) acc[a][i] = 0.f;
  while (rest) {  // up to kSIF slots: all loads issued, then added in order
    int32_t row[kSIF];
    float wt[kSIF];
    int m = 0;
#pragma unroll
    for (int i = 0; i < kSIF; ++i) {
      row[i] = 0;
      wt[i] = 0.f;
      if (rest) {
        const int j = __builtin_ctzll(rest);
        rest &= rest - 1;
        row[i] = readlane_i32(p, j);
        wt[i] = readlane_f32(w, j);
        m = i + 1;
      }
    }
    typename U::Raw v[kSIF][UPL];
#pragma unroll
    for (int i = 0; i < kSIF; ++i)
      if (i < m) {
#pragma unroll
        for (int a = 0; a < UPL; ++a) v[i][a] = U::raw(Yp + (int64_t)row[i] * d, uc[a]);
      }
#pragma unroll
    for (int i = 0; i < kSIF; ++i)
      if (i < m) {
#pragma unroll
        for (int a = 0; a < UPL; ++a)
#pragma unroll
          for (int e = 0; e < N; ++e) acc[a][e] = fmaf(wt[i], U::at(v[i][a], e), acc[a][e]);
      }
  }
#pragma unroll
  for (int a = 0; a < UPL; ++a) {
    if (shared) {
#pragma unroll
      for (int e = 0; e < N; ++e) acc[a][e] += U::at(sh[a], e);
    }
    const int64_t u = ((int64_t)c * UPL + a) * kWave + lane;
    if (u < units) U::store(y + t * d, u, acc[a]);
  }
}

template <class Elem, int N, int UPL>
hipError_t launch_combine_upl(int32_t T, int32_t k, int32_t d, int64_t units, const void* Yp,
                              int32_t R, const int32_t* inv, const float* weights,
                              const void* shared, void* y, int32_t* dev_err,
                              hipStream_t stream) {
  const int32_t nchunks = (int32_t)((units + UPL * kWave - 1) / (UPL * kWave));
  const int64_t waves = (int64_t)T * nchunks;
  if ((waves + kCombineWaves - 1) / kCombineWaves > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)((waves + kCombineWaves - 1) / kCombineWaves));
  const dim3 block(kCombineWaves * kWave);
  return launch(kStageCombine, combine_kernel<Elem, N, UPL>, grid, block, stream, T, k, d,
                nchunks, static_cast<const Elem*>(Yp), R, inv, weights,
                static_cast<const Elem*>(shared), static_cast<Elem*>(y), dev_err);
}

template <class Elem>
hipError_t launch_elem(int32_t T, int32_t k, int32_t d, const void* Yp, int32_t R,
                       const int32_t* inv, const float* weights, const void* shared, void* y,
                       int32_t* dev_err, hipStream_t stream) {
  constexpr int N = 16 / (int)sizeof(Elem);
  const auto a16 = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  const bool vec = d % N == 0 && a16(Yp) && a16(y) && (!shared || a16(shared));
  if (!vec)
    return launch_combine_upl<Elem, 1, 1>(T, k, d, d, Yp, R, inv, weights, shared, y, dev_err,
                                          stream);
  // units per lane by slot count: 1 or 2 slots take 4, 3 or 4 take 2 (a
  // Switch-like top-1 combine 88.7 -> 61.9 us, gpt-oss-like k = 4
  // 374 -> 363 us; 5 or more slots fill the loads with one unit per lane)
  const int64_t units = d / N;
  if (k <= 2)
    return launch_combine_upl<Elem, N, 4>(T, k, d, units, Yp, R, inv, weights,
                                      shared, y, dev_err, stream);
  if (k <= 4)
    return launch_combine_upl<Elem, N, 2>(T, k, d, units, Yp, R, inv, weights,
                                      shared, y, dev_err, stream);
  return launch_combine_upl<Elem, N, 1>(T, k, d, units, Yp, R, inv, weights, shared, y,
                                        dev_err, stream);
}

// The send buffer of expert parallelism ("I modelli MoE open hanno router
// opposti": with experts spread over GPUs every routing choice becomes
// all-to-all traffic; the dispatch order is the send order): the row of
// route r is the hidden state of its token, placed at row inv[r] of out --
// dispatch order with the dispatch's inverse, the expert-major slots
// e*C + rank with a capacity limit's.  It is written from the token side:
// each token row is read once and stored once per placed route, so x moves
// over HBM once (T*d) and the buffer once (R*d); a gather over the dispatch
// order would read each token row k times.
// One wavefront per (token, 256 units of its row): each lane loads its 4
// units, lanes 0..63 read 64 of the token's places at a time, and each
// placed route's row index comes to every lane with readlane; the stores are
// non-temporal (the buffer is written once; non-temporal loads of x measured
// 2-3% slower).  2, 4 or 8 units per lane and 2, 4 or 8 wavefronts per
// workgroup all run within 5% of each other (4.8-5.4 TB/s): the stream of
// row writes sets the pace.  Bytes are moved as they are, in 16-byte units
// where rows and pointers allow (U = u32x4), else in elements.
constexpr int kPermuteUPL = 4;
template <class U>
__global__ __launch_bounds__(kCombineWaves * kWave) void permute_kernel(
    int32_t T, int32_t k, int64_t units, int32_t nchunks, int32_t out_rows,
    const U* __restrict__ x, const int32_t* __restrict__ inv, U* __restrict__ out,
    int32_t* __restrict__ dev_err) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  const int64_t t = g / nchunks;
  const int c = (int)(g - t * nchunks);
  if (t >= T) return;  // whole wavefronts
  U v[kPermuteUPL];
#pragma unroll
  for (int a = 0; a < kPermuteUPL; ++a) {
    const int64_t u = ((int64_t)c * kPermuteUPL + a) * kWave + lane;
    if (u < units) v[a] = x[t * units + u];
  }
  for (int j0 = 0; j0 < k; j0 += kWave) {
    const int n = min(kWave, k - j0);
    const int32_t q_l = lane < n ? inv[t * k + j0 + lane] : -1;
    if (c == 0 && lane == 0 && dev_err) {
      int bad = 0;
      for (int jj = 0; jj < n; ++jj) bad += inv[t * k + j0 + jj] >= out_rows;
      if (bad) atomicAdd(dev_err, bad);
    }
    for (int jj = 0; jj < n; ++jj) {
      const int32_t q = __builtin_amdgcn_readlane(q_l, jj);
      if (q < 0 || q >= out_rows) continue;  // not placed, or no such row
      U* __restrict__ row = out + (int64_t)q * units;
#pragma unroll
      for (int a = 0; a < kPermuteUPL; ++a) {
        const int64_t u = ((int64_t)c * kPermuteUPL + a) * kWave + lane;
        if (u < units) {
          if constexpr (sizeof(U) == 16)
            __builtin_nontemporal_store(v[a], row + u);
          else
            row[u] = v[a];
        }
      }
    }
  }
}

// Per-rank send counts and offsets: rank n owns experts [n*E/N, (n+1)*E/N),
// so its block of the dispatch order starts at offsets[n*E/N].
__global__ __launch_bounds__(256) void ep_layout_kernel(const int32_t* __restrict__ offsets,
                                                        int32_t E, int32_t N,
                                                        int32_t* __restrict__ send_counts,
                                                        int32_t* __restrict__ send_offsets) {
  for (int n = threadIdx.x; n <= N; n += 256) {
    const int32_t o = offsets[(int64_t)n * E / N];
    send_offsets[n] = o;
    if (n < N) send_counts[n] = offsets[(int64_t)(n + 1) * E / N] - o;
  }
}

template <class U>
hipError_t launch_permute_units(int32_t T, int32_t k, int64_t units, const void* x,
                                const int32_t* inv, int32_t out_rows, void* out,
                                int32_t* dev_err, hipStream_t stream) {
  const int32_t nchunks = (int32_t)((units + kPermuteUPL * kWave - 1) / (kPermuteUPL * kWave));
  const int64_t blocks = ((int64_t)T * nchunks + kCombineWaves - 1) / kCombineWaves;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  return launch(kStagePermute, permute_kernel<U>, dim3((uint32_t)blocks),
                dim3(kCombineWaves * kWave), stream, T, k, units, nchunks, out_rows,
                static_cast<const U*>(x), inv, static_cast<U*>(out), dev_err);
}

}  // namespace

hipError_t launch_permute(int32_t T, int32_t k, int32_t d, int32_t dtype, const void* x,
                          const int32_t* inv, int32_t out_rows, void* out, int32_t* dev_err,
                          hipStream_t stream) {
  if (T == 0 || d == 0) return hipSuccess;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t row_bytes = (int64_t)d * (dtype == 1 ? 2 : 4);
  const auto a16 = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  if (row_bytes % 16 == 0 && a16(x) && a16(out))
    return launch_permute_units<u32x4>(T, k, row_bytes / 16, x, inv, out_rows, out, dev_err,
                                       stream);
  if (dtype == 1)
    return launch_permute_units<uint16_t>(T, k, d, x, inv, out_rows, out, dev_err, stream);
  return launch_permute_units<uint32_t>(T, k, d, x, inv, out_rows, out, dev_err, stream);
}

hipError_t launch_ep_layout(const int32_t* offsets, int32_t E, int32_t N, int32_t* send_counts,
                            int32_t* send_offsets, hipStream_t stream) {
  return launch(kStageEpLayout, ep_layout_kernel, dim3(1), dim3(256), stream, offsets, E, N,
                send_counts, send_offsets);
}

hipError_t launch_combine(int32_t T, int32_t k, int32_t d, int32_t dtype, const void* Yp,
                          int32_t R, const int32_t* inv, const float* weights,
                          const void* shared, void* y, int32_t* dev_err, hipStream_t stream) {
  if (T == 0 || d == 0) return hipSuccess;
  if (dtype == 1)
    return launch_elem<uint16_t>(T, k, d, Yp, R, inv, weights, shared, y, dev_err, stream);
  return launch_elem<float>(T, k, d, Yp, R, inv, weights, shared, y, dev_err, stream);
}

}  // namespace moe
