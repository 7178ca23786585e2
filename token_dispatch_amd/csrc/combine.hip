// Combine on gfx950: the output row of each token is the weighted sum of the
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
// One wavefront per token.  Lanes 0..k-1 read the token's inv and weights;
// each valid slot's row index and weight then come to every lane with
// readlane (scalar registers), in slot order.  Each lane owns 16-byte units
// of the row (8 bf16 or 4 fp32), UPL of them per pass, and accumulates in
// fp32 with one fma per element per slot: sum_j w_j * Y_j, slots in order,
// then + shared.  Two slots' loads are issued before either is used.  The
// result is stored in the input type (bf16: round to nearest even).  Rows
// whose length is not a whole number of 16-byte units, or unaligned
// pointers, take the same loop with one element per unit.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kCombineWaves = 4;
constexpr int kUPL = 4;  // units per lane per pass

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
// single element (N = 1).
template <class Elem, int N>
struct Unit {
  static constexpr int kBytes = N * (int)sizeof(Elem);
  __device__ static void load(const Elem* row, int64_t u, float (&v)[N]) {
    if constexpr (N == 1) {
      if constexpr (sizeof(Elem) == 2)
        v[0] = bf16_to_f32(row[u]);
      else
        v[0] = row[u];
    } else {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 q = reinterpret_cast<const u32x4*>(row)[u];
      if constexpr (sizeof(Elem) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(q[i] << 16);
          v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(q[i]);
      }
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
      reinterpret_cast<u32x4*>(row)[u] = q;
    }
  }
};

// Elem: float or uint16_t (bf16 bits); N elements per unit (N * sizeof(Elem)
// = 16, or 1).
template <class Elem, int N>
__global__ __launch_bounds__(kCombineWaves * kWave) void combine_kernel(
    int32_t T, int32_t k, int32_t d, const Elem* __restrict__ Yp, int32_t R,
    const int32_t* __restrict__ inv, const float* __restrict__ weights,
    const Elem* __restrict__ shared, Elem* __restrict__ y, int32_t* __restrict__ dev_err) {
  using U = Unit<Elem, N>;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefronts leave together

  // the token's slots: lane j < k holds slot j
  int32_t p = -1;
  float w = 0.f;
  if (lane < k) {
    p = inv[t * k + lane];
    w = weights[t * k + lane];
  }
  const bool bad = lane < k && p >= R;
  const uint64_t bad_mask = __ballot(bad);
  if (bad_mask && lane == 0 && dev_err) atomicAdd(dev_err, (int)__popcll(bad_mask));
  uint64_t slots = __ballot(lane < k && p >= 0 && p < R);  // valid slots, in order

  const int64_t units = d / N;  // N divides d
  const Elem* sh = shared ? shared + t * d : nullptr;
  Elem* out = y + t * d;
  for (int64_t u0 = 0; u0 < units; u0 += (int64_t)kUPL * kWave) {
    float acc[kUPL][N];
#pragma unroll
    for (int a = 0; a < kUPL; ++a)
#pragma unroll
      for (int i = 0; i < N; ++i) acc[a][i] = 0.f;
    int64_t uu[kUPL];
#pragma unroll
    for (int a = 0; a < kUPL; ++a) {
      const int64_t u = u0 + (int64_t)a * kWave + lane;
      uu[a] = u < units ? u : units - 1;  // clamped: loads stay in the row
    }
    uint64_t rest = slots;
    while (rest) {  // two slots per step, both loaded before either is used
      const int j0 = __builtin_ctzll(rest);
      rest &= rest - 1;
      const int j1 = rest ? __builtin_ctzll(rest) : -1;
      if (j1 >= 0) rest &= rest - 1;
      const int32_t p0 = readlane_i32(p, j0);
      const float w0 = readlane_f32(w, j0);
      const int32_t p1 = j1 >= 0 ? readlane_i32(p, j1) : p0;
      const float w1 = j1 >= 0 ? readlane_f32(w, j1) : 0.f;
      const Elem* r0 = Yp + (int64_t)p0 * d;
      const Elem* r1 = Yp + (int64_t)p1 * d;
      float v0[kUPL][N], v1[kUPL][N];
#pragma unroll
      for (int a = 0; a < kUPL; ++a) U::load(r0, uu[a], v0[a]);
      if (j1 >= 0) {
#pragma unroll
        for (int a = 0; a < kUPL; ++a) U::load(r1, uu[a], v1[a]);
      }
#pragma unroll
      for (int a = 0; a < kUPL; ++a)
#pragma unroll
        for (int i = 0; i < N; ++i) acc[a][i] = fmaf(w0, v0[a][i], acc[a][i]);
      if (j1 >= 0) {
#pragma unroll
        for (int a = 0; a < kUPL; ++a)
#pragma unroll
          for (int i = 0; i < N; ++i) acc[a][i] = fmaf(w1, v1[a][i], acc[a][i]);
      }
    }
    if (sh) {
#pragma unroll
      for (int a = 0; a < kUPL; ++a) {
        float s[N];
        U::load(sh, uu[a], s);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[a][i] += s[i];
      }
    }
#pragma unroll
    for (int a = 0; a < kUPL; ++a) {
      const int64_t u = u0 + (int64_t)a * kWave + lane;
      if (u < units) U::store(out, u, acc[a]);
    }
  }
}

template <class Elem>
hipError_t launch_elem(int32_t T, int32_t k, int32_t d, const void* Yp, int32_t R,
                       const int32_t* inv, const float* weights, const void* shared, void* y,
                       int32_t* dev_err, hipStream_t stream) {
  constexpr int N = 16 / (int)sizeof(Elem);
  const auto a16 = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  const bool vec = d % N == 0 && a16(Yp) && a16(y) && (!shared || a16(shared));
  const dim3 grid((uint32_t)((T + kCombineWaves - 1) / kCombineWaves));
  const dim3 block(kCombineWaves * kWave);
  if (vec)
    return launch(kStageCombine, combine_kernel<Elem, N>, grid, block, stream, T, k, d,
                  static_cast<const Elem*>(Yp), R, inv, weights,
                  static_cast<const Elem*>(shared), static_cast<Elem*>(y), dev_err);
  return launch(kStageCombine, combine_kernel<Elem, 1>, grid, block, stream, T, k, d,
                static_cast<const Elem*>(Yp), R, inv, weights, static_cast<const Elem*>(shared),
                static_cast<Elem*>(y), dev_err);
}

}  // namespace

hipError_t launch_combine(int32_t T, int32_t k, int32_t d, int32_t dtype, const void* Yp,
                          int32_t R, const int32_t* inv, const float* weights,
                          const void* shared, void* y, int32_t* dev_err, hipStream_t stream) {
  if (T == 0 || d == 0) return hipSuccess;
  if (dtype == 1)
    return launch_elem<uint16_t>(T, k, d, Yp, R, inv, weights, shared, y, dev_err, stream);
  return launch_elem<float>(T, k, d, Yp, R, inv, weights, shared, y, dev_err, stream);
}

}  // namespace moe
