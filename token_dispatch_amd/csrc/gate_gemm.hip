// Gate contraction on gfx950 matrix cores.
//
// logits[t][e] = sum_i x[t][i] * W[e][i] (+ logit_bias[e]), fp32 accumulate.
// The gate of "DeepSeek-V3.2-Exp - Select experts" (gate-forward excerpt)
// casts both operands to fp32 before the linear map; bf16 products are exact
// in fp32, so bf16 inputs go through v_mfma_f32_16x16x32_bf16 and fp32
// inputs through v_mfma_f32_16x16x4_f32 (never rounded to bf16).
//
// Shape: M = T tokens (thousands), N = E experts (8..1024), K = d.  A
// workgroup of 4 waves owns BM tokens x BN experts (BN = all of E when
// E <= 384) so x, the large operand, streams from HBM once.  Each stage moves
// a 128-byte K slice of the x rows and W rows into LDS (16-byte loads, rows
// padded to 144 bytes so the 16 lanes of an MFMA row group hit distinct
// banks); the next stage's global loads are issued before the MFMAs of the
// current one.  Wave w computes all BM rows against experts
// [w*BN/4, (w+1)*BN/4).
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;             // K slice per stage, bytes
constexpr int kLdsStride = kRowBytes + 16; // padded LDS row, bytes
constexpr int kChunks = kRowBytes / 16;    // 16-byte chunks per row slice

template <typename In>
struct ElemInfo;
template <>
struct ElemInfo<uint16_t> {  // bf16 bits
  static constexpr int kPerChunk = 8;
};
template <>
struct ElemInfo<float> {
  static constexpr int kPerChunk = 4;
};

// Load one 16-byte chunk (elements [k, k+kPerChunk) of row `row`), zero
// outside [0, rows) x [0, d).  VEC: the row pitch and base are 16-byte
// aligned and d is a multiple of kPerChunk.
template <typename In, bool VEC>
__device__ __forceinline__ u32x4_t load_chunk(const In* base, int64_t row,
                                              int rows, int k, int d) {
  constexpr int P = ElemInfo<In>::kPerChunk;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (row >= rows) return v;
  const In* p = base + row * (int64_t)d + k;
  if (VEC) {
    if (k < d) v = *reinterpret_cast<const u32x4_t*>(p);
  } else {
    In tmp[P];
#pragma unroll
    for (int i = 0; i < P; ++i) tmp[i] = (k + i < d) ? p[i] : In(0);
    __builtin_memcpy(&v, tmp, 16);
  }
  return v;
}

template <typename In, int BM, int BN, bool VEC>
__global__ __launch_bounds__(kThreads) void gate_gemm_kernel(
    const In* __restrict__ x, const In* __restrict__ W,
    const float* __restrict__ logit_bias, float* __restrict__ logits, int T,
    int d, int E) {
  constexpr int P = ElemInfo<In>::kPerChunk;
  constexpr int BK = kRowBytes / sizeof(In);  // K elements per stage
  constexpr int MB = BM / 16;                 // 16-row blocks per wave
  constexpr int NW = BN / 4;                  // experts per wave
  constexpr int NB = NW / 16;                 // 16-col blocks per wave
  constexpr int A_CHUNKS = BM * kChunks / kThreads;
  constexpr int B_CHUNKS = BN * kChunks / kThreads;
  static_assert(BM % 16 == 0 && BN % 64 == 0, "tile shape");
  static_assert(A_CHUNKS >= 1 && BM * kChunks % kThreads == 0, "A tile chunks");
  static_assert(BN * kChunks % kThreads == 0, "B tile chunks");

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[BM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[BN * kLdsStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;

  u32x4_t ra[A_CHUNKS], rb[B_CHUNKS];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / kChunks, ck = c % kChunks;
      ra[i] = load_chunk<In, VEC>(x, m0 + r, T, k0 + ck * P, d);
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / kChunks, ck = c % kChunks;
      rb[i] = load_chunk<In, VEC>(W, (int64_t)n0 + r, E, k0 + ck * P, d);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int c = tid + i * kThreads;
      *reinterpret_cast<u32x4_t*>(lds_a + (c / kChunks) * kLdsStride + (c % kChunks) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const int c = tid + i * kThreads;
      *reinterpret_cast<u32x4_t*>(lds_b + (c / kChunks) * kLdsStride + (c % kChunks) * 16) = rb[i];
    }
  };

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int row16 = lane & 15;  // row of A / column of B this lane feeds
  const int kq = lane >> 4;     // which quarter of the MFMA's K this lane feeds
  const uint8_t* a_base = lds_a + row16 * kLdsStride;
  const uint8_t* b_base = lds_b + (wave * NW + row16) * kLdsStride;

  fetch(0);
  for (int k0 = 0; k0 < d; k0 += BK) {
    __syncthreads();  // previous stage's MFMAs are done with LDS
    stash();
    __syncthreads();
    if (k0 + BK < d) fetch(k0 + BK);  // in flight while the MFMAs run

    if constexpr (sizeof(In) == 2) {
      // two K=32 steps; lane feeds elements [kq*8, kq*8+8) of each step
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t af[MB], bfr[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(a_base + i * 16 * kLdsStride + ks * 64 + kq * 16);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8_t*>(b_base + j * 16 * kLdsStride + ks * 64 + kq * 16);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    } else {
      // two 16-wide K steps of four K=4 MFMAs.  A and B use the same
      // permutation of K: MFMA s takes element kq*4 + s of the step, so the
      // lane reads one float4 per operand and the sum is unchanged.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        f32x4_t af[MB], bfr[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
          af[i] = *reinterpret_cast<const f32x4_t*>(a_base + i * 16 * kLdsStride + ks * 64 + kq * 16);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          bfr[j] = *reinterpret_cast<const f32x4_t*>(b_base + j * 16 * kLdsStride + ks * 64 + kq * 16);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][s], bfr[j][s], acc[i][j], 0, 0, 0);
      }
    }
  }

  // D layout of a 16x16 MFMA: lane holds rows 4*(lane/16) + r, column lane%16.
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int e = n0 + wave * NW + j * 16 + row16;
    if (e >= E) continue;
    const float b = logit_bias ? logit_bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = m0 + i * 16 + kq * 4 + r;
        if (t < T) logits[t * E + e] = acc[i][j][r] + b;
      }
  }
}

template <typename In, int BM, int BN>
hipError_t launch_tile(const void* x, const void* W, const float* logit_bias,
                       float* logits, int T, int d, int E, hipStream_t s) {
  dim3 grid((E + BN - 1) / BN, (T + BM - 1) / BM);
  const bool vec = (d % ElemInfo<In>::kPerChunk == 0) &&
                   (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(W) % 16 == 0);
  if (vec) {
    prof_begin(kStageGate, s);
    hipLaunchKernelGGL((gate_gemm_kernel<In, BM, BN, true>), grid, dim3(kThreads), 0, s,
                       (const In*)x, (const In*)W, logit_bias, logits, T, d, E);
    prof_end(kStageGate, s);
  } else {
    prof_begin(kStageGate, s);
    hipLaunchKernelGGL((gate_gemm_kernel<In, BM, BN, false>), grid, dim3(kThreads), 0, s,
                       (const In*)x, (const In*)W, logit_bias, logits, T, d, E);
    prof_end(kStageGate, s);
  }
  return hipGetLastError();
}

template <typename In>
hipError_t launch_typed(const void* x, const void* W, const float* logit_bias,
                        float* logits, int T, int d, int E, hipStream_t s) {
  if (E <= 64) return launch_tile<In, 64, 64>(x, W, logit_bias, logits, T, d, E, s);
  if (E <= 128) {
    if (T >= 32768) return launch_tile<In, 128, 128>(x, W, logit_bias, logits, T, d, E, s);
    return launch_tile<In, 64, 128>(x, W, logit_bias, logits, T, d, E, s);
  }
  if (E <= 256) return launch_tile<In, 32, 256>(x, W, logit_bias, logits, T, d, E, s);
  return launch_tile<In, 32, 384>(x, W, logit_bias, logits, T, d, E, s);
}

}  // namespace

hipError_t launch_gate_gemm(int32_t dtype, const void* x, const void* W,
                            const float* logit_bias, float* logits, int32_t T,
                            int32_t d, int32_t E, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (dtype == 1) return launch_typed<uint16_t>(x, W, logit_bias, logits, T, d, E, stream);
  return launch_typed<float>(x, W, logit_bias, logits, T, d, E, stream);
}

}  // namespace moe
