// Token dispatch on gfx950: group routes r = t*k_stride + j by expert with a
// stable counting sort (counts, exclusive-scan offsets, permutation, inverse).
//
// Three kernels over tiles of kTile routes (4 waves x 4 chunks of 64):
//  1. histogram: each wave counts its chunks without atomics -- the lanes
//     holding the same expert are found with one ballot per distinct expert
//     (the leader lane adds the popcount to the wave's own LDS row), and the
//     tile's per-expert totals go to tile_hist[e][tile];
//  2. scan (one workgroup): per expert, the exclusive scan of its counts over
//     tiles (wave-wide scans, 64 tiles at a time), then the exclusive scan of
//     the per-expert totals over experts -> counts, offsets;
//  3. scatter: each tile recounts per wave, turns the counts into per-wave
//     starting positions (offsets[e] + earlier tiles + earlier waves), and
//     places every route at start + (same-expert lanes below it in the
//     ballot), advancing the start by the ballot's popcount -- so positions
//     rise with r inside every expert and nothing depends on scheduling.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kChunksPerWave = 4;
constexpr int kTile = kWaves * kChunksPerWave * kWave;  // routes per tile
constexpr int kMaxE = 1024;
constexpr int kScanThreads = 1024;

__device__ __forceinline__ int load_id(const int32_t* ids, int64_t r, int64_t R, int E,
                                       int* err) {
  int e = (r < R) ? ids[r] : -1;
  if (e >= E) {
    ++*err;
    e = -1;
  }
  return e;
}

// Count this wave's chunks into its LDS row (leader-per-distinct-id ballots).
__device__ __forceinline__ void count_chunks(const int32_t* ids, int64_t r0, int64_t R, int E,
                                             int32_t* row, int* err) {
  const int lane = lane_id();
  for (int ch = 0; ch < kChunksPerWave; ++ch) {
    const int e = load_id(ids, r0 + ch * kWave + lane, R, E, err);
    uint64_t mask = __ballot(e >= 0);
    while (mask) {
      const int leader = __ffsll((unsigned long long)mask) - 1;
      const int v = readlane_i32(e, leader);
      const uint64_t m = __ballot(e == v);
      if (lane == leader) row[v] += __popcll(m);
      mask &= ~m;
    }
  }
}

__global__ __launch_bounds__(kWaves * kWave) void disp_hist_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int nt,
    int32_t* __restrict__ tile_hist, int32_t* __restrict__ dev_err) {
  __shared__ int32_t wh[kWaves][kMaxE];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int e = tid & 63; e < E; e += kWave) wh[wave][e] = 0;
  __syncthreads();
  int err = 0;
  const int64_t r0 = (int64_t)blockIdx.x * kTile + wave * (kChunksPerWave * kWave);
  count_chunks(ids, r0, R, E, wh[wave], &err);
  __syncthreads();
  for (int e = tid; e < E; e += kWaves * kWave)
    tile_hist[(int64_t)e * nt + blockIdx.x] = wh[0][e] + wh[1][e] + wh[2][e] + wh[3][e];
  err = wave_sum_i32(err);
  if ((tid & 63) == 0 && err && dev_err) atomicAdd(dev_err, err);
}

__global__ __launch_bounds__(kScanThreads) void disp_scan_kernel(
    const int32_t* __restrict__ tile_hist, int nt, int E, int32_t* __restrict__ tile_base,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[kMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int nwaves = kScanThreads / kWave;
  for (int e = wave; e < E; e += nwaves) {
    int carry = 0;
    for (int b = 0; b < nt; b += kWave) {
      const int i = b + lane;
      const int v = (i < nt) ? tile_hist[(int64_t)e * nt + i] : 0;
      const int inc = wave_incl_scan_i32(v);
      if (i < nt) tile_base[(int64_t)e * nt + i] = carry + inc - v;
      carry += readlane_i32(inc, 63);
    }
    if (lane == 0) tot[e] = carry;
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int b = 0; b < E; b += kWave) {
      const int e = b + lane;
      const int v = (e < E) ? tot[e] : 0;
      const int inc = wave_incl_scan_i32(v);
      if (e < E) {
        counts[e] = v;
        offsets[e] = carry + inc - v;
      }
      carry += readlane_i32(inc, 63);
    }
    if (lane == 0) offsets[E] = carry;
  }
}

__global__ __launch_bounds__(kWaves * kWave) void disp_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int nt,
    const int32_t* __restrict__ tile_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int32_t wh[kWaves][kMaxE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = lane; e < E; e += kWave) wh[wave][e] = 0;
  __syncthreads();
  int err = 0;
  const int64_t r0 = (int64_t)blockIdx.x * kTile + wave * (kChunksPerWave * kWave);
  count_chunks(ids, r0, R, E, wh[wave], &err);
  __syncthreads();
  // per-wave starting positions of each expert inside this tile
  for (int e = tid; e < E; e += kWaves * kWave) {
    const int c0 = wh[0][e], c1 = wh[1][e], c2 = wh[2][e];
    const int base = offsets[e] + tile_base[(int64_t)e * nt + blockIdx.x];
    wh[0][e] = base;
    wh[1][e] = base + c0;
    wh[2][e] = base + c0 + c1;
    wh[3][e] = base + c0 + c1 + c2;
  }
  __syncthreads();
  const uint64_t below = lanemask_lt();
  int32_t* row = wh[wave];
  for (int ch = 0; ch < kChunksPerWave; ++ch) {
    const int64_t r = r0 + ch * kWave + lane;
    const int e = load_id(ids, r, R, E, &err);
    int pos = -1;
    uint64_t mask = __ballot(e >= 0);
    while (mask) {
      const int leader = __ffsll((unsigned long long)mask) - 1;
      const int v = readlane_i32(e, leader);
      const uint64_t m = __ballot(e == v);
      const int start = row[v];
      if (e == v) pos = start + __popcll(m & below);
      if (lane == leader) row[v] = start + __popcll(m);
      mask &= ~m;
    }
    if (r < R) {
      if (inv) inv[r] = pos;
      if (pos >= 0 && pos < R) perm[pos] = (int32_t)r;
    }
  }
}

}  // namespace

size_t dispatch_workspace_bytes(int64_t R, int32_t E) {
  const int64_t nt = (R + kTile - 1) / kTile;
  return (size_t)(2 * nt * (int64_t)E * sizeof(int32_t));
}

hipError_t launch_dispatch(const int32_t* ids, int64_t R, int32_t E,
                           int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv, void* workspace, int32_t* dev_err,
                           hipStream_t stream) {
  const int nt = (int)((R + kTile - 1) / kTile);
  int32_t* tile_hist = static_cast<int32_t*>(workspace);
  int32_t* tile_base = tile_hist + (int64_t)nt * E;
  if (nt > 0) {
    prof_begin(kStageDispHist, stream);
    hipLaunchKernelGGL(disp_hist_kernel, dim3(nt), dim3(kWaves * kWave), 0, stream, ids, R, E,
                       nt, tile_hist, dev_err);
    prof_end(kStageDispHist, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  prof_begin(kStageDispScan, stream);
  hipLaunchKernelGGL(disp_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, tile_hist, nt, E,
                     tile_base, counts, offsets);
  prof_end(kStageDispScan, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nt == 0) return e;
  prof_begin(kStageDispScatter, stream);
  hipLaunchKernelGGL(disp_scatter_kernel, dim3(nt), dim3(kWaves * kWave), 0, stream, ids, R, E,
                     nt, tile_base, offsets, perm, inv);
  prof_end(kStageDispScatter, stream);
  return hipGetLastError();
}

}  // namespace moe
