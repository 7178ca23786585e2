// Token dispatch on gfx950: group routes r = t*k_stride + j by expert with a
// stable counting sort (counts, exclusive-scan offsets, permutation, inverse).
//
// Routes are cut into tiles of 4 waves x CPW chunks of 64 lanes (512, 1024 or
// 2048 routes).  Lanes that hold the same expert id ("peers") are found
// without atomics: one ballot per bit of the id narrows each lane's peer
// mask, so a chunk of 64 routes costs ceil(log2 E) ballots.  A lane's rank
// among its peers is the popcount of the peers below it, and the lowest peer
// (the leader) alone updates the wave's own LDS row for that expert.
//
// Two kernels when the tile histograms are small (tiles x E <= 32 Ki
// counts, the tile size grown to get there):
//  1. histogram: per-tile, per-expert counts -> tile_hist[tile][e].
//  2. scatter: every workgroup reads the whole (L2-resident) histogram once,
//     with all loads in flight together, and forms each expert's total and
//     its count in earlier tiles; scans the totals over experts (offsets;
//     workgroup 0 writes counts and offsets); recounts its tile per wave and
//     places route r at offsets[e] + (earlier tiles) + (earlier waves) +
//     (earlier chunks) + rank.
// Three kernels otherwise (tiles of 512): the histogram as tile_hist[e][tile],
// one wave per expert scanning its counts over tiles (exclusive) ->
// tile_base[e][tile] and totals[e], then the same scatter reading those.
// Positions rise with r inside each expert and do not depend on how
// workgroups are scheduled; integer sums make every path exact.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kChunksPerWave = 2;                       // three-kernel path
constexpr int kTile = kWaves * kChunksPerWave * kWave;  // 512 routes per tile
constexpr int kMaxE = 1024;
constexpr int kFusedMaxCounts = 32 * 1024;              // tiles x E, two-kernel path
constexpr int kFusedBatch = 16;                         // 16-byte loads in flight per thread
constexpr int kScanWaves = 16;                          // experts per scan workgroup
constexpr int kScanPrefetch = 8;                        // chunks of 64 tiles in registers

// This wave's CPW chunks of 64 routes starting at r0 (ids >= E
// count as errors and become -1).  All loads are issued before any is used:
// clamped addresses, validity applied afterwards.
template <int CPW>
__device__ __forceinline__ void load_chunks(const int32_t* __restrict__ ids, int64_t r0,
                                            int64_t R, int E, int (&e)[CPW], int* err) {
  const int lane = __lane_id();
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch) {
    const int64_t r = r0 + ch * kWave + lane;
    e[ch] = ids[r < R ? r : R - 1];
  }
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch) {
    const int64_t r = r0 + ch * kWave + lane;
    if (r >= R) e[ch] = -1;
    if (e[ch] >= E) {
      ++*err;
      e[ch] = -1;
    }
  }
}

// Count this wave's chunks into its LDS row.
template <int CPW>
__device__ __forceinline__ void count_chunks(const int (&e)[CPW], int nbits, int32_t* row) {
  const uint64_t below = lanemask_lt();
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch) {
    const uint64_t p = peer_mask(e[ch], nbits);
    if (e[ch] >= 0 && (p & below) == 0) row[e[ch]] += __popcll(p);
  }
}

// Per-tile histogram; tile-major (tile_hist[tile][e]) for the two-kernel
// path, expert-major (tile_hist[e][tile]) for the tile scan.
template <int CPW, bool TILE_MAJOR>
__global__ __launch_bounds__(kThreads) void disp_hist_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int nbits, int nt,
    int32_t* __restrict__ tile_hist, int32_t* __restrict__ dev_err) {
  __shared__ int32_t wh[kWaves][kMaxE];
  const int tid = threadIdx.x, wave = tid >> 6;
  int err = 0;
  int ev[CPW];
  load_chunks<CPW>(ids, (int64_t)blockIdx.x * (kWaves * CPW * kWave) + wave * (CPW * kWave), R,
                   E, ev, &err);
  for (int e = tid & 63; e < E; e += kWave) wh[wave][e] = 0;
  __syncthreads();
  count_chunks<CPW>(ev, nbits, wh[wave]);
  __syncthreads();
  for (int e = tid; e < E; e += kThreads)
    tile_hist[TILE_MAJOR ? (int64_t)blockIdx.x * E + e : (int64_t)e * nt + blockIdx.x] =
        wh[0][e] + wh[1][e] + wh[2][e] + wh[3][e];
  err = wave_sum_i32(err);
  if ((tid & 63) == 0 && err && dev_err) atomicAdd(dev_err, err);
}

// One wave per expert: exclusive scan of its per-tile counts, and its total.
__global__ __launch_bounds__(kScanWaves * kWave) void disp_tile_scan_kernel(
    const int32_t* __restrict__ tile_hist, int nt, int E, int32_t* __restrict__ tile_base,
    int32_t* __restrict__ totals) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * kScanWaves + (threadIdx.x >> 6);
  if (e >= E) return;
  const int32_t* src = tile_hist + (int64_t)e * nt;
  int32_t* dst = tile_base + (int64_t)e * nt;
  int carry = 0;
  for (int b0 = 0; b0 < nt; b0 += kScanPrefetch * kWave) {
    int v[kScanPrefetch];
#pragma unroll
    for (int c = 0; c < kScanPrefetch; ++c) {
      const int i = b0 + c * kWave + lane;
      v[c] = (i < nt) ? src[i] : 0;
    }
#pragma unroll
    for (int c = 0; c < kScanPrefetch; ++c) {
      const int i = b0 + c * kWave + lane;
      const int inc = wave_incl_scan_i32(v[c]);
      if (i < nt) dst[i] = carry + inc - v[c];
      carry += readlane_i32(inc, 63);
    }
  }
  if (lane == 0) totals[e] = carry;
}

// Stable placement.  FUSED: totals and earlier-tile counts come from the
// tile-major histogram (tile_hist[nt][E], E % 4 == 0, nt * E <=
// kFusedMaxCounts); otherwise from tile_base[e][tile] and totals[e].
template <int CPW, bool FUSED>
__global__ __launch_bounds__(kThreads) void disp_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int nbits, int nt,
    const int32_t* __restrict__ tile_hist, const int32_t* __restrict__ tile_base,
    const int32_t* __restrict__ totals, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int32_t wh[kWaves][kMaxE];
  __shared__ int32_t off[kMaxE];
  __shared__ int32_t tot[FUSED ? kMaxE : 1];
  __shared__ int32_t wsum[kWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tile = blockIdx.x;

  int err = 0;
  int ev[CPW];
  const int64_t r0 = (int64_t)tile * (kWaves * CPW * kWave) + wave * (CPW * kWave);
  if (tile < nt) load_chunks<CPW>(ids, r0, R, E, ev, &err);

  if constexpr (FUSED) {
    // Thread (g, p) owns experts 4g .. 4g+3 and tiles p, p + P, p + 2P, ...
    // (P = 1024 / E threads per expert group): 16-byte loads, 16 in flight,
    // register sums of all tiles and of the tiles before this one, then the
    // P partial sums of each expert added through LDS (wh rows 0 and 1).
    using i32x4 = int __attribute__((ext_vector_type(4)));
    const int G = E / 4, P = kMaxE / E;
    const int g = tid % G, p = tid / G;
    i32x4 all = {0, 0, 0, 0}, before = {0, 0, 0, 0};
    if (p < P) {
      const i32x4* src = reinterpret_cast<const i32x4*>(tile_hist) + g;
      for (int t0 = p; t0 < nt; t0 += kFusedBatch * P) {
        i32x4 v[kFusedBatch];
#pragma unroll
        for (int i = 0; i < kFusedBatch; ++i) {
          const int t = t0 + i * P;
          v[i] = src[(int64_t)(t < nt ? t : 0) * G];  // tile 0 always exists
        }
#pragma unroll
        for (int i = 0; i < kFusedBatch; ++i) {
          const int t = t0 + i * P;
          if (t < nt) all += v[i];
          if (t < tile) before += v[i];
        }
      }
    }
    int32_t* part_all = wh[0];     // [P][E], P * E <= kMaxE
    int32_t* part_before = wh[1];
    if (p < P)
      for (int c = 0; c < 4; ++c) {
        part_all[p * E + 4 * g + c] = all[c];
        part_before[p * E + 4 * g + c] = before[c];
      }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
      int a = 0, b = 0;
      for (int q = 0; q < P; ++q) {
        a += part_all[q * E + e];
        b += part_before[q * E + e];
      }
      tot[e] = a;
      off[e] = b;
    }
    __syncthreads();
  }

  // offsets: exclusive scan of totals over experts (4 experts per thread)
  int t4[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    if constexpr (FUSED)
      t4[i] = e < E ? tot[e] : 0;
    else
      t4[i] = (e < E && totals != nullptr) ? totals[e] : 0;
    s += t4[i];
  }
  const int inc = wave_incl_scan_i32(s);
  if (lane == 63) wsum[wave] = inc;
  for (int e = lane; e < E; e += kWave) wh[wave][e] = 0;
  __syncthreads();
  int base = inc - s;
  for (int w = 0; w < wave; ++w) base += wsum[w];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    if (e < E) {
      // FUSED: off[e] held this tile's earlier-tile count; only this thread
      // touches entry e between the barriers
      off[e] = FUSED ? base + off[e] : base;
      if (blockIdx.x == 0) {
        counts[e] = t4[i];
        offsets[e] = base;
      }
    }
    base += t4[i];
  }
  if (blockIdx.x == 0 && tid == kThreads - 1) offsets[E] = base;
  if (tile >= nt) return;  // only when there are no routes at all

  count_chunks<CPW>(ev, nbits, wh[wave]);
  __syncthreads();
  // per-wave starting positions of each expert inside this tile
  for (int e = tid; e < E; e += kThreads) {
    const int c0 = wh[0][e], c1 = wh[1][e], c2 = wh[2][e];
    const int b = FUSED ? off[e] : off[e] + tile_base[(int64_t)e * nt + tile];
    wh[0][e] = b;
    wh[1][e] = b + c0;
    wh[2][e] = b + c0 + c1;
    wh[3][e] = b + c0 + c1 + c2;
  }
  __syncthreads();
  const uint64_t below = lanemask_lt();
  int32_t* row = wh[wave];
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch) {
    const int64_t r = r0 + ch * kWave + lane;
    const int e = ev[ch];
    const uint64_t p = peer_mask(e, nbits);
    int pos = -1;
    if (e >= 0) {
      const int start = row[e];
      pos = start + __popcll(p & below);
      if ((p & below) == 0) row[e] = start + __popcll(p);
    }
    if (r < R) {
      if (inv) inv[r] = pos;
      if (pos >= 0 && pos < R) perm[pos] = (int32_t)r;
    }
  }
}

int bits_for(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

// Chunks per wave for the two-kernel path: the smallest tile that keeps the
// histogram within kFusedMaxCounts, or 0 (three-kernel path).
int fused_cpw(int64_t R, int32_t E) {
  if (E % 4 != 0 || std::getenv("MOE_DISPATCH_UNFUSED")) return 0;  // tuning: 3 kernels
  for (int cpw : {2, 4, 8}) {
    const int64_t nt = (R + kWaves * cpw * kWave - 1) / (kWaves * cpw * kWave);
    if (nt * E > kFusedMaxCounts) continue;
    // Large tiles leave few placement workgroups, each reading every count
    // (DeepSeek-V4-like, 48 tiles x 384 experts: 17.5 us against 13.8 us
    // for three kernels over 192 tiles): three kernels once their tiles
    // give at least 128 workgroups and these give fewer.
    if (nt < 128 && (R + kTile - 1) / kTile >= 128) return 0;
    return cpw;
  }
  return 0;
}

template <int CPW>
hipError_t launch_fused(const int32_t* ids, int64_t R, int32_t E, int nbits, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* tile_hist,
                        int32_t* dev_err, hipStream_t stream) {
  const int nt = (int)((R + kWaves * CPW * kWave - 1) / (kWaves * CPW * kWave));
  hipError_t e = launch(kStageDispHist, disp_hist_kernel<CPW, true>, dim3(nt), dim3(kThreads),
                        stream, ids, R, E, nbits, nt, tile_hist, dev_err);
  if (e != hipSuccess) return e;
  return launch(kStageDispScatter, disp_scatter_kernel<CPW, true>, dim3(nt), dim3(kThreads),
                stream, ids, R, E, nbits, nt, (const int32_t*)tile_hist, (const int32_t*)nullptr,
                (const int32_t*)nullptr, counts, offsets, perm, inv);
}

template <int CPW>
hipError_t launch_placement(const int32_t* ids, int64_t R, int32_t E, int nbits, int nt,
                            const int32_t* tile_hist, int32_t* counts, int32_t* offsets,
                            int32_t* perm, int32_t* inv, hipStream_t stream) {
  return launch(kStageDispScatter, disp_scatter_kernel<CPW, true>, dim3(nt), dim3(kThreads),
                stream, ids, R, E, nbits, nt, tile_hist, (const int32_t*)nullptr,
                (const int32_t*)nullptr, counts, offsets, perm, inv);
}

}  // namespace

bool dispatch_hist_ok(int64_t R, int32_t E, int32_t tile_routes) {
  if (R <= 0 || E % 4 != 0 || E > kMaxE) return false;
  if (tile_routes != 256 && tile_routes != 512 && tile_routes != 1024 && tile_routes != 2048)
    return false;
  return (R + tile_routes - 1) / tile_routes * E <= kFusedMaxCounts;
}

hipError_t launch_dispatch_from_hist(const int32_t* ids, int64_t R, int32_t E,
                                     int32_t* counts, int32_t* offsets, int32_t* perm,
                                     int32_t* inv, const int32_t* tile_hist,
                                     int32_t tile_routes, hipStream_t stream) {
  if (!dispatch_hist_ok(R, E, tile_routes)) return hipErrorInvalidValue;
  const int nt = (int)((R + tile_routes - 1) / tile_routes);
  const int nbits = bits_for(E);
  switch (tile_routes) {
    case 256: return launch_placement<1>(ids, R, E, nbits, nt, tile_hist, counts, offsets, perm, inv, stream);
    case 512: return launch_placement<2>(ids, R, E, nbits, nt, tile_hist, counts, offsets, perm, inv, stream);
    case 1024: return launch_placement<4>(ids, R, E, nbits, nt, tile_hist, counts, offsets, perm, inv, stream);
    default: return launch_placement<8>(ids, R, E, nbits, nt, tile_hist, counts, offsets, perm, inv, stream);
  }
}

int dispatch_kernels(int64_t R, int32_t E) {
  if (R <= 0) return 1;  // zero counts and offsets only
  return fused_cpw(R, E) ? 2 : 3;
}

size_t dispatch_workspace_bytes(int64_t R, int32_t E) {
  if (R <= 0) return 0;  // no routes: only counts and offsets are written
  if (const int cpw = fused_cpw(R, E)) {
    const int64_t nt = (R + kWaves * cpw * kWave - 1) / (kWaves * cpw * kWave);
    return (size_t)(nt * E * (int64_t)sizeof(int32_t));
  }
  const int64_t nt = (R + kTile - 1) / kTile;
  return (size_t)((2 * nt + 1) * (int64_t)E * sizeof(int32_t));
}

hipError_t launch_dispatch(const int32_t* ids, int64_t R, int32_t E,
                           int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv, void* workspace, int32_t* dev_err,
                           hipStream_t stream) {
  const int nbits = bits_for(E);
  int32_t* ws = static_cast<int32_t*>(workspace);
  if (R > 0) {
    switch (fused_cpw(R, E)) {
      case 2: return launch_fused<2>(ids, R, E, nbits, counts, offsets, perm, inv, ws, dev_err, stream);
      case 4: return launch_fused<4>(ids, R, E, nbits, counts, offsets, perm, inv, ws, dev_err, stream);
      case 8: return launch_fused<8>(ids, R, E, nbits, counts, offsets, perm, inv, ws, dev_err, stream);
      default: break;
    }
  }
  const int nt = (int)((R + kTile - 1) / kTile);
  int32_t* tile_hist = ws;
  int32_t* tile_base = tile_hist + (int64_t)nt * E;
  int32_t* totals = tile_base + (int64_t)nt * E;
  hipError_t e;
  if (nt > 0) {
    e = launch(kStageDispHist, disp_hist_kernel<kChunksPerWave, false>, dim3(nt),
               dim3(kThreads), stream, ids, R, E, nbits, nt, tile_hist, dev_err);
    if (e != hipSuccess) return e;
    e = launch(kStageDispScan, disp_tile_scan_kernel, dim3((E + kScanWaves - 1) / kScanWaves),
               dim3(kScanWaves * kWave), stream, (const int32_t*)tile_hist, nt, E, tile_base,
               totals);
    if (e != hipSuccess) return e;
  }
  // with no routes the scatter kernel runs one workgroup that only writes
  // zero counts and offsets (totals is not read then)
  return launch(kStageDispScatter, disp_scatter_kernel<kChunksPerWave, false>,
                dim3(nt > 0 ? nt : 1), dim3(kThreads), stream, ids, R, E, nbits, nt,
                (const int32_t*)nullptr, (const int32_t*)tile_base,
                (const int32_t*)(nt > 0 ? totals : nullptr), counts, offsets, perm, inv);
}

}  // namespace moe
