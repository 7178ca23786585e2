// Token dispatch on gfx950: group routes r = t*k_stride + j by expert with a
// stable counting sort (counts, exclusive-scan offsets, permutation, inverse).
//
// Routes are cut into tiles of 256 to 2048 routes, chunks of 64 lanes.
// Lanes that hold the same expert id ("peers") are found without atomics:
// one ballot per bit of the id narrows each lane's peer mask, so a chunk of
// 64 routes costs ceil(log2 E) ballots.  A lane's rank among its peers is
// the popcount of the peers below it, and the lowest peer (the leader)
// alone updates the wave's own LDS row for that expert.
//
// Two kernels when the tile histograms are small (tiles x E <= 32 Ki
// counts, E % 8 == 0, the tile size grown to get there):
//  1. histogram: per-tile, per-expert counts -> tile_hist[tile][e], 16-bit
//     (or written by the routing kernels themselves, see kernels.h).
//  2. placement: every workgroup reads the whole (L2-resident) histogram,
//     with all loads in flight together, and forms each expert's total and
//     its count in earlier tiles; scans the totals over experts (offsets;
//     workgroup 0 writes counts and offsets); recounts its tile (up to 16
//     waves of one chunk, keeping each route's offset inside its wave) and
//     places route r at offsets[e] + (earlier tiles) + (earlier waves) +
//     (offset in the wave).
// Three kernels otherwise (tiles of 512): the histogram as 32-bit
// tile_hist[e][tile], one wave per expert scanning its counts over tiles
// (exclusive) -> tile_base[e][tile] and totals[e], then the same placement
// reading those.  Positions rise with r inside each expert and do not
// depend on how workgroups are scheduled; integer sums make every path
// exact.
#include <cstdlib>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "place_core.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kChunksPerWave = 2;                       // three-kernel path
constexpr int kTile = kWaves * kChunksPerWave * kWave;  // 512 routes per tile
constexpr int kMaxE = 1024;
constexpr int kIdBits = 10;                             // bits of an expert id below kMaxE

// Ballots per peer mask: the bits of the largest id (fewer instructions for
// small E; the kernels take it as a template argument).
int id_bits(int32_t E) { return E <= 128 ? 7 : E <= 256 ? 8 : kIdBits; }
constexpr int kFusedMaxCounts = 32 * 1024;              // tiles x E, two-kernel path
constexpr int kFusedBatch = 16;                         // 16-byte loads in flight per thread
constexpr int kScanWaves = 16;                          // experts per scan workgroup
constexpr int kScanPrefetch = 8;                        // chunks of 64 tiles in registers

// This wave's CPW chunks of 64 routes starting at r0: issue_chunks issues
// the loads (clamped addresses, so that other loads can follow before any
// is used), check_chunks applies validity (routes past R and ids >= E
// become -1; the latter count as errors).
template <int CPW>
__device__ __forceinline__ void issue_chunks(const int32_t* __restrict__ ids, int64_t r0,
                                             int64_t R, int (&e)[CPW]) {
  const int lane = __lane_id();
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch) {
    const int64_t r = r0 + ch * kWave + lane;
    e[ch] = ids[r < R ? r : R - 1];
  }
}
template <int CPW>
__device__ __forceinline__ void check_chunks(int64_t r0, int64_t R, int E, int (&e)[CPW],
                                             int* err) {
  const int lane = __lane_id();
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
template <int CPW>
__device__ __forceinline__ void load_chunks(const int32_t* __restrict__ ids, int64_t r0,
                                            int64_t R, int E, int (&e)[CPW], int* err) {
  issue_chunks<CPW>(ids, r0, R, e);
  check_chunks<CPW>(r0, R, E, e, err);
}

// Count this wave's chunks into its LDS row (ids < 2^NB).
template <int CPW, int NB>
__device__ __forceinline__ void count_chunks(const int (&e)[CPW], int32_t* row) {
  const uint64_t below = lanemask_lt();
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch) {
    const uint64_t p = peer_mask<NB>(e[ch]);
    if (e[ch] >= 0 && (p & below) == 0) row[e[ch]] += __popcll(p);
  }
}

// Per-tile histogram; tile-major 16-bit counts (tile_hist[tile][e]) for the
// two-kernel path, expert-major 32-bit counts (tile_hist[e][tile]) for the
// tile scan.
template <int CPW, bool TILE_MAJOR, int NB>
__global__ __launch_bounds__(kThreads) void disp_hist_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int nt,
    std::conditional_t<TILE_MAJOR, hist_t, int32_t>* __restrict__ tile_hist,
    int32_t* __restrict__ dev_err) {
  __shared__ int32_t wh[kWaves][kMaxE];
  const int tid = threadIdx.x, wave = tid >> 6;
  int err = 0;
  int ev[CPW];
  load_chunks<CPW>(ids, (int64_t)blockIdx.x * (kWaves * CPW * kWave) + wave * (CPW * kWave), R,
                   E, ev, &err);
  for (int e = tid & 63; e < E; e += kWave) wh[wave][e] = 0;
  __syncthreads();
  count_chunks<CPW, NB>(ev, wh[wave]);
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    const int n = wh[0][e] + wh[1][e] + wh[2][e] + wh[3][e];
    if constexpr (TILE_MAJOR)
      tile_hist[(int64_t)blockIdx.x * E + e] = (hist_t)n;
    else
      tile_hist[(int64_t)e * nt + blockIdx.x] = n;
  }
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

// Sum over the lanes l' = l (mod G) of a wave, G = 1, 2, 4, ..., 64: DPP
// row rotations by 1, 2, 4, 8 fold the lanes of a 16-lane row, then
// permlane16_swap and permlane32_swap (each lane receives the other row's,
// or the other half's, value in one of the two results) fold the four rows.
template <int G>
__device__ __forceinline__ int lanes_sum_i32(int v) {
  if constexpr (G <= 1) v += dpp_i32<0x121>(v);  // row_ror:1
  if constexpr (G <= 2) v += dpp_i32<0x122>(v);  // row_ror:2
  if constexpr (G <= 4) v += dpp_i32<0x124>(v);  // row_ror:4
  if constexpr (G <= 8) v += dpp_i32<0x128>(v);  // row_ror:8
  if constexpr (G <= 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = r[0] + r[1];
  }
  if constexpr (G <= 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = r[0] + r[1];
  }
  return v;
}
template <int G>
__device__ __forceinline__ void lanes_sum_all(int (&a)[8], int (&b)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    a[c] = lanes_sum_i32<G>(a[c]);
    b[c] = lanes_sum_i32<G>(b[c]);
  }
}

// Stable placement of tiles of TILE routes by WAVES waves (one chunk of 64
// routes per wave up to 16 waves, then CPW chunks per wave; a wave past the
// tile holds no routes).  FUSED: totals and earlier-tile counts come from
// the tile-major histogram (tile_hist[nt][E] 16-bit counts, E % 8 == 0, nt *
// E <= kFusedMaxCounts); otherwise from tile_base[e][tile] and totals[e].
// NB: bits of the ballot peer masks (ids < 2^NB).  These kernels run for a
// few microseconds, so their cost is mostly latency: one round trip for all
// loads, straight-line code (branches and runtime loops cost instruction
// fetches), short LDS chains.
template <int WAVES, int TILE, bool FUSED, int NB>
__global__ __launch_bounds__(WAVES * kWave) void disp_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int nt,
    const hist_t* __restrict__ tile_hist, const int32_t* __restrict__ tile_base,
    const int32_t* __restrict__ totals, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    double* __restrict__ maxvio) {
  constexpr int NT = WAVES * kWave;
  static_assert(NT >= kMaxE / 4, "offsets scan: 4 experts per thread");
  __shared__ int32_t wh[WAVES][kMaxE];
  __shared__ int32_t off[kMaxE];
  __shared__ int32_t tot[FUSED ? kMaxE : 1];
  __shared__ int32_t wsum[WAVES];
  __shared__ int32_t wmax[WAVES];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tile = blockIdx.x;

  constexpr int CPW = TILE / (WAVES * kWave) > 0 ? TILE / (WAVES * kWave) : 1;
  static_assert(TILE % (CPW * kWave) == 0 && TILE / (CPW * kWave) <= WAVES, "tile shape");
  const bool routes = wave * CPW * kWave < TILE;  // wave-uniform
  int err = 0;
  int ev[CPW];
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch) ev[ch] = -1;
  const int64_t r0 = (int64_t)tile * TILE + wave * (CPW * kWave);
  if (tile < nt && routes) issue_chunks<CPW>(ids, r0, R, ev);  // checked after the counts' loads

  if constexpr (FUSED) {
    // Every workgroup reads all nt x E counts (from L2), so this read is
    // most of the kernel: neighbouring lanes load neighbouring 16 bytes of a
    // row (the loads coalesce) and the arithmetic per load is kept small.
    // A 16-byte load holds the counts of 8 experts (group g), two per dword.
    // The first RW waves read (RW * 64 threads, 16 rows each at 256 x 128
    // counts: the per-thread work after the loads is paid by few threads).
    // Thread (g, p), g = tid % G: rows p, p + P, p + 2P, ... (P = RW*64 / G
    // row lanes), B loads in flight.  Within a batch the dwords are added as
    // they are (at most 16 counts of at most 2048 per half: no carry
    // between the halves) and the sum over rows before this tile is the
    // running sum taken at the last such row (rows rise within a thread);
    // the halves are split once per batch.  When G divides 64 the lanes of
    // one group in a wave can be folded together in registers (one partial
    // set per wave); otherwise every row lane is a set.  J threads per
    // expert then add the NS sets from LDS.
    using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
    constexpr int B = kFusedBatch, RW = 4;
    static_assert(B * 2048 < 65536, "packed 16-bit sums per batch");
    const int G = E / 8, P = RW * kWave / G;  // G <= kMaxE / 8 <= RW * 64 / 2
    const int g = tid % G, p = tid / G;
    // fold in registers when few threads per expert would add the sets
    // (4-wave tiles); with 16 waves the LDS sum over 8 threads per expert is
    // cheaper (measured)
    const bool fold = (G & (G - 1)) == 0 && G <= kWave && 4 * E > NT;
    const int NS = fold ? RW : P, set = fold ? wave : p;
    int all[8], before[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) all[c] = before[c] = 0;
    if (p < P) {
      const u32x4* src = reinterpret_cast<const u32x4*>(tile_hist) + g;
      for (int t0 = p; t0 < nt; t0 += B * P) {
        u32x4 v[B];
#pragma unroll
        for (int i = 0; i < B; ++i)  // clamped rows: no branches between the loads
          v[i] = src[(int64_t)min(t0 + i * P, nt - 1) * G];
        u32x4 pa = {0, 0, 0, 0}, pb = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < B; ++i) {
          if (t0 + i * P < nt) pa += v[i];
          if (t0 + i * P < tile) pb = pa;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          all[2 * c] += (int)(pa[c] & 0xFFFFu);
          all[2 * c + 1] += (int)(pa[c] >> 16);
          before[2 * c] += (int)(pb[c] & 0xFFFFu);
          before[2 * c + 1] += (int)(pb[c] >> 16);
        }
      }
    }
    if (fold && wave < RW) {  // one branch on G, then straight-line code
      switch (G) {
        case 1: lanes_sum_all<1>(all, before); break;
        case 2: lanes_sum_all<2>(all, before); break;
        case 4: lanes_sum_all<4>(all, before); break;
        case 8: lanes_sum_all<8>(all, before); break;
        case 16: lanes_sum_all<16>(all, before); break;
        case 32: lanes_sum_all<32>(all, before); break;
        default: break;  // 64: one lane per group
      }
    }
    // set partial sums: [NS][pitch] each (NS * E * 2 <= WAVES * kMaxE); a
    // pitch of E + 1 where it fits spreads the J readers of one expert over
    // the LDS banks
    int J = 1;
    while (J < 16 && 2 * J <= NS && 2 * E * J <= NT) J *= 2;
    const int pitch = J > 1 && NS * (E + 1) * 2 <= WAVES * kMaxE ? E + 1 : E;
    int32_t* part_all = &wh[0][0];
    int32_t* part_before = part_all + NS * pitch;
    if (fold ? wave < RW && lane < G : p < P)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        part_all[set * pitch + 8 * g + c] = all[c];
        part_before[set * pitch + 8 * g + c] = before[c];
      }
    __syncthreads();
    for (int i0 = 0; i0 < E * J; i0 += NT) {  // the same trip count in every lane
      const int idx = i0 + tid, e = idx / J, j = idx % J;
      int a = 0, b = 0;
      if (e < E)
        for (int s2 = j; s2 < NS; s2 += J) {
          a += part_all[s2 * pitch + e];
          b += part_before[s2 * pitch + e];
        }
      a = group_sum_i32(a, J);
      b = group_sum_i32(b, J);
      if (e < E && j == 0) {
        tot[e] = a;
        off[e] = b;
      }
    }
    __syncthreads();
  }

  if (tile < nt) check_chunks<CPW>(r0, R, E, ev, &err);

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
  if (blockIdx.x == 0 && maxvio) {  // the busiest expert, for the load statistic
    const uint32_t mx = wave_max_u32((uint32_t)max(max(t4[0], t4[1]), max(t4[2], t4[3])));
    if (lane == 0) wmax[wave] = (int32_t)mx;
  }
  for (int e = lane; e < E; e += kWave) wh[wave][e] = 0;
  __syncthreads();
  if (blockIdx.x == 0 && maxvio && tid == 0) {
    // MaxVio = max_e count_e / (R / E) - 1 ("I modelli MoE open hanno router
    // opposti", loss-free balancing paragraph), 0 without routes
    int64_t R_all = 0;
    int32_t mx = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      R_all += wsum[w];
      mx = max(mx, wmax[w]);
    }
    *maxvio = R_all > 0 ? (double)mx / ((double)R_all / (double)E) - 1.0 : 0.0;
  }
  int base = inc - s;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) base += w < wave ? wsum[w] : 0;  // straight-line
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
  if (blockIdx.x == 0 && tid == NT - 1) offsets[E] = base;
  if (tile >= nt) return;  // only when there are no routes at all

  // count this wave's chunks into its row, keeping each route's offset in
  // the wave (the expert's count in earlier chunks plus the peers below it)
  int32_t* row = wh[wave];
  int in_wave[CPW];
  {
    const uint64_t below = lanemask_lt();
#pragma unroll
    for (int ch = 0; ch < CPW; ++ch) {
      const int e = ev[ch];
      const uint64_t p = peer_mask<NB>(e);
      in_wave[ch] = 0;
      if (e >= 0) {
        const int start = row[e];
        in_wave[ch] = start + __popcll(p & below);
        if ((p & below) == 0) row[e] = start + __popcll(p);
      }
    }
  }
  __syncthreads();
  // per-wave starting positions of each expert inside this tile
  for (int e = tid; e < E; e += NT) {
    int b = FUSED ? off[e] : off[e] + tile_base[(int64_t)e * nt + tile];
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const int c = wh[w][e];
      wh[w][e] = b;
      b += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch) {
    const int64_t r = r0 + ch * kWave + lane;
    const int e = ev[ch];
    const int pos = e >= 0 ? row[e] + in_wave[ch] : -1;
    if (routes && r < R) {
      if (inv) inv[r] = pos;
      if (pos >= 0 && pos < R) perm[pos] = (int32_t)r;
    }
  }
}

// Chunks per wave for the two-kernel path: the smallest tile that keeps the
// histogram within kFusedMaxCounts, or 0 (three-kernel path).
int fused_cpw(int64_t R, int32_t E) {
  if (E % 8 != 0 || std::getenv("MOE_DISPATCH_UNFUSED")) return 0;  // tuning: 3 kernels
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

// The placement kernel for tiles of TILE routes: one chunk per wave up to 16
// waves, then more chunks per wave.
template <int TILE, bool FUSED>
hipError_t launch_scatter(const int32_t* ids, int64_t R, int32_t E, int nt,
                          const hist_t* tile_hist, const int32_t* tile_base,
                          const int32_t* totals, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, double* maxvio, hipStream_t stream) {
  constexpr int W = TILE / kWave >= 16 ? 16 : TILE / kWave;
  // with no routes (three-kernel path only) one workgroup writes zero
  // counts and offsets
  auto go = [&](auto kernel) {
    return launch(kStageDispScatter, kernel, dim3(nt > 0 ? nt : 1), dim3(W * kWave), stream,
                  ids, R, E, nt, tile_hist, tile_base, totals, counts, offsets, perm, inv,
                  maxvio);
  };
  switch (id_bits(E)) {
    case 7: return go(disp_scatter_kernel<W, TILE, FUSED, 7>);
    case 8: return go(disp_scatter_kernel<W, TILE, FUSED, 8>);
    default: return go(disp_scatter_kernel<W, TILE, FUSED, kIdBits>);
  }
}

// The histogram kernel (tiles of kWaves x CPW x 64 routes).
template <int CPW, bool TILE_MAJOR>
hipError_t launch_hist(const int32_t* ids, int64_t R, int32_t E, int nt,
                       std::conditional_t<TILE_MAJOR, hist_t, int32_t>* tile_hist,
                       int32_t* dev_err, hipStream_t stream) {
  auto go = [&](auto kernel) {
    return launch(kStageDispHist, kernel, dim3(nt), dim3(kThreads), stream, ids, R, E, nt,
                  tile_hist, dev_err);
  };
  switch (id_bits(E)) {
    case 7: return go(disp_hist_kernel<CPW, TILE_MAJOR, 7>);
    case 8: return go(disp_hist_kernel<CPW, TILE_MAJOR, 8>);
    default: return go(disp_hist_kernel<CPW, TILE_MAJOR, kIdBits>);
  }
}

hipError_t launch_placement(int tile_routes, const int32_t* ids, int64_t R, int32_t E, int nt,
                            const hist_t* tile_hist, int32_t* counts, int32_t* offsets,
                            int32_t* perm, int32_t* inv, double* maxvio,
                            hipStream_t stream) {
  switch (tile_routes) {
#define MOE_PLACE(T_)                                                                        \
  case T_:                                                                                   \
    return launch_scatter<T_, true>(ids, R, E, nt, tile_hist, nullptr, nullptr, counts, \
                                    offsets, perm, inv, maxvio, stream);
    MOE_PLACE(256)
    MOE_PLACE(512)
    MOE_PLACE(1024)
    MOE_PLACE(2048)
#undef MOE_PLACE
    default: return hipErrorInvalidValue;
  }
}

template <int CPW>
hipError_t launch_fused(const int32_t* ids, int64_t R, int32_t E, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv, double* maxvio,
                        hist_t* tile_hist, int32_t* dev_err, hipStream_t stream) {
  constexpr int kRoutes = kWaves * CPW * kWave;
  const int nt = (int)((R + kRoutes - 1) / kRoutes);
  hipError_t e = launch_hist<CPW, true>(ids, R, E, nt, tile_hist, dev_err, stream);
  if (e != hipSuccess) return e;
  return launch_placement(kRoutes, ids, R, E, nt, tile_hist, counts, offsets, perm, inv,
                          maxvio, stream);
}

// Capacity limit on a dispatch (top-1 routing with a Switch-style capacity;
// the rule taken: each expert keeps its first C routes in route order).  The
// stable dispatch puts route r of expert e at inv[r] = offsets[e] + (its rank
// among e's routes), so slot[r] = e*C + rank when the rank is below C, else
// -1.  Workgroup 0 also writes kept[e] = min(count_e, C) and the number of
// routes over capacity.  Ids and positions are re-checked, so inputs that do
// not come from one dispatch cannot lead outside the arrays.
__global__ __launch_bounds__(kThreads) void disp_capacity_kernel(
    const int32_t* __restrict__ ids, int64_t R, int32_t E, int32_t C,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ inv,
    int32_t* __restrict__ slot, int32_t* __restrict__ kept, int32_t* __restrict__ dropped) {
  const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (r < R) {
    const int32_t p = inv[r];
    int32_t s = -1;
    if (p >= 0) {
      const int32_t e = ids[r];
      if (e >= 0 && e < E) {
        const int32_t q = p - offsets[e];
        if (q >= 0 && q < C) s = e * C + q;
      }
    }
    slot[r] = s;
  }
  if (blockIdx.x == 0) {  // the whole workgroup: the barrier below is uniform
    __shared__ int32_t part[kWaves];
    int32_t over = 0;
    for (int e = threadIdx.x; e < E; e += kThreads) {
      const int32_t n = offsets[e + 1] - offsets[e];
      kept[e] = min(n, C);
      over += max(n - C, 0);
    }
    over = wave_sum_i32(over);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = over;
    __syncthreads();
    if (threadIdx.x == 0) *dropped = part[0] + part[1] + part[2] + part[3];
  }
}

// Placement from tile histograms plus super-tile sums: one workgroup per G
// tiles (place_super_tiles).
template <int CPW, int NB>
__global__ __launch_bounds__(kPlaceWaves * kWave) void disp_place_super_kernel(
    const int32_t* __restrict__ ids, int64_t R, int E, int nt, int TR, int S, int G,
    const hist_t* __restrict__ tile_hist, const int32_t* __restrict__ super_sum,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, double* __restrict__ maxvio) {
  __shared__ PlaceLds sh;
  place_super_tiles<CPW, NB>((int)blockIdx.x, ids, R, E, nt, TR, S, G, tile_hist, super_sum,
                             counts, offsets, perm, inv, maxvio, sh);
}

}  // namespace

hipError_t launch_capacity(const int32_t* ids, int64_t R, int32_t E, int32_t C,
                           const int32_t* offsets, const int32_t* inv, int32_t* slot,
                           int32_t* kept, int32_t* dropped, hipStream_t stream) {
  const int64_t blocks = R > 0 ? (R + kThreads - 1) / kThreads : 1;
  return launch(kStageCapacity, disp_capacity_kernel, dim3((uint32_t)blocks), dim3(kThreads),
                stream, ids, R, E, C, offsets, inv, slot, kept, dropped);
}

bool dispatch_hist_ok(int64_t R, int32_t E, int32_t tile_routes) {
  if (R <= 0 || E % 8 != 0 || E > kMaxE) return false;
  if (tile_routes != 256 && tile_routes != 512 && tile_routes != 1024 && tile_routes != 2048)
    return false;
  return (R + tile_routes - 1) / tile_routes * E <= kFusedMaxCounts;
}

hipError_t launch_dispatch_from_hist(const int32_t* ids, int64_t R, int32_t E,
                                     int32_t* counts, int32_t* offsets, int32_t* perm,
                                     int32_t* inv, double* maxvio, const hist_t* tile_hist,
                                     int32_t tile_routes, hipStream_t stream) {
  if (!dispatch_hist_ok(R, E, tile_routes)) return hipErrorInvalidValue;
  const int nt = (int)((R + tile_routes - 1) / tile_routes);
  return launch_placement(tile_routes, ids, R, E, nt, tile_hist, counts, offsets,
                          perm, inv, maxvio, stream);
}

bool dispatch_super_ok(int64_t R, int32_t E, int32_t tile_routes) {
  return R > 0 && R <= 2147483647 && E >= 1 && E <= kMaxE && tile_routes >= 1 &&
         tile_routes <= 2 * kPlaceWaves * kWave;
}

// Tiles per placement workgroup: small tiles are placed two (or more) to a
// workgroup while there are more tiles than CUs and their routes fit the
// workgroup's two chunks per lane.
// Measured (placement us): DeepSeek-V4-like, 512 tiles of 192 routes, 9.35
// at one tile per workgroup, 7.1-7.2 at two or four, 8.2 at eight; the
// Qwen3- and DeepSeek-V3-like shapes (<= 256 tiles) slower at four and eight.
int place_group(int64_t nt, int32_t tile_routes) {
  int G = 1;
  if (const char* env = std::getenv("MOE_PLACE_GROUP")) {  // tuning: 1, 2, 4, 8
    const int want = std::atoi(env);
    while (G < want && 2 * G * tile_routes <= 2 * kPlaceWaves * kWave) G *= 2;
    return G;
  }
  while (nt > 256 * (int64_t)G && 2 * G * tile_routes <= 2 * kPlaceWaves * kWave) G *= 2;
  return G;
}

int dispatch_super_size(int64_t R, int32_t tile_routes) {
  const int64_t nt = (R + tile_routes - 1) / tile_routes;
  int S = 1;
  while ((int64_t)S * S < nt) ++S;  // about sqrt(nt): ns + S rows per workgroup
  const int G = place_group(nt, tile_routes);
  return (S + G - 1) / G * G;       // a workgroup's tiles share one super tile
}

hipError_t launch_dispatch_from_super(const int32_t* ids, int64_t R, int32_t E,
                                      int32_t* counts, int32_t* offsets, int32_t* perm,
                                      int32_t* inv, double* maxvio, const hist_t* tile_hist,
                                      const int32_t* super_sum, int32_t tile_routes,
                                      hipStream_t stream) {
  if (!dispatch_super_ok(R, E, tile_routes)) return hipErrorInvalidValue;
  const int nt = (int)((R + tile_routes - 1) / tile_routes);
  const int S = dispatch_super_size(R, tile_routes);
  const int G = place_group(nt, tile_routes);
  auto go = [&](auto kernel) {
    return launch(kStageDispScatter, kernel, dim3((nt + G - 1) / G), dim3(kPlaceWaves * kWave),
                  stream, ids, R, E, nt, (int)tile_routes, S, G, tile_hist, super_sum, counts,
                  offsets, perm, inv, maxvio);
  };
  const bool two = G * tile_routes > kPlaceWaves * kWave;
  switch (id_bits(E)) {
    case 7: return two ? go(disp_place_super_kernel<2, 7>) : go(disp_place_super_kernel<1, 7>);
    case 8: return two ? go(disp_place_super_kernel<2, 8>) : go(disp_place_super_kernel<1, 8>);
    default:
      return two ? go(disp_place_super_kernel<2, kIdBits>)
                 : go(disp_place_super_kernel<1, kIdBits>);
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
    return (size_t)(nt * E * (int64_t)sizeof(hist_t));
  }
  const int64_t nt = (R + kTile - 1) / kTile;
  return (size_t)((2 * nt + 1) * (int64_t)E * sizeof(int32_t));
}

hipError_t launch_dispatch(const int32_t* ids, int64_t R, int32_t E,
                           int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv, double* maxvio, void* workspace,
                           int32_t* dev_err, hipStream_t stream) {
  int32_t* ws = static_cast<int32_t*>(workspace);
  if (R > 0) {
    switch (fused_cpw(R, E)) {
      case 2:
        return launch_fused<2>(ids, R, E, counts, offsets, perm, inv, maxvio,
                                 static_cast<hist_t*>(workspace), dev_err, stream);
      case 4:
        return launch_fused<4>(ids, R, E, counts, offsets, perm, inv, maxvio,
                                 static_cast<hist_t*>(workspace), dev_err, stream);
      case 8:
        return launch_fused<8>(ids, R, E, counts, offsets, perm, inv, maxvio,
                                 static_cast<hist_t*>(workspace), dev_err, stream);
      default: break;
    }
  }
  const int nt = (int)((R + kTile - 1) / kTile);
  int32_t* tile_hist = ws;
  int32_t* tile_base = tile_hist + (int64_t)nt * E;
  int32_t* totals = tile_base + (int64_t)nt * E;
  hipError_t e;
  if (nt > 0) {
    e = launch_hist<kChunksPerWave, false>(ids, R, E, nt, tile_hist, dev_err, stream);
    if (e != hipSuccess) return e;
    e = launch(kStageDispScan, disp_tile_scan_kernel, dim3((E + kScanWaves - 1) / kScanWaves),
               dim3(kScanWaves * kWave), stream, (const int32_t*)tile_hist, nt, E, tile_base,
               totals);
    if (e != hipSuccess) return e;
  }
  // with no routes the scatter kernel runs one workgroup that only writes
  // zero counts and offsets (totals is not read then)
  return launch_scatter<kTile, false>(ids, R, E, nt, nullptr, tile_base,
                                      nt > 0 ? totals : nullptr, counts, offsets, perm, inv,
                                      maxvio, stream);
}

}  // namespace moe
