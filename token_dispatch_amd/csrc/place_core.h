// Stable placement of dispatch tiles from per-tile counts plus super-tile
// sums, as a device function of one 16-wavefront workgroup: the placement
// kernel of the dispatch runs it once per workgroup, and the hash layer's
// dot-product kernel runs it on the workgroups that have no slice of d to
// work on (the dispatch of table ids needs no dot product).  Internal to the
// HIP library.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kPlaceWaves = 16;
constexpr int kPlaceMaxE = 1024;  // experts of a placement (MOE_MAX_EXPERTS)
constexpr int kPlaceIdBits = 10;  // bits of an expert id below kPlaceMaxE

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
// Sum over aligned groups of Q lanes (Q = 1, 2, 4, 8 or 16, the same in the
// whole wave) inside 16-lane DPP rows: quad_perm [1,0,3,2] and [2,3,0,1],
// then row_half_mirror and row_mirror pair each partial sum with the one
// of the other half; every lane of a group ends with the group's sum.
__device__ __forceinline__ int group_sum_i32(int v, int Q) {
  if (Q >= 2) v += dpp_i32<0xB1>(v);
  if (Q >= 4) v += dpp_i32<0x4E>(v);
  if (Q >= 8) v += dpp_i32<0x141>(v);
  if (Q >= 16) v += dpp_i32<0x140>(v);
  return v;
}

// LDS of one placement (73.9 KB).
struct PlaceLds {
  int32_t wh[kPlaceWaves][kPlaceMaxE];
  int32_t tot[kPlaceMaxE];
  int32_t off[kPlaceMaxE];
  int32_t wsum[kPlaceWaves];
  int32_t wmax[kPlaceWaves];
};

// Placement from tile histograms plus super-tile sums ("reduce, then
// scan").  The routing kernel that selected tile t's routes wrote the tile's
// 16-bit histogram hist[t][E] and added it into super_sum[t / S][E] (int32
// integer atomics, order-independent; the array was zeroed by the gate kernel
// earlier in the same call).  The workgroup placing tile t therefore reads
// the ns = ceil(nt / S) super rows -- every expert's total, and its count in
// super tiles before tile t's -- and the at most S - 1 tile rows before it
// inside its own super tile: (ns + S) * E counts instead of the nt * E the
// all-counts kernel reads.
// Tiles hold TR routes; placement w places the G tiles [w*G, w*G + G) (G *
// TR up to 64 * kPlaceWaves * CPW routes; S is a multiple of G, so they lie
// in one super tile and the rows before the first of them are the rows
// before each), one chunk of 64 routes per wave and chunk slot, 16 waves.
// J threads per expert (adjacent lanes) split its rows and add their sums
// with DPP.
//
// Placement w == 0 also writes counts, offsets and MaxVio.  With S = 1 the
// super rows are the tiles' own rows (int32) and no tile_hist row is read:
// every expert's total and its count before tile t come from all nt rows.
// The caller's 16 wavefronts all enter; LDS is reused only after a barrier.
template <int CPW, int NB>
__device__ __forceinline__ void place_super_tiles(
    int w, const int32_t* __restrict__ ids, int64_t R, int E, int nt, int TR, int S, int G,
    const hist_t* __restrict__ tile_hist, const int32_t* __restrict__ super_sum,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, double* __restrict__ maxvio, PlaceLds& sh) {
  constexpr int NT = kPlaceWaves * kWave;
  static_assert(NT >= kPlaceMaxE / 4, "offsets scan: 4 experts per thread");
  int32_t(*wh)[kPlaceMaxE] = sh.wh;
  int32_t* tot = sh.tot;
  int32_t* off = sh.off;
  int32_t* wsum = sh.wsum;
  int32_t* wmax = sh.wmax;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tile = w * G;  // this placement's first tile (G tiles each)
  const int TRG = TR * G;  // its routes
  const int64_t tbase = (int64_t)tile * TR;

  // this wave's chunks of the tile: slot c = wave * CPW + ch covers routes
  // tbase + c * 64 + lane while c * 64 + lane < TR (loads issued first)
  int ev[CPW];
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch) {
    const int c = wave * CPW + ch;
    const int64_t r = tbase + c * kWave + lane;
    const bool mine = c * kWave + lane < TRG && r < R;
    ev[ch] = ids[mine ? r : 0];
    if (!mine) ev[ch] = -1;
  }

  // every expert's total and its count before this tile: J threads per
  // expert (adjacent lanes) split its super rows and tile rows, loads issued
  // in batches, sums added with DPP
  int J = 1;
  while (J < 16 && 2 * J * E <= NT) J *= 2;
  const int e_of = tid / J, j = tid % J;
  const int st = tile / S, ns = (nt + S - 1) / S;
  int a = 0, b = 0;
  if (e_of < E) {
    constexpr int B = 8;  // loads in flight per thread
    for (int s0 = j; s0 < ns; s0 += B * J) {
      int v[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int sr = s0 + i * J;
        v[i] = sr < ns ? super_sum[(int64_t)sr * E + e_of] : 0;
      }
#pragma unroll
      for (int i = 0; i < B; ++i) {
        a += v[i];
        b += s0 + i * J < st ? v[i] : 0;
      }
    }
    for (int u0 = st * S + j; u0 < tile; u0 += B * J) {
      int v[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int u = u0 + i * J;
        v[i] = u < tile ? (int)tile_hist[(int64_t)u * E + e_of] : 0;
      }
#pragma unroll
      for (int i = 0; i < B; ++i) b += v[i];
    }
  }
  a = group_sum_i32(a, J);
  b = group_sum_i32(b, J);
  if (e_of < E && j == 0) {
    tot[e_of] = a;
    off[e_of] = b;
  }
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch)
    if (ev[ch] >= E) ev[ch] = -1;  // (routing kernels write ids below E or -1)
  __syncthreads();

  // offsets: exclusive scan of the totals over experts (4 experts per thread)
  int t4[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    t4[i] = e < E ? tot[e] : 0;
    s += t4[i];
  }
  const int inc = wave_incl_scan_i32(s);
  if (lane == 63) wsum[wave] = inc;
  if (w == 0 && maxvio) {
    const uint32_t mx = wave_max_u32((uint32_t)max(max(t4[0], t4[1]), max(t4[2], t4[3])));
    if (lane == 0) wmax[wave] = (int32_t)mx;
  }
  for (int e = lane; e < E; e += kWave) wh[wave][e] = 0;
  __syncthreads();
  if (w == 0 && maxvio && tid == 0) {
    // MaxVio = max_e count_e / (R / E) - 1 ("I modelli MoE open hanno router
    // opposti", loss-free balancing paragraph), 0 without routes
    int64_t R_all = 0;
    int32_t mx = 0;
#pragma unroll
    for (int w = 0; w < kPlaceWaves; ++w) {
      R_all += wsum[w];
      mx = max(mx, wmax[w]);
    }
    *maxvio = R_all > 0 ? (double)mx / ((double)R_all / (double)E) - 1.0 : 0.0;
  }
  int base = inc - s;
#pragma unroll
  for (int w = 0; w < kPlaceWaves; ++w) base += w < wave ? wsum[w] : 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    if (e < E) {
      off[e] = base + off[e];  // only this thread touches entry e here
      if (w == 0) {
        counts[e] = t4[i];
        offsets[e] = base;
      }
    }
    base += t4[i];
  }
  if (w == 0 && tid == NT - 1) offsets[E] = base;

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
    int bb = off[e];
#pragma unroll
    for (int w = 0; w < kPlaceWaves; ++w) {
      const int c = wh[w][e];
      wh[w][e] = bb;
      bb += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch) {
    const int c = wave * CPW + ch;
    const int64_t r = tbase + c * kWave + lane;
    const int e = ev[ch];
    if (c * kWave + lane < TRG && r < R) {
      const int pos = e >= 0 ? row[e] + in_wave[ch] : -1;
      if (inv) inv[r] = pos;
      if (pos >= 0 && pos < R) perm[pos] = (int32_t)r;
    }
  }
}

}  // namespace
}  // namespace moe
