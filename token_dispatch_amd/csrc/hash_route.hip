// Hash routing on gfx950 (ferrox_moe crate docs, route_hash: in a
// DeepSeek-V4 hash layer the expert ids are the token id's row of a fixed
// token-id -> expert-id table, with no learned selection and no selection
// bias).
//
// Lanes j < k of a token's segment gather the table row (validating the
// token id and every entry), then, when weights are wanted, lane j takes the
// logit of slot j and the segment turns the k logits into weights with the
// layer's score function.  The logits come from
//  * the method's own work, k dot products per token (bf16, k <= 8, aligned
//    rows): hash_dots_kernel holds one slice of W's columns for every
//    expert in LDS and streams the matching slice of every token's x row
//    through it, so x is read once from HBM and W once per workgroup; the
//    per-slice partial dot products are added in slice order by the hash
//    kernel (several tokens per wavefront, optionally the dispatch's tile
//    histograms).  Gathering each token's k rows of W instead would re-read
//    them from L2 for every token, about 64 times the dense gate's L2
//    traffic at E = 384, k = 6;
//  * or the gate contraction of every expert (the tiled matrix-core kernel,
//    into a workspace; NSPLIT K-split partial arrays added in order) for the
//    other shapes;
//  * or, with no workspace, k dot products of length d computed here (one
//    wavefront per token, the lanes striding over d with 16-byte loads).
#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <type_traits>
#include <unordered_map>

#include "device_common.h"
#include "kernels.h"
#include "place_core.h"
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

// k dot products per token over slices of d: the hash layer's own work.
// Workgroup (s, c) holds columns [s*SL, s*SL + SL) of every expert's W row
// in LDS (rows padded by one 16-byte piece to spread the banks) and passes
// the tokens of chunk c through them in tiles; the slices of one chunk are
// neighbours in launch order, so each x row is read by all of them at about
// the same time.  A wavefront takes 64 / L tokens per tile: lane r of a
// token loads pieces r, r + L, ... (16 bytes each) of the token's x slice
// straight into registers, PF tiles ahead, and forms partial sums for the
// token's k slots with bf16 dot2 instructions (fp32 accumulation) against
// the W rows in LDS; the L partials of each slot are added with DPP moves,
// giving part[s][t*k + j] = slice s's share of x[t] . W[ids[t*k + j]] (0
// for ids < 0).  The token's ids are loaded once per group (lane r holds
// slots r, r + L, ...) and swizzled to its lanes.  Every x byte is read
// once and each workgroup reads one slice of W.
// Measured on the DeepSeek-V4-like shape (16384 tokens, d 7168, 384
// experts, k 6), kernel time in us: x staged through LDS with a token's
// lanes splitting its slots 64.4; one token per lane with x in registers
// 97.7; the pieces split over 4, 8 or 16 lanes 61.9, 59.5, 71.9 at 16
// wavefronts per workgroup (8 lanes at 8 wavefronts: 65.7); 192- and
// 128-column slices 58.7-60.6 and 59.4-60.3, 112 columns (rows not cut at
// 128-byte lines) 68.8; the (slice, token) pairs cut into equal ranges for
// every CU instead of slices x chunks (which leaves 28-32 CUs idle) 64.7,
// as the slices then read each x row at different times.
// zero[0 .. zero_words): the super-tile sums the hash kernel adds into,
// cleared here (each workgroup a share) as the gate kernel does on the
// other paths.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// acc + the dot product of two 16-byte pieces of 8 bf16 (four dot2 steps).
// The whole vectors are bit-cast: a bit cast of a subscripted 32-bit element
// compiled to element 0 for every subscript with this compiler.
__device__ __forceinline__ float dot8(u32x4_t a, u32x4_t b, float acc) {
  const bf16x8_t p = __builtin_bit_cast(bf16x8_t, a), q = __builtin_bit_cast(bf16x8_t, b);
  acc = __builtin_amdgcn_fdot2_f32_bf16(p.s01, q.s01, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(p.s23, q.s23, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(p.s45, q.s45, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(p.s67, q.s67, acc, false);
}

constexpr int kDotMaxK = 8;

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>());
  }
}

// Sum over the aligned groups of L lanes (L = 1, 2, 4, 8 or 16) with DPP
// moves: a butterfly whose every step adds two equal-size halves, so each
// lane of a group ends with the same sum.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  auto mv = [](float a, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a),
                                                      decltype(ctrl)::value, 0xF, 0xF, false));
  };
  if constexpr (L >= 2) v += mv(v, std::integral_constant<int, 0xB1>());   // lane ^ 1
  if constexpr (L >= 4) v += mv(v, std::integral_constant<int, 0x4E>());   // lane ^ 2
  if constexpr (L >= 8) v += mv(v, std::integral_constant<int, 0x141>());  // 7 - lane in 8
  if constexpr (L >= 16) v += mv(v, std::integral_constant<int, 0x140>()); // 15 - lane in 16
  return v;
}

// PLACE: a one-dimensional grid of ns x chunks slice workgroups (slice =
// block % ns) followed by place.n_place workgroups that place the dispatch
// tiles t = w, w + n_place, ... of the table ids (place_super_tiles with
// every tile's own row, S = 1) and stream no x.
// KC > 0: k == KC, known when compiling -- the slots are then straight-line
// code that the compiler interleaves (their LDS reads, dot products and DPP
// sums); with k known only at run time each slot sits behind its own branch
// (DeepSeek-V4-like layer, k = 6: 58.0-58.6 -> 56.1-56.2 us).
template <int SL, int EMAX, int L, int NW, int PF, bool PLACE = false, int KC = 0>
__global__ __launch_bounds__(NW * kWave) void hash_dots_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ ids, int T, int d, int E, int k, int64_t per,
    float* __restrict__ part, int32_t* __restrict__ zero, int zero_words, int ns,
    BesidePlace place) {
  constexpr int PC = SL / 8;                     // 16-byte pieces per row slice
  // Pieces per LDS row.  The two tokens of a 16-lane LDS cycle read 128 bytes
  // each from two unrelated W rows: rows of an odd number of 128-byte lines
  // start in alternate halves of the 64 banks, so only rows of the same
  // parity collide (a one-piece pad made nearly every pair overlap: 54 % of
  // the kernel's LDS cycles were bank conflicts on the DeepSeek-V4-like
  // layer); other widths keep the pad.
  constexpr int PITCH = (PC % 16 == 8) ? PC : PC + 1;
  constexpr int TPW = kWave / L;                 // tokens per wave and tile
  constexpr int TPT = NW * TPW;                  // tokens per tile
  constexpr int CPL = (PC + L - 1) / L;          // pieces per lane
  constexpr int OPL = (kDotMaxK + L - 1) / L;    // output slots per lane
  constexpr int EPL = (kDotMaxK + L - 1) / L;    // ids per lane
  static_assert(SL % 8 == 0 && (L & (L - 1)) == 0 && L >= 2 && L <= 16, "shapes");
  __shared__ u32x4_t wl[EMAX * PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (PLACE) {
    const int n_dots = place.n_dots;
    static_assert(sizeof(PlaceLds) <= sizeof(wl) && NW == kPlaceWaves, "placement workgroup");
    if ((int)blockIdx.x >= n_dots) {  // uniform: a placement workgroup
      PlaceLds& sh = *reinterpret_cast<PlaceLds*>(wl);
      for (int t = (int)blockIdx.x - n_dots; t < place.nt; t += place.n_place) {
        place_super_tiles<kBesideTile / (kPlaceWaves * kWave), kPlaceIdBits>(
            t, place.ids, place.R, place.E, place.nt, kBesideTile, 1, 1, nullptr, place.rows,
            place.counts, place.offsets, place.perm, place.inv, place.maxvio, sh);
        __syncthreads();  // LDS reused by the next tile
      }
      return;
    }
  }
  if (zero_words > 0) {
    const int n = (int)(gridDim.x * gridDim.y);
    const int each = (zero_words + n - 1) / n;
    const int beg = (int)(blockIdx.y * gridDim.x + blockIdx.x) * each;
    const int end = min(beg + each, zero_words);
    for (int i = beg + tid; i < end; i += NW * kWave) zero[i] = 0;
  }
  const int64_t Rk = (int64_t)T * k;
  const u32x4_t z4 = {0u, 0u, 0u, 0u};
  const int it = lane / L, r = lane % L;

  const int sl = PLACE ? (int)blockIdx.x % ns : (int)blockIdx.x;  // slice of d
  const int64_t c0 = (int64_t)(PLACE ? (int)blockIdx.x / ns : (int)blockIdx.y) * per;  // chunk
  const int64_t c1 = min((int64_t)T, c0 + per);
  if (c0 >= c1) return;  // uniform: a chunk past the last token
  const int col0 = sl * SL;
  const int ntiles = (int)((c1 - c0 + TPT - 1) / TPT);
  float* __restrict__ out = part + (int64_t)sl * Rk;

  auto tok = [&](int i) { return c0 + (int64_t)i * TPT + wave * TPW + it; };
  // Loads without branches (a branch around each load made the compiler
  // wait for every load in flight at each step): addresses past the range
  // or the row are clamped into it and the values are discarded at use.
  auto load_x = [&](int i, u32x4_t (&v)[CPL]) {
    const int64_t t = min(tok(i), c1 - 1);
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int col = min(col0 + (q * L + r) * 8, d - 8);
      v[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + t * d + col));
    }
  };
  auto load_e = [&](int i, int (&ev)[EPL]) {
    const int64_t t = min(tok(i), c1 - 1);
#pragma unroll
    for (int j = 0; j < EPL; ++j) ev[j] = ids[t * k + min(j * L + r, k - 1)];
  };

  // tiles 0 .. PF-1 in flight while the W slice is loaded; a ring of PF + 1
  // register slots
  constexpr int RS = PF + 1;
  u32x4_t xr[RS][CPL];
  int er[RS][EPL];
  static_for<PF>([&](auto q) {
    constexpr int Q = decltype(q)::value;
    load_x(Q, xr[Q]);
    load_e(Q, er[Q]);
  });
  for (int i = tid; i < E * PC; i += NW * kWave) {
    const int e = i / PC, pc = i % PC, col = col0 + pc * 8;
    wl[e * PITCH + pc] =
        col < d ? *reinterpret_cast<const u32x4_t*>(W + (int64_t)e * d + col) : z4;
  }
  __syncthreads();

  // tile i from ring slot Q; the loads of tile i + PF go to slot (Q + PF) % RS
  auto step = [&](int i, auto q) {
    constexpr int Q = decltype(q)::value;
    constexpr int N = (Q + PF) % RS;
    load_x(i + PF, xr[N]);
    load_e(i + PF, er[N]);
    float acc[kDotMaxK];
    static_for<kDotMaxK>([&](auto mm) {
      constexpr int m = decltype(mm)::value;
      acc[m] = 0.f;
      if (m < (KC > 0 ? KC : k)) {  // uniform
        // slot m's id from lane m % L of the group (ds_swizzle bit mode:
        // the and-mask keeps the group's first lane, the or-mask adds m % L)
        constexpr int kSwz = (0x1F & ~(L - 1)) | ((m % L) << 5);
        const int e = __builtin_amdgcn_ds_swizzle(er[Q][m / L], kSwz);
        const bool live = e >= 0 && e < E;
        const int row = live ? e * PITCH : 0;
#pragma unroll
        for (int qq = 0; qq < CPL; ++qq) {
          const int pc = qq * L + r;
          const u32x4_t xv = (pc < PC && col0 + pc * 8 < d) ? xr[Q][qq] : z4;
          acc[m] = dot8(xv, wl[row + min(pc, PC - 1)], acc[m]);
        }
        acc[m] = group_sum<L>(acc[m]);
        if (!live) acc[m] = 0.f;
      }
    });
    const int64_t t = tok(i);
    if (t < c1) {
#pragma unroll
      for (int o = 0; o < OPL; ++o) {
        float v = acc[o * L];
#pragma unroll
        for (int rr = 1; rr < L; ++rr)
          if (o * L + rr < kDotMaxK && r == rr) v = acc[o * L + rr];
        if (o * L + r < k) out[t * k + o * L + r] = v;
      }
    }
  };
  for (int i = 0; i < ntiles; i += RS)
    static_for<RS>([&](auto q) {
      if (i + decltype(q)::value < ntiles) step(i + decltype(q)::value, q);
    });
}

// The table's expert ids, one thread per route (checked; -1 for a bad token
// id or entry, no error count: the hash kernel that follows counts them).
__global__ __launch_bounds__(256) void hash_ids_kernel(const int32_t* __restrict__ token_ids,
                                                       const int32_t* __restrict__ tid2eid,
                                                       int32_t vocab, int64_t R, int k, int E,
                                                       int32_t* __restrict__ ids) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  const int v = token_ids[r / k];
  int e = -1;
  if (v >= 0 && v < vocab) {
    e = tid2eid[(int64_t)v * k + r % k];
    if (e < 0 || e >= E) e = -1;
  }
  ids[r] = e;
}

// The table's expert ids as hash_ids_kernel writes them, for dispatch tiles
// of kBesideTile routes (one 16-wavefront workgroup per tile, two chunks of
// 64 routes per wavefront), plus each tile's count of every expert:
// rows[tile][e] (int32), counted without atomics by ballot peer masks into
// one LDS row per wavefront and added over the wavefronts.
template <int NB>
__global__ __launch_bounds__(kPlaceWaves * kWave) void hash_ids_rows_kernel(
    const int32_t* __restrict__ token_ids, const int32_t* __restrict__ tid2eid, int32_t vocab,
    int64_t R, int k, int E, int32_t* __restrict__ ids, int32_t* __restrict__ rows) {
  constexpr int CPW = kBesideTile / (kPlaceWaves * kWave);
  __shared__ int32_t wh[kPlaceWaves][kPlaceMaxE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int ev[CPW];
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch) {
    const int64_t r = (int64_t)blockIdx.x * kBesideTile + (wave * CPW + ch) * kWave + lane;
    int e = -1;
    if (r < R) {
      const int v = token_ids[r / k];
      if (v >= 0 && v < vocab) {
        e = tid2eid[(int64_t)v * k + r % k];
        if (e < 0 || e >= E) e = -1;
      }
      ids[r] = e;
    }
    ev[ch] = e;
  }
  for (int e = lane; e < E; e += kWave) wh[wave][e] = 0;
  __syncthreads();
  const uint64_t below = lanemask_lt();
#pragma unroll
  for (int ch = 0; ch < CPW; ++ch) {
    const uint64_t p = peer_mask<NB>(ev[ch]);
    if (ev[ch] >= 0 && (p & below) == 0) wh[wave][ev[ch]] += __popcll(p);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPlaceWaves * kWave) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < kPlaceWaves; ++w) n += wh[w][e];
    rows[(int64_t)blockIdx.x * E + e] = n;
  }
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
// NSPLIT == 0: the logits are the sum, in slice order, of n_parts arrays of
// per-slot partial dot products part[s][t * k + j] (split_stride = T * k
// apart, hash_dots_kernel), plus logit_bias[e].
template <int SEG, int NSPLIT, int WPB, bool HIST, int NB>
__global__ __launch_bounds__(WPB * kWave) void hash_route_tiles_kernel(
    RouteCfg c, const int32_t* __restrict__ token_ids, const int32_t* __restrict__ tid2eid,
    int32_t vocab, const float* __restrict__ logits, int64_t split_stride, int n_parts,
    const float* __restrict__ logit_bias, int32_t* __restrict__ ids,
    float* __restrict__ weights, int32_t* __restrict__ dev_err, hist_t* __restrict__ hist,
    int32_t* __restrict__ super_sum, int super_S) {
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
  if constexpr (NSPLIT > 0) {
    if (e >= 0) {
      float pv[NSPLIT];
#pragma unroll
      for (int sp = 0; sp < NSPLIT; ++sp) pv[sp] = logits[sp * split_stride + t * E + e];
      my_l = pv[0];
#pragma unroll
      for (int sp = 1; sp < NSPLIT; ++sp) my_l += pv[sp];
    }
  } else if (e >= 0) {
    constexpr int B = 16;  // loads in flight
    const float* src = logits + t * k + sl;
    for (int s0 = 0; s0 < n_parts; s0 += B) {
      float pv[B];
#pragma unroll
      for (int i = 0; i < B; ++i)
        pv[i] = s0 + i < n_parts ? src[(int64_t)(s0 + i) * split_stride] : 0.f;
#pragma unroll
      for (int i = 0; i < B; ++i)
        if (s0 + i < n_parts) my_l += pv[i];
    }
    if (logit_bias) my_l += logit_bias[e];
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
                           int32_t vocab, const float* logits, int64_t stride, int n_parts,
                           const float* lb, int32_t* ids, float* w, int32_t* err, hist_t* hist,
                           int32_t* super_sum, int S, hipStream_t s) {
  constexpr int tpb = kHashTileWaves * (kWave / SEG);
  const dim3 grid((uint32_t)(((int64_t)c.T + tpb - 1) / tpb));
  const dim3 block(kHashTileWaves * kWave);
  auto go = [&](auto kernel) {
    return launch(kStageHash, kernel, grid, block, s, c, tok, tab, vocab, logits, stride,
                  n_parts, lb, ids, w, err, hist, super_sum, S);
  };
  if (c.E <= 128) return go(hash_route_tiles_kernel<SEG, NS, kHashTileWaves, HIST, 7>);
  if (c.E <= 256) return go(hash_route_tiles_kernel<SEG, NS, kHashTileWaves, HIST, 8>);
  return go(hash_route_tiles_kernel<SEG, NS, kHashTileWaves, HIST, 10>);
}

// splits > 0: the gate's K-split arrays of every expert's logit; splits ==
// 0: n_parts arrays of per-slot partial dot products (+ logit bias lb).
template <int SEG>
hipError_t launch_tiles_seg(const RouteCfg& c, const int32_t* tok, const int32_t* tab,
                            int32_t vocab, const float* logits, int32_t splits, int64_t stride,
                            int n_parts, const float* lb, int32_t* ids, float* w, int32_t* err,
                            hist_t* hist, int32_t* super_sum, int S, hipStream_t s) {
#define MOE_HT(NS_)                                                                            \
  if (splits == NS_)                                                                           \
    return hist ? launch_tiles_nb<SEG, NS_, true>(c, tok, tab, vocab, logits, stride, n_parts,  \
                                                  lb, ids, w, err, hist, super_sum, S, s)       \
                : launch_tiles_nb<SEG, NS_, false>(c, tok, tab, vocab, logits, stride, n_parts, \
                                                   lb, ids, w, err, hist, super_sum, S, s);
  MOE_HT(0)
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

hipError_t launch_hash_ids(const RouteCfg& c, const int32_t* token_ids, const int32_t* tid2eid,
                           int32_t vocab, int32_t* ids, hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  const int64_t R = (int64_t)c.T * c.k;
  return launch(kStageHashIds, hash_ids_kernel, dim3((uint32_t)((R + 255) / 256)), dim3(256),
                stream, token_ids, tid2eid, vocab, R, c.k, c.E, ids);
}

hipError_t launch_hash_tiles(const RouteCfg& c, const int32_t* token_ids,
                             const int32_t* tid2eid, int32_t vocab, const float* logits,
                             int32_t splits, int64_t split_stride, int32_t n_parts,
                             const float* logit_bias, int32_t* ids, float* weights,
                             int32_t* dev_err, hist_t* hist, int32_t* super_sum,
                             hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  if (c.E > 1024 || c.k > 32 || (splits == 0 && n_parts < 1)) return hipErrorInvalidValue;
  int S = 1;
  if (hist) {
    const int64_t R = (int64_t)c.T * c.k;
    const int tr = hash_tile_tokens(c.k) * c.k;
    if (!dispatch_super_ok(R, c.E, tr)) return hipErrorInvalidValue;
    S = dispatch_super_size(R, tr);
  }
  const float* lb = splits == 0 ? logit_bias : nullptr;
  switch (hash_seg(c.k)) {
    case 4: return launch_tiles_seg<4>(c, token_ids, tid2eid, vocab, logits, splits, split_stride,
                                       n_parts, lb, ids, weights, dev_err, hist, super_sum, S,
                                       stream);
    case 8: return launch_tiles_seg<8>(c, token_ids, tid2eid, vocab, logits, splits, split_stride,
                                       n_parts, lb, ids, weights, dev_err, hist, super_sum, S,
                                       stream);
    case 16: return launch_tiles_seg<16>(c, token_ids, tid2eid, vocab, logits, splits,
                                         split_stride, n_parts, lb, ids, weights, dev_err, hist,
                                         super_sum, S, stream);
    default: return launch_tiles_seg<64>(c, token_ids, tid2eid, vocab, logits, splits,
                                         split_stride, n_parts, lb, ids, weights, dev_err, hist,
                                         super_sum, S, stream);
  }
}

// The slice width of hash_dots_kernel for E experts (the W slice of every
// expert fits the LDS), or 0 when the kernel does not apply: bf16, k <= 8,
// E <= 768, d a multiple of 8, 16-byte aligned rows.  192 columns up to 384
// experts (fewer partial sums for the hash kernel to add than 128, as fast
// in the dot products; 64 measured 76 against 60 us on the DeepSeek-V4-like
// shape), else 64.
int hash_dot_slice(const RouteCfg& c, int32_t dtype, bool aligned) {
  if (dtype != 1 || !aligned || c.k > kDotMaxK || c.d % 8 != 0 || c.E > 768 ||
      std::getenv("MOE_HASH_DENSE"))
    return 0;
  const bool small = c.E <= 384;
  if (const char* env = std::getenv("MOE_HASH_SLICE")) {  // tuning: 64 (+ 112, 128, 192)
    const int v = std::atoi(env);
    if (small && (v == 112 || v == 128 || v == 192)) return v;
    if (v == 64) return v;
  }
  return small ? 192 : 64;
}

int hash_dot_slices(const RouteCfg& c, int32_t dtype, bool aligned) {
  const int sl = hash_dot_slice(c, dtype, aligned);
  return sl ? (c.d + sl - 1) / sl : 0;
}

// Workgroups of `threads` threads of this kernel one CU holds at once
// (registers and LDS), looked up once per kernel.
int resident_blocks(const void* kernel, int threads) {
  static std::mutex mu;
  static std::unordered_map<const void*, int> cache;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(kernel);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1)
    n = 1;
  cache.emplace(kernel, n);
  return n;
}

// slices x token chunks, as many workgroups as the CUs hold at once (a
// second round of a few workgroups would double the time); the slices of
// one chunk are neighbours in launch order, so they read each x row at
// about the same time
constexpr int kDotCus = 256, kDotWaves = 16;
struct DotsGrid {
  int ns = 0, chunks = 0, per_cu = 1;
  int64_t per = 0;
};
DotsGrid dots_grid(const RouteCfg& c, int sl, const void* kernel) {
  DotsGrid g;
  g.ns = (c.d + sl - 1) / sl;
  g.per_cu = resident_blocks(kernel, kDotWaves * kWave);
  g.chunks = std::max(1, std::min((c.T + 255) / 256, kDotCus * g.per_cu / g.ns));
  g.per = (c.T + g.chunks - 1) / g.chunks;
  return g;
}

// The dot-product kernel for slice width sl and E experts (nullptr: none),
// with or without the placement workgroups.  8 lanes per token (pieces
// split over them), 16 wavefronts, 3 tiles ahead.
template <bool PLACE>
const void* dots_kernel(int sl, int32_t E, int32_t kk) {
  auto k = [](auto kernel) { return reinterpret_cast<const void*>(kernel); };
  if (sl == 192 && E <= 384) {  // the widest slices: k of 4, 6 and 8 compiled in
    switch (kk) {
      case 4: return k(hash_dots_kernel<192, 384, 8, kDotWaves, 3, PLACE, 4>);
      case 6: return k(hash_dots_kernel<192, 384, 8, kDotWaves, 3, PLACE, 6>);
      case 8: return k(hash_dots_kernel<192, 384, 8, kDotWaves, 3, PLACE, 8>);
      default: return k(hash_dots_kernel<192, 384, 8, kDotWaves, 3, PLACE>);
    }
  }
  if (sl == 128 && E <= 384) return k(hash_dots_kernel<128, 384, 8, kDotWaves, 3, PLACE>);
  if (sl == 112 && E <= 384) return k(hash_dots_kernel<112, 384, 8, kDotWaves, 3, PLACE>);
  if constexpr (!PLACE)  // its 48 KB W slice holds no placement's LDS
    if (sl == 64 && E <= 384) return k(hash_dots_kernel<64, 384, 8, kDotWaves, 3, PLACE>);
  if (sl == 64 && E <= 768) return k(hash_dots_kernel<64, 768, 8, kDotWaves, 3, PLACE>);
  return nullptr;
}

hipError_t launch_dots(const RouteCfg& c, const void* kernel, const DotsGrid& g, dim3 grid,
                       const void* x, const void* W, const int32_t* ids, float* part,
                       int32_t* zero, int32_t zero_words, const BesidePlace& place,
                       hipStream_t stream) {
  typedef void (*Fn)(const uint16_t*, const uint16_t*, const int32_t*, int, int, int, int,
                     int64_t, float*, int32_t*, int, int, BesidePlace);
  return launch(kStageHashDots, reinterpret_cast<Fn>(const_cast<void*>(kernel)), grid,
                dim3(kDotWaves * kWave), stream, (const uint16_t*)x, (const uint16_t*)W, ids,
                c.T, c.d, c.E, c.k, g.per, part, zero, zero_words, g.ns, place);
}

hipError_t launch_hash_dots(const RouteCfg& c, int32_t dtype, const void* x, const void* W,
                            const int32_t* ids, float* part, int32_t* zero, int32_t zero_words,
                            hipStream_t stream) {
  const bool aligned = reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(W) % 16 == 0;
  const int sl = hash_dot_slice(c, dtype, aligned);
  if (sl == 0) return hipErrorInvalidValue;
  if (c.T == 0) return hipSuccess;
  const void* kernel = dots_kernel<false>(sl, c.E, c.k);
  if (!kernel) return hipErrorInvalidValue;
  const DotsGrid g = dots_grid(c, sl, kernel);
  return launch_dots(c, kernel, g, dim3((uint32_t)g.ns, (uint32_t)g.chunks), x, W, ids, part,
                     zero, zero_words, BesidePlace{}, stream);
}

// Placement workgroups beside the dot products: the CUs the slices x chunks
// grid leaves free, at most one per tile.  Taken when the placements should
// end well inside the dot products: each round of them reads every tile's
// row (nt * E * 4 bytes, ~50 GB/s into one CU) after a few microseconds of
// latency, against x streaming at ~4 TB/s (DeepSeek-V4-like hash layer: 48
// tiles on 28 free CUs, two rounds of ~4 us against ~60 us of dot products).
int hash_beside_places(const RouteCfg& c, int32_t dtype, bool aligned) {
  const char* env = std::getenv("MOE_HASH_BESIDE");  // tuning: 0 never, 1 whenever possible
  if (env && env[0] == '0') return 0;
  const int sl = hash_dot_slice(c, dtype, aligned);
  if (sl == 0 || c.T == 0 || c.E > kPlaceMaxE) return 0;
  const void* kernel = dots_kernel<true>(sl, c.E, c.k);
  if (!kernel) return 0;
  const DotsGrid g = dots_grid(c, sl, kernel);
  const int64_t R = (int64_t)c.T * c.k;
  const int64_t nt = (R + kBesideTile - 1) / kBesideTile;
  const int64_t free_cus = (int64_t)kDotCus * g.per_cu - (int64_t)g.ns * g.chunks;
  if (free_cus < 1) return 0;
  const int n_place = (int)std::min<int64_t>(nt, free_cus);
  if (env && env[0] == '1') return n_place;
  const double rounds = (double)((nt + n_place - 1) / n_place);
  const double place_us = rounds * (4.0 + (double)nt * c.E * 4 / 50e3);
  const double dots_us = (double)c.T * c.d * 2 / 4e6;
  return place_us <= 0.5 * dots_us ? n_place : 0;
}

hipError_t launch_hash_ids_rows(const RouteCfg& c, const int32_t* token_ids,
                                const int32_t* tid2eid, int32_t vocab, int32_t* ids,
                                int32_t* rows, hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  if (c.E > kPlaceMaxE) return hipErrorInvalidValue;
  const int64_t R = (int64_t)c.T * c.k;
  const dim3 grid((uint32_t)((R + kBesideTile - 1) / kBesideTile));
  return launch(kStageHashIds, hash_ids_rows_kernel<kPlaceIdBits>, grid,
                dim3(kPlaceWaves * kWave), stream, token_ids, tid2eid, vocab, R, c.k, c.E, ids,
                rows);
}

hipError_t launch_hash_dots_beside(const RouteCfg& c, int32_t dtype, const void* x,
                                   const void* W, float* part, const BesidePlace& place,
                                   hipStream_t stream) {
  const bool aligned = reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(W) % 16 == 0;
  const int sl = hash_dot_slice(c, dtype, aligned);
  const void* kernel = sl ? dots_kernel<true>(sl, c.E, c.k) : nullptr;
  if (!kernel || c.T == 0 || place.n_place < 1 || place.E != c.E ||
      place.R != (int64_t)c.T * c.k || place.nt != (place.R + kBesideTile - 1) / kBesideTile)
    return hipErrorInvalidValue;
  const DotsGrid g = dots_grid(c, sl, kernel);
  BesidePlace pl = place;
  pl.n_dots = g.ns * g.chunks;  // chunks past the last token return at once
  return launch_dots(c, kernel, g, dim3((uint32_t)(pl.n_dots + pl.n_place)), x, W, pl.ids,
                     part, nullptr, 0, pl, stream);
}

}  // namespace moe
