// Gate contraction on gfx950 matrix cores.
//
// logits[t][e] = sum_i x[t][i] * W[e][i] (+ logit_bias[e]), fp32 accumulate.
// The gate of "DeepSeek-V3.2-Exp - Select experts" (gate-forward excerpt)
// casts both operands to fp32 before the linear map; bf16 products are exact
// in fp32, so bf16 inputs go through v_mfma_f32_16x16x32_bf16 and fp32
// inputs through v_mfma_f32_16x16x4_f32 (never rounded to bf16).
//
// Shape: M = T tokens (thousands), N = E experts (8..1024), K = d.  The
// contraction is skinny (E flop per byte of x), so x must stream from HBM
// once and the chip must be filled: a workgroup (4 waves, 2 x 2, or 8 waves,
// 4 x 2 or 2 x 4) owns a BM x BN tile, N is split into E/BN tiles and K into
// up to 8 partial sums when whole tiles would leave CUs idle; the row pieces
// re-read from L2 bound the large gates, so the planner scores tiles and
// splits by those bytes.  Tiles are ordered so that the N tiles of one M
// tile -- which read the same x rows -- run together on one XCD and share
// its L2 (workgroups are handed to the 8 XCDs round-robin).
//
// Two kernels share the tiling.  The pipelined one (16-byte aligned rows)
// copies each stage's x and W row slices straight into an LDS ring with
// buffer_load ... lds, keeps NS-1 stages in flight, and writes its tile
// through LDS as whole rows -- or, for whole-row tiles, runs the selection
// on them there (the fused epilogue).  The general one (any d, any
// alignment) stages through registers into two padded LDS buffers, one
// stage ahead.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "select_core.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kXcds = 8;

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

// One 16-byte chunk (elements [k, k + kPerChunk) of row `row`), zero outside
// [0, rows) x [0, d).  VEC: rows are 16-byte aligned and d % kPerChunk == 0.
template <typename In, bool VEC>
__device__ __forceinline__ u32x4_t load_chunk(const In* base, int64_t row, int rows, int k,
                                              int d) {
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

// BM x BN tile, KB bytes of K per stage.
template <typename In, int BM, int BN, int KB, bool VEC>
__global__ __launch_bounds__(kThreads) void gate_gemm_kernel(
    const In* __restrict__ x, const In* __restrict__ W, const float* __restrict__ logit_bias,
    float* __restrict__ logits, int T, int d, int E, int n_m, int n_n, int per_xcd) {
  constexpr int P = ElemInfo<In>::kPerChunk;
  constexpr int BK = KB / (int)sizeof(In);  // K elements per stage
  constexpr int CPR = KB / 16;              // 16-byte chunks per row per stage
  constexpr int STRIDE = KB + 16;           // padded LDS row (bytes)
  constexpr int MB = BM / 32;               // 16-row blocks per wave
  constexpr int NB = BN / 32;               // 16-col blocks per wave
  constexpr int A_CH = BM * CPR / kThreads;
  constexpr int B_CH = BN * CPR / kThreads;
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile shape");
  static_assert(BM * CPR % kThreads == 0 && BN * CPR % kThreads == 0, "chunk split");
  static_assert(KB % 64 == 0, "stage size");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * STRIDE];

  // XCD-aware tile order: consecutive tile ids (the N tiles of one M tile,
  // then the next M tile) go to one XCD.
  const int L = blockIdx.x;
  const int tile = (L % kXcds) * per_xcd + L / kXcds;
  if (tile >= n_m * n_n) return;
  const int64_t m0 = (int64_t)(tile / n_n) * BM;
  const int n0 = (tile % n_n) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  u32x4_t ra[A_CH], rb[B_CH];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * kThreads;
      ra[i] = load_chunk<In, VEC>(x, m0 + c / CPR, T, k0 + (c % CPR) * P, d);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * kThreads;
      rb[i] = load_chunk<In, VEC>(W, (int64_t)n0 + c / CPR, E, k0 + (c % CPR) * P, d);
    }
  };
  auto stash = [&](uint8_t* buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * kThreads;
      *reinterpret_cast<u32x4_t*>(buf + (c / CPR) * STRIDE + (c % CPR) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * kThreads;
      *reinterpret_cast<u32x4_t*>(buf + (BM + c / CPR) * STRIDE + (c % CPR) * 16) = rb[i];
    }
  };

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int row16 = lane & 15;  // row of A / column of B this lane feeds
  const int kq = lane >> 4;     // which quarter of the MFMA's K this lane feeds
  const int a_off = (wm * (BM / 2) + row16) * STRIDE + kq * 16;
  const int b_off = (BM + wn * (BN / 2) + row16) * STRIDE + kq * 16;

  auto compute = [&](const uint8_t* buf) {
#pragma unroll
    for (int ks = 0; ks < KB / 64; ++ks) {
      if constexpr (sizeof(In) == 2) {
        // one K=32 MFMA step: lane feeds elements [kq*8, kq*8+8)
        bf16x8_t af[MB], bfr[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(buf + a_off + i * 16 * STRIDE + ks * 64);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8_t*>(buf + b_off + j * 16 * STRIDE + ks * 64);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      } else {
        // a 16-wide K step as four K=4 MFMAs.  A and B use the same
        // permutation of K: MFMA s takes element kq*4 + s of the step, so
        // each lane reads one float4 per operand and the sum is unchanged.
        f32x4_t af[MB], bfr[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
          af[i] = *reinterpret_cast<const f32x4_t*>(buf + a_off + i * 16 * STRIDE + ks * 64);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          bfr[j] = *reinterpret_cast<const f32x4_t*>(buf + b_off + j * 16 * STRIDE + ks * 64);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][s], bfr[j][s], acc[i][j], 0, 0, 0);
      }
    }
  };

  const int n_stages = (d + BK - 1) / BK;
  fetch(0);
  stash(lds[0]);
  __syncthreads();
  for (int s = 0; s < n_stages; ++s) {
    const bool more = s + 1 < n_stages;
    if (more) fetch((s + 1) * BK);  // in flight during this stage's MFMAs
    compute(lds[s & 1]);
    if (more) stash(lds[(s + 1) & 1]);
    __syncthreads();
  }

  // D layout of a 16x16 MFMA: lane holds rows 4*(lane/16) + r, column lane%16.
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int e = n0 + wn * (BN / 2) + j * 16 + row16;
    if (e >= E) continue;
    const float b = logit_bias ? logit_bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = m0 + wm * (BM / 2) + i * 16 + kq * 4 + r;
        if (t < T) logits[t * E + e] = acc[i][j][r] + b;
      }
  }
}


// ---------------------------------------------------------------------------
// Deep pipeline for 16-byte aligned rows (the common case): global -> LDS
// copies with buffer_load ... lds, an NS-stage ring, NS-1 stages in flight
// while one is multiplied.  A stage holds RB bytes of K of every tile row:
// 64, 128, 256 or 512.  Longer row segments give each barrier RB / 64
// matrix-core k-steps of work; shorter ones let large tiles keep a deep ring
// (x streams from HBM at about 3 TB/s with 8 KB in flight per CU and at
// about 5.9 TB/s from 32 KB on).
//
// LDS layout of a stage: the tile's BM x rows then BN W rows, RB bytes each,
// no padding; the 16-byte chunk c of row r sits in slot c ^ swz(r), so the
// eight rows one ds_read_b128 pass touches cover all banks: swz(r) = r % 8
// for rows of 128 bytes or more, (r / 2) % 4 for 64-byte rows (two rows per
// bank sweep).  One load instruction of a wave fills 1 KB = 1024 / RB rows:
// lane l writes slot l % (RB / 16) of row l / (RB / 16) (the hardware places
// lane data contiguously), so it fetches chunk slot ^ swz(row) of that row.
// Rows past T or E, chunks past the end of a row (d need not fill the last
// stage) and the unused stages after the last one read past the buffer
// descriptor's range and load zeros without touching memory.
// gfx9 s_waitcnt immediate: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] << 14.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_counts() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (LGKM << 8) | ((VM >> 4) << 14));
}

// Barrier between pipeline stages.  __syncthreads() would add a release
// fence, i.e. wait for every copy still in flight; here each wave waits only
// until at most VM of its copies are outstanding (the older ones -- the stage
// about to be read -- have landed in LDS) and its own LDS reads are done
// (the stage about to be overwritten is no longer read), then meets the
// other waves.
template <int VM>
__device__ __forceinline__ void stage_barrier() {
  wait_counts<VM, 0>();
  __builtin_amdgcn_s_barrier();
}

template <int RB>
__device__ __forceinline__ int stage_swizzle(int row) {
  return RB >= 128 ? (row & 7) : ((row >> 1) & 3);
}

template <typename In>
struct Frag;
template <>
struct Frag<uint16_t> {
  typedef bf16x8_t type;
};
template <>
struct Frag<float> {
  typedef f32x4_t type;
};

// The fused selection: the tile's BM rows of logits (+ logit bias) are in
// LDS (lo, PITCH floats per row, all of E); the workgroup's NW wavefronts
// route NW * 64 / LPT tokens per pass with the select kernel's per-token
// code, and with HIST count their picks into the tile's dispatch histogram
// (row mt: the tile's BM tokens x k routes form one dispatch tile).
// `pick` ([NW * 64 / LPT][kMaxK]) and `whist` ([NW][kFusedMaxE]) are LDS
// scratch carved from the ring behind the tile's rows.
constexpr int kFusedMaxE = 128;  // experts of the fused selection
constexpr int kFusedIdBits = 7;  // bits of an expert id below kFusedMaxE

template <class EPI, int BM, int NW, int PITCH>
__device__ __forceinline__ void fused_select(const float* lo, int32_t (*pick)[sel::kMaxK],
                                             int32_t (*whist)[kFusedMaxE], int m0, int T,
                                             int lane, int wave, int mt, const SelectArgs& sa) {
  constexpr int LPT = EPI::kLpt, VPL = EPI::kVpl;
  constexpr int TPW = kWave / LPT;  // tokens per wavefront and pass
  constexpr int TPP = NW * TPW;     // tokens per pass
  constexpr int KPL = (sel::kMaxK + LPT - 1) / LPT;
  static_assert(BM % TPP == 0, "passes");
  const int E = sa.c.E;
  const int seg = lane / LPT, sl = lane % LPT;
  const int e0 = sl * VPL;
  const int nval = min(max(E - e0, 0), VPL);
  const bool lvec = sa.vec && nval == VPL;
  float sb[VPL];  // the same experts for every token of this lane
  sel::load_sbias<VPL, EPI::kMono>(sa.select_bias, e0, E, lvec, sb);
  if constexpr (EPI::kHist)
    for (int e = lane; e < E; e += kWave) whist[wave][e] = 0;
  for (int ps = 0; ps < BM / TPP; ++ps) {
    const int tw = ps * TPP + wave * TPW;  // the wavefront's first tile row
    if (m0 + tw >= T) break;              // wave-uniform
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();      // pick rows (and histogram) reused
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int tb = tw + seg;
    const int64_t t = (int64_t)m0 + tb;
    const bool tok_ok = t < T;
    const int64_t trow = tok_ok ? t : (int64_t)m0 + tw;
    const float* row = lo + tb * PITCH;
    float lv[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) lv[j] = (tok_ok && j < nval) ? row[e0 + j] : -INFINITY;
    const int kraw = sa.k_per_token ? sa.k_per_token[trow] : sa.c.k;
    int pid[KPL];
    sel::select_token<LPT, VPL, EPI::kMono, EPI::kK>(sa.c, sl, seg, tok_ok, t, lv, nval, sb, kraw, row,
                                            pick[wave * TPW + seg], sa.ids, sa.weights,
                                            sa.dev_err, pid);
    if constexpr (EPI::kHist) sel::count_picks<LPT, kFusedIdBits>(pid, sl, sa.c.k, whist[wave]);
  }
  if constexpr (EPI::kHist) {
    __syncthreads();
    for (int e = wave * kWave + lane; e < E; e += NW * kWave) {
      int n = 0;
#pragma unroll
      for (int w8 = 0; w8 < NW; ++w8) n += whist[w8][e];
      sa.hist[(int64_t)mt * E + e] = (hist_t)n;
    }
  }
}

// Epilogue policies of the pipelined kernel: store the logits (NoSel), or
// also run the selection on the tile's rows in LDS (FusedSel: LPT lanes per
// token, VPL experts per lane, the monotone-key case, dispatch histograms).
struct NoSel {
  static constexpr bool kOn = false;
};
template <int LPT, int VPL, bool MONO, bool HIST, int KC = 0>
struct FusedSel {
  static constexpr bool kOn = true, kMono = MONO, kHist = HIST;
  static constexpr int kLpt = LPT, kVpl = VPL, kK = KC;  // kK > 0: k == kK
};

// NS: stages of x in the ring; NSW: stages of W.  With NSW == NS each stage
// is one slot (the tile's x rows, then its W rows); with NSW == NS - 1 the x
// and W rings are separate, so that a tile too large for NS slots of both
// still keeps NS - 1 stages of x (the rows that come from HBM) in flight
// while W, read from L2, runs one stage ahead.
template <typename In, int BM, int BN, int NS, int RB, int WM, int WN, class EPI, int NSW>
__global__ __launch_bounds__(WM * WN * kWave) void gate_gemm_pipe_kernel(
    const In* __restrict__ x, const In* __restrict__ W, const float* __restrict__ logit_bias,
    float* __restrict__ out, int T, int d, int E, int n_m, int n_n, int splits, int per_xcd,
    int stages_per_split, SelectArgs sa) {
  constexpr int ROWS = BM + BN;
  constexpr int STAGE = ROWS * RB;             // bytes per stage
  constexpr bool SPLIT_RING = NSW != NS;
  static_assert(NSW == NS || NSW == NS - 1, "W ring depth");
  constexpr int LDS_BYTES = NS * BM * RB + NSW * BN * RB;
  constexpr int RPI = 1024 / RB;               // rows per load instruction
  constexpr int CPR = RB / 16;                 // 16-byte chunks per row and stage
  constexpr int NW = WM * WN;                  // waves: WM along M x WN along N
  constexpr int BLOCKS = ROWS / RPI;           // load instructions per stage
  constexpr int LPS = (BLOCKS + NW - 1) / NW;  // ... per wave (the last one by some waves)
  constexpr int LPS_SHORT = BLOCKS / NW;       // ... per wave without the last one
  constexpr int KSTEPS = RB / 64;              // 64-byte matrix-core k-steps per stage
  constexpr int MB = BM / WM / 16;             // 16-row blocks per wave
  constexpr int NB = BN / WN / 16;             // 16-column blocks per wave
  static_assert(RB == 64 || RB == 128 || RB == 256 || RB == 512, "stage row bytes");
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0 && ROWS % RPI == 0, "tile shape");
  static_assert(NS >= 2 && (NS - 2) * LPS < 64, "pipeline depth");
  // split rings: whole 1-KB blocks of x and of W for every wave
  constexpr int LX = BM / RPI / NW, LW = BN / RPI / NW;
  static_assert(!SPLIT_RING || (NSW >= 2 && LX * NW * RPI == BM && LW * NW * RPI == BN &&
                                LX + (NSW - 2) * (LX + LW) < 64),
                "split ring shape");
  typedef typename Frag<In>::type FragT;

  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
  // ring slots of stage st (counted from st_begin): x rows, then W rows
  auto x_slot = [&](int st) -> uint8_t* {
    return SPLIT_RING ? lds + (st % NS) * (BM * RB) : lds + (st % NS) * STAGE;
  };
  auto w_slot = [&](int st) -> uint8_t* {
    return SPLIT_RING ? lds + NS * BM * RB + (st % NSW) * (BN * RB)
                      : lds + (st % NS) * STAGE + BM * RB;
  };

  if (sa.zero_words > 0) {  // a slice of the array the next kernel adds into
    const int per = (sa.zero_words + (int)gridDim.x - 1) / (int)gridDim.x;
    const int beg = (int)blockIdx.x * per, end = min(beg + per, sa.zero_words);
    for (int i = beg + (int)threadIdx.x; i < end; i += WM * WN * kWave) sa.zero[i] = 0;
  }

  // Tile order: tile ids run N tile fastest, then M tile, then K split, and
  // consecutive ids go to one XCD, so the N tiles of one (M tile, split) --
  // which read the same x rows -- share that XCD's L2.
  const int L = blockIdx.x;
  const int tile = (L % kXcds) * per_xcd + L / kXcds;
  if (tile >= n_m * n_n * splits) return;
  const int split = tile / (n_m * n_n);
  const int mt = (tile / n_n) % n_m;
  const int nt = tile % n_n;
  const int m0 = mt * BM;
  const int n0 = nt * BN;
  float* __restrict__ logits = out + (int64_t)split * T * E;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  // waves that own a copy in the last, partial round of a stage's blocks
  const bool full = LPS == LPS_SHORT || wave + NW * (LPS - 1) < BLOCKS;

  const uint32_t row_bytes = (uint32_t)d * sizeof(In);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, (short)0, (int)((uint32_t)T * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)W, (short)0, (int)((uint32_t)E * row_bytes), 0x00020000);
  const int n_stages = (int)((row_bytes + RB - 1) / RB);
  const int st_begin = split * stages_per_split;
  const int st_end = min(n_stages, st_begin + stages_per_split);

  // per-lane source offsets (bytes, stage 0) of this wave's load instructions
  // and the byte position of the lane's chunk within a stage's row segment
  uint32_t src_off[LPS];
  uint32_t chunk_b[LPS];
  bool src_is_x[LPS];
#pragma unroll
  for (int i = 0; i < LPS; ++i) {
    const int blk = wave + NW * i;             // RPI-row block of the tile
    const int r = blk * RPI + lane / CPR;      // tile row (past ROWS: no such copy)
    const int chunk = (lane % CPR) ^ stage_swizzle<RB>(r);
    src_is_x[i] = r < BM;
    const uint32_t grow = src_is_x[i] ? (uint32_t)(m0 + r) : (uint32_t)(n0 + r - BM);
    const uint32_t nrows = src_is_x[i] ? (uint32_t)T : (uint32_t)E;
    chunk_b[i] = (uint32_t)chunk * 16;
    // rows past the end: an offset past the descriptor range reads zeros
    src_off[i] = grow < nrows ? grow * row_bytes + chunk_b[i] : 0x80000000u;
  }
  // With the selection fused every tile spans all experts, so each x byte is
  // read by one workgroup: its copies are non-temporal (the nt bit), which
  // kept the gpt-oss-like gate at 83.5 instead of 85.8 us; with several
  // expert tiles (x re-read from L2) or a large W it was slower (DeepSeek-
  // V3-like 41 -> 46 us), so the other shapes keep the default policy.
  constexpr int kXPolicy = EPI::kOn ? 2 : 0;
  // copies of stage st (counted from st_begin) of x (X) and of W (!X) rows;
  // blocks of the combined ring are the stage's x rows, then its W rows
  auto issue_part = [&](int st, bool X) {  // X: a constant at every call
    const uint32_t koff = st < st_end ? (uint32_t)st * RB : 0x80000000u;
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      if (i == LPS - 1 && !full) break;  // wave-uniform
      if (SPLIT_RING && (i < LX) != X) continue;
      const int blk = wave + NW * i;
      uint8_t* dst8 = SPLIT_RING ? (X ? x_slot(st - st_begin) + blk * 1024
                                      : w_slot(st - st_begin) + (blk - LX * NW) * 1024)
                                 : x_slot(st - st_begin) + blk * 1024;
      auto* dst = (__attribute__((address_space(3))) void*)dst8;
      const bool live = (src_off[i] | koff) < 0x80000000u && koff + chunk_b[i] < row_bytes;
      const uint32_t off = live ? src_off[i] + koff : 0x80000000u;
      if (src_is_x[i])
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst, 16, off, 0, 0, kXPolicy);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16, off, 0, 0, 0);
    }
  };
  // the copies that refill the slots of the stage all waves just finished:
  // stage st of x, and (split rings) stage st - (NS - NSW) of W, issued first
  auto issue = [&](int st) {
    if constexpr (SPLIT_RING) {
      if (st - (NS - NSW) >= st_begin) issue_part(st - (NS - NSW), false);
      issue_part(st, true);
    } else {
      issue_part(st, true);
    }
  };
  // each wave waits for its own copies: the stages issued after the one about
  // to be read may stay in flight (combined ring: NS - 2 stages; split rings:
  // that refill's x stage, then NSW - 2 refills of W and x)
  auto barrier = [&]() {
    if constexpr (SPLIT_RING)
      stage_barrier<LX + (NSW - 2) * (LX + LW)>();
    else if (full)
      stage_barrier<(NS - 2) * LPS>();
    else
      stage_barrier<(NS - 2) * LPS_SHORT>();
  };

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int row16 = lane & 15;
  const int kq = lane >> 4;
  const int sw = stage_swizzle<RB>(row16);  // swz of every row this lane reads
  const int a_row = wm * (BM / WM) + row16;
  const int b_row = wn * (BN / WN) + row16;  // within the stage's W rows

  // Operand fragments of one k-step, double-buffered so that the LDS reads
  // of the next k-step are in flight while this one's MFMAs run.
  FragT fa[2][MB], fb[2][NB];
  auto load = [&](int p, const uint8_t* xb, const uint8_t* wb, int ks) {
    const int slot = ((ks * 4 + kq) ^ sw) * 16;
#pragma unroll
    for (int i = 0; i < MB; ++i)
      fa[p][i] = *reinterpret_cast<const FragT*>(xb + (a_row + i * 16) * RB + slot);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      fb[p][j] = *reinterpret_cast<const FragT*>(wb + (b_row + j * 16) * RB + slot);
  };
  auto mma = [&](int p) {
    if constexpr (sizeof(In) == 2) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[p][i], fb[p][j], acc[i][j], 0, 0, 0);
    } else {
      // a 16-wide K step as four K=4 MFMAs.  A and B use the same
      // permutation of K: MFMA s takes element kq*4 + s of the step, so each
      // lane reads one float4 per operand and the sum is unchanged.
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[p][i][s4], fb[p][j][s4], acc[i][j],
                                                              0, 0, 0);
    }
  };

  // One stage; P0: the fragment buffer its first k-step reads (a constant,
  // so the fragment arrays stay in registers).
  auto run_stage = [&](int s, auto p0) {
    constexpr int P0 = decltype(p0)::value;
    const uint8_t* xb = x_slot(s - st_begin);
    const uint8_t* wb = w_slot(s - st_begin);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int p = (P0 + ks) & 1;
      if (ks + 1 < KSTEPS) {
        load(p ^ 1, xb, wb, ks + 1);
      } else if (s + 1 < st_end) {
        // stage s + 1 is in LDS and every wave has read all of stage s (this
        // wave's last reads included): refill stage s's buffer, then read the
        // next stage's first k-step behind this one's MFMAs
        barrier();
        issue(s + NS);
        load(p ^ 1, x_slot(s + 1 - st_begin), w_slot(s + 1 - st_begin), 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mma(p);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (st_begin < st_end) {
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st_begin + st);
    barrier();                  // stage st_begin is in LDS
    issue(st_begin + NS - 1);   // into the one buffer not yet used
    load(0, x_slot(0), w_slot(0), 0);
    if constexpr (KSTEPS % 2 == 0) {
      for (int s = st_begin; s < st_end; ++s) run_stage(s, std::integral_constant<int, 0>());
    } else {  // one k-step per stage: the buffers alternate between stages
      for (int s = st_begin; s < st_end; s += 2) {
        run_stage(s, std::integral_constant<int, 0>());
        if (s + 1 < st_end) run_stage(s + 1, std::integral_constant<int, 1>());
      }
    }
  }
  wait_counts<0, 15>();  // no copy may still target LDS when the workgroup ends

  // Epilogue.  A 16 x 16 MFMA result gives a lane one column of four rows,
  // so direct stores write 64-byte row pieces from scattered lanes (measured:
  // about 1.5 TB/s for a 33.5 MB logits array).  Instead the tile (+ logit
  // bias) goes through the ring, now free, and whole rows leave with 16-byte
  // stores from consecutive lanes.  PITCH: padded LDS row, so the four lane
  // groups of one accumulator write hit different banks.
  constexpr int PITCH = BN + 4;                         // floats
  constexpr int WROWS = BM / WM;                        // rows of one wave row
  constexpr int G = LDS_BYTES / (WROWS * PITCH * 4);    // wave rows per pass
  static_assert(!EPI::kOn || G >= WM, "the fused selection needs the whole tile in LDS");
  if constexpr (G >= 1) {
    constexpr int GP = G < WM ? G : WM;
    constexpr int PASSES = (WM + GP - 1) / GP;
    constexpr int C4 = BN / 4;  // float4 per tile row
    float* lo = reinterpret_cast<float*>(lds);
    const bool vec = E % 4 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0;
    const bool bias = logit_bias != nullptr && split == 0;
    const bool store = !EPI::kOn || sa.write_logits;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      __syncthreads();  // the ring (or the previous pass) is no longer read
      if (wm / GP == p) {
        const int rbase = (wm - p * GP) * WROWS;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int col = wn * (BN / WN) + j * 16 + row16;
          const float b = (bias && n0 + col < E) ? logit_bias[n0 + col] : 0.0f;
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              lo[(rbase + i * 16 + kq * 4 + r) * PITCH + col] = acc[i][j][r] + b;
        }
      }
      __syncthreads();
      if (!store) continue;
      const int prow0 = p * GP * WROWS;
      const int prows = (WM - p * GP < GP ? WM - p * GP : GP) * WROWS;
      for (int idx = tid; idx < prows * C4; idx += NW * kWave) {
        const int rr = idx / C4, c4 = idx % C4;
        const int64_t t = (int64_t)m0 + prow0 + rr;
        const int e0 = n0 + c4 * 4;
        if (t >= T || e0 >= E) continue;
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(lo + rr * PITCH + c4 * 4);
        if (vec && e0 + 4 <= E) {
          // non-temporal: the next kernel reads the logits from another
          // XCD, and streamed stores leave L2 clean at the end of the
          // kernel (gpt-oss-like gate: 80.9 -> 74.3 us).  Rows of 384 or
          // more experts keep the default policy: the select kernel then
          // reads the DeepSeek-V4-like partial arrays (50 MB) faster
          // (14.6 -> 13.3 us; step 118.2 -> 116.0 us), while the Qwen3-,
          // OLMoE- and DeepSeek-V3-like steps measured equal or slightly
          // faster with non-temporal stores.
          if (E >= 384)
            *reinterpret_cast<f32x4_t*>(logits + t * E + e0) = v;
          else
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(logits + t * E + e0));
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (e0 + q < E) logits[t * E + e0 + q] = v[q];
        }
      }
    }
    if constexpr (EPI::kOn) {
      // the selection's LDS scratch lies in the ring behind the tile's rows
      // (a workgroup above 144 KB of LDS measured 25-35 % slower)
      constexpr int TPP = NW * (kWave / EPI::kLpt);
      constexpr int PICK_OFF = BM * PITCH * 4;
      constexpr int HIST_OFF = PICK_OFF + TPP * sel::kMaxK * 4;
      static_assert(HIST_OFF + NW * kFusedMaxE * 4 <= LDS_BYTES, "fused scratch in the ring");
      fused_select<EPI, BM, NW, PITCH>(lo, reinterpret_cast<int32_t(*)[sel::kMaxK]>(lds + PICK_OFF),
                                       reinterpret_cast<int32_t(*)[kFusedMaxE]>(lds + HIST_OFF),
                                       m0, T, lane, wave, mt, sa);
    }
  } else {  // the ring cannot hold one wave row of the tile: direct stores
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int e = n0 + wn * (BN / WN) + j * 16 + row16;
      if (e >= E) continue;
      const float b = (logit_bias && split == 0) ? logit_bias[e] : 0.0f;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t t = (int64_t)m0 + wm * (BM / WM) + i * 16 + kq * 4 + r;
          if (t < T) logits[t * E + e] = acc[i][j][r] + b;
        }
    }
  }
}

template <typename In, int BM, int BN, int NS, int RB, int WM, int WN, class EPI = NoSel,
          int NSW = NS>
hipError_t launch_pipe(const void* x, const void* W, const float* logit_bias, float* out,
                       int T, int d, int E, int splits, hipStream_t s,
                       const SelectArgs& sa = SelectArgs{}) {
  const int n_m = (T + BM - 1) / BM;
  const int n_n = (E + BN - 1) / BN;
  const int n_stages = (int)(((int64_t)d * sizeof(In) + RB - 1) / RB);
  const int per_split = (n_stages + splits - 1) / splits;
  const int tiles = n_m * n_n * splits;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  return launch(EPI::kOn ? kStageGateSelect : kStageGate,
                gate_gemm_pipe_kernel<In, BM, BN, NS, RB, WM, WN, EPI, NSW>, dim3(per_xcd * kXcds),
                dim3(WM * WN * kWave), s, (const In*)x, (const In*)W, logit_bias, out, T, d, E,
                n_m, n_n, splits, per_xcd, per_split, sa);
}

template <typename In, int BM, int BN, int KB>
hipError_t launch_tile(const void* x, const void* W, const float* logit_bias, float* logits,
                       int T, int d, int E, hipStream_t s) {
  const int n_m = (T + BM - 1) / BM;
  const int n_n = (E + BN - 1) / BN;
  const int tiles = n_m * n_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const dim3 grid(per_xcd * kXcds);
  const bool vec = (d % ElemInfo<In>::kPerChunk == 0) &&
                   (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(W) % 16 == 0);
  if (vec)
    return launch(kStageGate, gate_gemm_kernel<In, BM, BN, KB, true>, grid, dim3(kThreads), s,
                  (const In*)x, (const In*)W, logit_bias, logits, T, d, E, n_m, n_n, per_xcd);
  return launch(kStageGate, gate_gemm_kernel<In, BM, BN, KB, false>, grid, dim3(kThreads), s,
                (const In*)x, (const In*)W, logit_bias, logits, T, d, E, n_m, n_n, per_xcd);
}

// Tile shapes (BM x BN) and pipeline depth.  The default takes the largest
// useful tile that still gives at least kMinTiles workgroups;
// MOE_GATE_TILE="BMxBN" overrides it (tuning sweeps).
// wm x wn waves per workgroup; `planned`: the planner may pick the tile on
// its own (the others are taken only through MOE_GATE_TILE).
struct TileChoice {
  int bm, bn;
  int wm = 2, wn = 2;
  bool planned = true;
};
constexpr TileChoice kTiles[] = {
    {256, 128}, {128, 256}, {128, 192}, {64, 384}, {128, 128}, {64, 256}, {64, 192},
    {64, 128},  {32, 256},  {64, 64},   {32, 128}, {32, 64},   {32, 32},
    // eight waves (two per SIMD) on large tiles, planned by choose_tile8
    {256, 256, 4, 2, false}, {256, 192, 4, 2, false}, {128, 384, 2, 4, false},
    {256, 128, 4, 2, false}, {128, 256, 2, 4, false}, {128, 192, 2, 4, false},
    {128, 128, 2, 4, false}, {32, 64, 2, 4, false}, {64, 64, 2, 4, false},
    {32, 128, 2, 4, false}};
constexpr int kMinTiles = 256;

// Ring depths and stage lengths the pipelined kernel is built for; a
// combination is usable when the ring fits in LDS and its outstanding copies
// fit the vmcnt counter.
constexpr int kLdsBytes = 160 * 1024;
// Rings stay within 144 KB: a workgroup with more LDS (152 or 160 KB)
// measured 25-35 % slower on the same work.
constexpr int kLdsBudget = 144 * 1024;

// `waves` is the tile's wave count (4: 2 x 2, 8: 4 x 2 or 2 x 4); a wave
// issues at most ceil(load blocks / waves) copies per stage.
constexpr bool depth_ok(int bm, int bn, int ns, int rb, int waves = 4) {
  return ns * (bm + bn) * rb <= kLdsBytes &&
         (ns - 2) * (((bm + bn) * rb / 1024 + waves - 1) / waves) < 64;
}

template <typename In, int BM, int BN, int NS, int RB, int WM, int WN>
hipError_t launch_depth(const void* x, const void* W, const float* lb, float* out, int T,
                        int d, int E, int splits, hipStream_t s, const SelectArgs& sa) {
  if constexpr (depth_ok(BM, BN, NS, RB, WM * WN))
    return launch_pipe<In, BM, BN, NS, RB, WM, WN>(x, W, lb, out, T, d, E, splits, s, sa);
  return hipErrorInvalidValue;
}

// Split rings (x three stages deep, W two) for the eight-wave tiles whose
// combined ring fits only two stages deep in the LDS budget: every wave
// copies whole 1-KB blocks of x and of W.
constexpr bool split_ring_ok(int bm, int bn, int rb, int waves) {
  const int rpi = 1024 / rb;
  return waves == 8 && rb == 128 && bm % (rpi * waves) == 0 && bn % (rpi * waves) == 0 &&
         (3 * bm + 2 * bn) * rb <= kLdsBudget && 3 * (bm + bn) * rb > kLdsBudget;
}

template <typename In, int BM, int BN, int RB, int WM, int WN>
hipError_t launch_split(const void* x, const void* W, const float* lb, float* out, int T,
                        int d, int E, int splits, hipStream_t s, const SelectArgs& sa) {
  if constexpr (split_ring_ok(BM, BN, RB, WM * WN))
    return launch_pipe<In, BM, BN, 3, RB, WM, WN, NoSel, 2>(x, W, lb, out, T, d, E, splits, s,
                                                            sa);
  return hipErrorInvalidValue;
}

// Ring depths 2..4; 64-byte stages (the deep rings of large tiles) also 5..8.
template <typename In, int BM, int BN, int RB, int WM, int WN>
hipError_t launch_rb(const GatePlan& g, const void* x, const void* W, const float* lb,
                     float* out, int T, int d, int E, hipStream_t s, const SelectArgs& sa) {
  if constexpr (RB == 64) {
    switch (g.ns) {
      case 8: return launch_depth<In, BM, BN, 8, RB, WM, WN>(x, W, lb, out, T, d, E, g.splits, s, sa);
      case 7: return launch_depth<In, BM, BN, 7, RB, WM, WN>(x, W, lb, out, T, d, E, g.splits, s, sa);
      case 6: return launch_depth<In, BM, BN, 6, RB, WM, WN>(x, W, lb, out, T, d, E, g.splits, s, sa);
      case 5: return launch_depth<In, BM, BN, 5, RB, WM, WN>(x, W, lb, out, T, d, E, g.splits, s, sa);
      default: break;
    }
  }
  switch (g.ns) {
    case 4: return launch_depth<In, BM, BN, 4, RB, WM, WN>(x, W, lb, out, T, d, E, g.splits, s, sa);
    case 3:
      if (g.nsw == 2)
        return launch_split<In, BM, BN, RB, WM, WN>(x, W, lb, out, T, d, E, g.splits, s, sa);
      return launch_depth<In, BM, BN, 3, RB, WM, WN>(x, W, lb, out, T, d, E, g.splits, s, sa);
    default: return launch_depth<In, BM, BN, 2, RB, WM, WN>(x, W, lb, out, T, d, E, g.splits, s, sa);
  }
}

template <typename In, int BM, int BN, int KB, int WM = 2, int WN = 2>
hipError_t launch_ns(const GatePlan& g, const void* x, const void* W, const float* lb,
                     float* out, int T, int d, int E, hipStream_t s, const SelectArgs& sa) {
  if (!g.pipe) {
    if constexpr (WM == 2 && WN == 2) return launch_tile<In, BM, BN, KB>(x, W, lb, out, T, d, E, s);
    return hipErrorInvalidValue;  // 8-wave tiles are planned for the pipelined kernel only
  }
  if constexpr (WM * WN == 8 && sizeof(In) != 2) {
    return hipErrorInvalidValue;  // 8-wave tiles: bf16 only
  } else {
    switch (g.rb) {
      case 512: return launch_rb<In, BM, BN, 512, WM, WN>(g, x, W, lb, out, T, d, E, s, sa);
      case 256: return launch_rb<In, BM, BN, 256, WM, WN>(g, x, W, lb, out, T, d, E, s, sa);
      case 64:
        if constexpr (WM * WN == 8)
          return launch_rb<In, BM, BN, 64, WM, WN>(g, x, W, lb, out, T, d, E, s, sa);
        return hipErrorInvalidValue;  // 64-byte stages: 8-wave tiles only
      default: return launch_rb<In, BM, BN, 128, WM, WN>(g, x, W, lb, out, T, d, E, s, sa);
    }
  }
}

template <typename In>
hipError_t launch_choice(const GatePlan& g, const void* x, const void* W, const float* lb,
                         float* out, int T, int d, int E, hipStream_t s, const SelectArgs& sa) {
#define MOE_TILE(BM_, BN_, KB_)                                             \
  if (g.bm == BM_ && g.bn == BN_ && g.wm * g.wn == 4)                        \
    return launch_ns<In, BM_, BN_, KB_>(g, x, W, lb, out, T, d, E, s, sa);
#define MOE_TILE8(BM_, BN_, WM_, WN_)                                       \
  if (g.bm == BM_ && g.bn == BN_ && g.wm == WM_ && g.wn == WN_)              \
    return launch_ns<In, BM_, BN_, 128, WM_, WN_>(g, x, W, lb, out, T, d, E, s, sa);
  MOE_TILE(256, 128, 128)
  MOE_TILE(128, 256, 128)
  MOE_TILE(128, 192, 128)
  MOE_TILE(64, 384, 128)
  MOE_TILE(128, 128, 128)
  MOE_TILE(64, 256, 128)
  MOE_TILE(64, 192, 128)
  MOE_TILE(64, 128, 128)
  MOE_TILE(32, 256, 128)
  MOE_TILE(64, 64, 256)
  MOE_TILE(32, 128, 256)
  MOE_TILE(32, 64, 256)
  MOE_TILE(32, 32, 256)
  MOE_TILE8(256, 256, 4, 2)
  MOE_TILE8(256, 192, 4, 2)
  MOE_TILE8(128, 384, 2, 4)
  MOE_TILE8(256, 128, 4, 2)
  MOE_TILE8(128, 256, 2, 4)
  MOE_TILE8(128, 192, 2, 4)
  MOE_TILE8(128, 128, 2, 4)
  MOE_TILE8(32, 64, 2, 4)
  MOE_TILE8(64, 64, 2, 4)
  MOE_TILE8(32, 128, 2, 4)
#undef MOE_TILE
#undef MOE_TILE8
  return hipErrorInvalidValue;
}

// Largest tile with at least `min_useful` non-padding columns that gives at
// least `min_tiles` workgroups, or {0, 0}.
TileChoice largest_tile(int T, int E, long min_tiles, double min_useful) {
  TileChoice best = {0, 0};
  double best_work = -1.0, best_useful = 0.0;
  for (const auto& t : kTiles) {
    if (!t.planned) continue;
    const int n_n = (E + t.bn - 1) / t.bn;
    const double useful = (double)E / (n_n * t.bn);
    if (useful < min_useful) continue;
    const long tiles = (long)((T + t.bm - 1) / t.bm) * n_n;
    const double work = (double)t.bm * t.bn * useful;  // useful outputs per tile
    // equal useful work: the tile with less padding (fewer wasted bytes)
    if (tiles >= min_tiles && (work > best_work || (work == best_work && useful > best_useful))) {
      best = t;
      best_work = work;
      best_useful = useful;
    }
  }
  return best;
}

// Bytes re-read from L2 bound these kernels (about 13 TB/s of L2-to-CU reads
// on the whole chip, against about 6 TB/s of HBM streaming), so tiles are as
// large as the chip allows: two workgroups per CU (512 tiles) when unpadded
// tiles of at least 128 x 128 still give that many -- eight waves per CU
// hide more latency than a deeper ring -- else one per CU (256 tiles, >= 74 %
// of the columns useful), else, for few tokens, the widest tile 32 rows high.
TileChoice choose_tile(int T, int E) {
  const TileChoice two = largest_tile(T, E, 2 * kMinTiles, 1.0);
  if (two.bm * two.bn >= 128 * 128) return two;
  const TileChoice one = largest_tile(T, E, kMinTiles, 0.74);
  if (one.bm > 0) return one;
  TileChoice fallback = {32, 32};
  double fallback_work = -1.0;
  for (const auto& t : kTiles) {
    const int n_n = (E + t.bn - 1) / t.bn;
    const double useful = (double)E / (n_n * t.bn);
    if (t.planned && t.bm == 32 && useful >= 0.74 && t.bn * useful > fallback_work) {
      fallback = t;
      fallback_work = t.bn * useful;
    }
  }
  return fallback;
}

// Eight-wave tiles (two waves per SIMD) for bf16 contractions that fill the
// chip: the tile and K split with the lowest estimated time.  Row pieces
// re-read from L2 bound these kernels (measured: about 21 bytes per clock
// per CU, 13 TB/s on the chip) unless x's single pass from HBM (about
// 6 TB/s) takes longer; a K split cuts each workgroup's share of the rows
// but writes one more T x E fp32 partial array, which the selection reads
// back.  Candidates give one or two workgroups per CU and leave at least
// eight 128-byte row pieces per split.  {0, 0}: none qualifies.
TileChoice choose_tile8(int T, int d, int E, bool allow_split, int* splits) {
  constexpr double kL2PerCu = 21.0 * 2.4e9;  // bytes/s
  constexpr double kHbm = 6.0e12;            // bytes/s
  constexpr int kCus = 256;
  const double row = 2.0 * d;                // bf16 row bytes
  const int64_t pieces = ((int64_t)d * 2 + 127) / 128;
  TileChoice best = {0, 0};
  double best_est = 0.0;
  int best_nn = 0;
  *splits = 1;
  for (const auto& t : kTiles) {
    if (t.wm * t.wn != 8) continue;
    const int n_n = (E + t.bn - 1) / t.bn;
    if ((double)E / (n_n * t.bn) < 0.74) continue;
    const long tiles = (long)((T + t.bm - 1) / t.bm) * n_n;
    for (int S = 1; S <= 8; S *= 2) {
      if (S > 1 && !allow_split) break;
      const long wgs = tiles * S;
      if (wgs < kMinTiles || wgs > 2 * kCus || pieces / S < 8) continue;
      const double per_cu = (double)((wgs + kCus - 1) / kCus) * (t.bm + t.bn) * row / S;
      const double t_l2 = per_cu / kL2PerCu;
      const double t_hbm = ((double)T * row + (double)E * row + (double)S * T * E * 4) / kHbm;
      const double t_part = (double)(S - 1) * T * E * 4 / kHbm;
      const double est = std::max(t_l2, t_hbm) + t_part;
      // ties: fewer N tiles (whole rows of logits per workgroup)
      if (best.bm == 0 || est < best_est * 0.999 ||
          (est <= best_est * 1.001 && n_n < best_nn)) {
        best = t;
        best_est = est;
        best_nn = n_n;
        *splits = S;
      }
    }
  }
  return best;
}

// Stage length and ring depth of the pipelined kernel.  The ring hides
// memory latency and takes the LDS that the workgroups sharing a CU leave it
// (all of it at one workgroup per CU, half at two).  Four-wave tiles: the
// longest row segment that still keeps two stages in flight (NS >= 3), else
// the longest with NS = 2.  Eight-wave tiles: small ones 256-byte stages
// three deep (measured on the Qwen3-like shape), large ones 128-byte stages
// as deep as fits.
void choose_ring(GatePlan& g, long wgs) {
  const int budget = (wgs > kMinTiles ? kLdsBytes / 2 : kLdsBudget);
  const int waves = g.wm * g.wn;
  if (waves == 8) {
    if (g.bm * g.bn < 128 * 128 && depth_ok(g.bm, g.bn, 3, 256, 8) &&
        3 * (g.bm + g.bn) * 256 <= budget) {
      g.rb = 256;
      g.ns = 3;
      return;
    }
    for (int ns : {4, 3, 2})
      if (depth_ok(g.bm, g.bn, ns, 128, 8) && ns * (g.bm + g.bn) * 128 <= budget) {
        g.rb = 128;
        g.ns = ns;
        // two stages of a large tile leave one stage of x in flight: the
        // loop then waits on each stage's round trip (DeepSeek-V4-like gate,
        // 256 x 192); x three deep and W two deep keep two x stages in flight
        if (ns == 2 && budget == kLdsBudget && split_ring_ok(g.bm, g.bn, 128, 8)) {
          g.ns = 3;
          g.nsw = 2;
        }
        return;
      }
    g.rb = 64;
    g.ns = 2;
    return;
  }
  const int budget4 = (wgs > kMinTiles ? kLdsBytes / 2 : kLdsBudget);
  for (int ns_min : {3, 2})
    for (int rb : {256, 128})
      for (int ns : {4, 3, 2})
        if (ns >= ns_min && depth_ok(g.bm, g.bn, ns, rb, waves) &&
            ns * (g.bm + g.bn) * rb <= budget4) {
          g.rb = rb;
          g.ns = ns;
          return;
        }
  g.rb = 128;
  g.ns = 2;
}

}  // namespace

GatePlan plan_gate(int32_t T, int32_t d, int32_t E, int32_t dtype, bool aligned,
                   bool allow_split) {
  const int esz = dtype == 1 ? 2 : 4;
  GatePlan g;
  const TileChoice c0 = choose_tile(T, E);
  g.bm = c0.bm;
  g.bn = c0.bn;
  g.wm = c0.wm;
  g.wn = c0.wn;
  g.splits = 1;
  // the pipelined kernel needs 16-byte aligned rows and byte offsets below 2^31
  g.pipe = aligned && ((int64_t)d * esz % 16 == 0) && (int64_t)T * d * esz < (1ll << 31) &&
           (int64_t)E * d * esz < (1ll << 31) && std::getenv("MOE_GATE_NOPIPE") == nullptr;
  // Large bf16 contractions take eight-wave tiles.  Otherwise: large
  // four-wave tiles at one workgroup per CU over a long K split K in two, so
  // that two workgroups share each CU; a tiny grid (few tokens and experts)
  // splits K up to 8 ways so more CUs take part, keeping at least four
  // 128-byte row pieces per split.
  const int64_t pieces = ((int64_t)d * esz + 127) / 128;
  int splits8 = 1;
  const TileChoice c8 =
      (g.pipe && dtype == 1) ? choose_tile8(T, d, E, allow_split, &splits8) : TileChoice{0, 0};
  if (c8.bm > 0) {
    g.bm = c8.bm;
    g.bn = c8.bn;
    g.wm = c8.wm;
    g.wn = c8.wn;
    g.splits = splits8;
  } else if (g.pipe && dtype == 1 && g.bm * g.bn < 128 * 128) {
    // Eight waves on the same small tile (two per SIMD; measured on the
    // Qwen3-like shape, 32 x 64: 12.7 -> 10.9 us)
    for (const auto& t : kTiles)
      if (t.wm * t.wn == 8 && t.bm == g.bm && t.bn == g.bn) {
        g.wm = t.wm;
        g.wn = t.wn;
      }
  }
  if (c8.bm == 0 && g.pipe && allow_split) {
    const long tiles = (long)((T + g.bm - 1) / g.bm) * ((E + g.bn - 1) / g.bn);
    if (tiles < 2 * kMinTiles && tiles * 2 <= 2 * kMinTiles && g.bm * g.bn >= 128 * 128 &&
        pieces >= 64)
      g.splits = 2;
    while (tiles * g.splits < 64 && g.splits < 8 && pieces / (2 * g.splits) >= 4) g.splits *= 2;
  }
  if (const char* env = std::getenv("MOE_GATE_TILE")) {  // "BMxBN" or "BMxBNw8"
    int bm = 0, bn = 0, w = 4;
    if (std::sscanf(env, "%dx%dw%d", &bm, &bn, &w) >= 2)
      for (const auto& t : kTiles)
        if (t.bm == bm && t.bn == bn && t.wm * t.wn == w && (w == 4 || (g.pipe && dtype == 1))) {
          g.bm = bm;
          g.bn = bn;
          g.wm = t.wm;
          g.wn = t.wn;
        }
  }
  if (const char* env = std::getenv("MOE_GATE_SPLITS"))
    if (g.pipe && allow_split) g.splits = std::max(1, std::min(8, std::atoi(env)));
  const long wgs = (long)((T + g.bm - 1) / g.bm) * ((E + g.bn - 1) / g.bn) * g.splits;
  choose_ring(g, wgs);
  const int waves = g.wm * g.wn;
  if (const char* env = std::getenv("MOE_GATE_RB")) {
    const int rb = std::atoi(env);
    if ((rb == 128 || rb == 256 || rb == 512 || (rb == 64 && waves == 8)) &&
        depth_ok(g.bm, g.bn, 2, rb, waves)) {
      g.rb = rb;
      g.nsw = 0;
    }
  }
  if (const char* env = std::getenv("MOE_GATE_NS")) {
    const int ns = std::atoi(env);
    if (ns >= 2 && ns <= (g.rb == 64 ? 8 : 4)) {
      g.ns = ns;
      g.nsw = 0;
    }
  }
  if (const char* env = std::getenv("MOE_GATE_NSW")) {  // tuning: 0 one ring, 2 split
    g.nsw = 0;
    if (std::atoi(env) == 2 && split_ring_ok(g.bm, g.bn, g.rb, waves)) {
      g.ns = 3;
      g.nsw = 2;
    }
  }
  if (g.nsw == 0 && !depth_ok(g.bm, g.bn, g.ns, g.rb, waves)) g.ns = 2;
  return g;
}

// Gate + selection in one kernel.  Built for the whole-row eight-wave tiles
// of E <= 128 experts (256 x 128 at a 3-deep ring, 128 x 128 at a 4-deep
// ring, 128-byte stages) and the selection shapes of such E (8 lanes x 16
// experts, 16 x 8).
namespace {

struct FusedTile {
  int bm, bn, wm, wn, ns, rb;
};
constexpr FusedTile kFusedTiles[] = {{256, 128, 4, 2, 3, 128}, {128, 128, 2, 4, 4, 128}};

template <int BM, int BN, int WM, int WN, int NS, int RB, int LPT, int VPL>
hipError_t launch_fused_shape(bool mono, bool hist, const void* x, const void* W,
                              const float* lb, float* logits, int T, int d, int E,
                              const SelectArgs& sa, hipStream_t s) {
  // k = 4 compiled into the selection of the 256-row tiles' monotone case
  // (top-4 over raw or softmax scores, as gpt-oss routes); other k at run time
  if constexpr (BM == 256) {
    if (mono && sa.c.k == 4) {
      if (hist)
        return launch_pipe<uint16_t, BM, BN, NS, RB, WM, WN, FusedSel<LPT, VPL, true, true, 4>>(
            x, W, lb, logits, T, d, E, 1, s, sa);
      return launch_pipe<uint16_t, BM, BN, NS, RB, WM, WN, FusedSel<LPT, VPL, true, false, 4>>(
          x, W, lb, logits, T, d, E, 1, s, sa);
    }
  }
#define MOE_F(M_, H_)                                                                   \
  if (mono == M_ && hist == H_)                                                         \
    return launch_pipe<uint16_t, BM, BN, NS, RB, WM, WN, FusedSel<LPT, VPL, M_, H_>>(   \
        x, W, lb, logits, T, d, E, 1, s, sa);
  MOE_F(true, true)
  MOE_F(true, false)
  MOE_F(false, true)
  MOE_F(false, false)
#undef MOE_F
  return hipErrorInvalidValue;
}

template <int BM, int BN, int WM, int WN, int NS, int RB>
hipError_t launch_fused_tile(int lpt, int vpl, bool mono, bool hist, const void* x,
                             const void* W, const float* lb, float* logits, int T, int d, int E,
                             const SelectArgs& sa, hipStream_t s) {
  if (lpt == 8 && vpl == 16)
    return launch_fused_shape<BM, BN, WM, WN, NS, RB, 8, 16>(mono, hist, x, W, lb, logits, T, d,
                                                             E, sa, s);
  if (lpt == 16 && vpl == 8)
    return launch_fused_shape<BM, BN, WM, WN, NS, RB, 16, 8>(mono, hist, x, W, lb, logits, T, d,
                                                             E, sa, s);
  return hipErrorInvalidValue;
}

bool grouped_cfg(const RouteCfg& c) { return c.n_groups > 1 && c.topk_groups < c.n_groups; }

}  // namespace

int gate_select_tokens(const GatePlan& g, int32_t dtype, const RouteCfg& c) {
  if (!g.pipe || dtype != 1 || g.splits != 1 || g.bn < c.E || c.E > kFusedMaxE ||
      std::getenv("MOE_NO_FUSED_SELECT"))
    return 0;
  int lpt = 0, vpl = 0;
  select_shape(c, &lpt, &vpl);
  if (!((lpt == 8 && vpl == 16) || (lpt == 16 && vpl == 8))) return 0;
  for (const auto& f : kFusedTiles)
    if (f.bm == g.bm && f.bn == g.bn && f.wm == g.wm && f.wn == g.wn && f.ns == g.ns &&
        f.rb == g.rb)
      return g.bm;
  return 0;
}

hipError_t launch_gate_select(const GatePlan& g, int32_t dtype, const void* x, const void* W,
                              const float* logit_bias, float* logits, const SelectArgs& sa,
                              hipStream_t stream) {
  const RouteCfg& c = sa.c;
  if (gate_select_tokens(g, dtype, c) == 0 || (sa.write_logits && !logits))
    return hipErrorInvalidValue;
  if (c.T == 0) return hipSuccess;
  int lpt = 0, vpl = 0;
  select_shape(c, &lpt, &vpl);
  const bool mono = sa.select_bias == nullptr && !grouped_cfg(c) && c.k_per_group == 0;
  const bool hist = sa.hist != nullptr;
  if (g.bm == 256)
    return launch_fused_tile<256, 128, 4, 2, 3, 128>(lpt, vpl, mono, hist, x, W, logit_bias,
                                                     logits, c.T, c.d, c.E, sa, stream);
  return launch_fused_tile<128, 128, 2, 4, 4, 128>(lpt, vpl, mono, hist, x, W, logit_bias,
                                                   logits, c.T, c.d, c.E, sa, stream);
}

hipError_t launch_gate_gemm(const GatePlan& g, int32_t dtype, const void* x, const void* W,
                            const float* logit_bias, float* out, int32_t T, int32_t d,
                            int32_t E, hipStream_t stream, int32_t* zero, int32_t zero_words) {
  if (T == 0) return hipSuccess;
  if (zero_words > 0 && !g.pipe) return hipErrorInvalidValue;  // the pipelined kernel zeroes
  SelectArgs sa{};
  sa.zero = zero;
  sa.zero_words = zero_words;
  if (dtype == 1) return launch_choice<uint16_t>(g, x, W, logit_bias, out, T, d, E, stream, sa);
  return launch_choice<float>(g, x, W, logit_bias, out, T, d, E, stream, sa);
}

}  // namespace moe
