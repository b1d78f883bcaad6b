// Max-over-offsets score kernel of libtri for gfx950.
//
// "The future-offset average in TriAttention can be precomputed", section "What it saves, and
// what it does not": the fold relies on the mean over offsets being linear and does not apply to
// the variant that takes the maximum over the offsets, so each offset is evaluated:
//     S_max(k) = max_{delta in D} Re{ sum_f E[q_f] conj(k_f) e^{i omega_f (Delta + delta)} }.
// Rotations compose by adding angles (section "The same score, read as arrows in the plane"):
// e^{i w (Delta + delta)} = e^{i w Delta} e^{i w delta}. Per key and band the kernel evaluates
// e^{i w Delta} once (fixed-point phase, hardware sine and cosine) and forms
//     P = x cos(w Delta) - y sin(w Delta),  Q = x sin(w Delta) + y cos(w Delta)
// (x, y as in the averaged score, with the raw center); then per offset the band's term is
//     P cos(w delta) - Q sin(w delta),
// two FMAs against a table of (cos, sin)(w_f delta) built in LDS once per workgroup. The lanes of
// a row add each offset's terms with DPP and keep the running maximum. For d = 128 the offset
// loop is a matrix product instead and runs on the matrix cores (score_max_mfma_kernel).
#include "score_device.h"

namespace tri {
namespace {

using dev::kDtBf16;
using dev::kDtF32;
using dev::kHalfSplit;
using dev::kInterleaved;
using dev::order_key;
using namespace sdev;

constexpr int kMaxThreads = 256;
constexpr int kMaxRowsPerLoad = 4;

template <int D>
constexpr int max_rows_per_block() { return 256; }

// This lane's four bands of one row at one offset: sum_j P_j cos(w_j delta) - Q_j sin(w_j delta),
// with w01 = (cos, sin) of bands 0 and 1 and w23 of bands 2 and 3.
__device__ __forceinline__ float band_terms(const float (&P)[4], const float (&Q)[4], const float4& w01,
                                            const float4& w23) {
  float v = fmaf(P[0], w01.x, -(Q[0] * w01.y));
  v = fmaf(P[1], w01.z, fmaf(-Q[1], w01.w, v));
  v = fmaf(P[2], w23.x, fmaf(-Q[2], w23.y, v));
  return fmaf(P[3], w23.z, fmaf(-Q[3], w23.w, v));
}

// Maximum over each aligned group of 16 lanes; every lane gets it.
__device__ __forceinline__ float group_max16(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // lane ^ 1
  v = fmaxf(v, dpp_f<0x4E>(v));   // lane ^ 2
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  return fmaxf(v, dpp_f<0x140>(v));  // row_mirror
}

template <int DT, int LAYOUT, int D, bool HIST>
__global__ __launch_bounds__(kMaxThreads) void score_max_kernel(ScoreArgs a, int chunks_per_unit, BandConst bc,
                                                                OffsetSet os) {
  constexpr int F = D / 2;
  constexpr int LPR = F / 4;
  constexpr int GPW = 64 / LPR;
  constexpr int M = kMaxRowsPerLoad;
  constexpr int ROWS_WAVE = GPW * M;
  constexpr int ROWS_ITER = ROWS_WAVE * (kMaxThreads / 64);
  constexpr int RPB = max_rows_per_block<D>();
  constexpr int ITERS = RPB / ROWS_ITER;
  static_assert(RPB % ROWS_ITER == 0, "rows per block");
  using L = RowLoad<DT, LAYOUT, D>;
  using KT = typename L::T;

  __shared__ __align__(16) float2 tab[kMaxOffsets][F];  // (cos, sin)(omega_f delta)
  __shared__ uint32_t lhist[HIST ? kHistBins : 1];

  const int unit = blockIdx.x / chunks_per_unit;
  const int chunk = blockIdx.x - unit * chunks_per_unit;
  const dev::UnitRows ur = dev::unit_rows(a.row_off, unit, a.total_rows, a.max_rows);
  const int64_t beg = ur.beg, end = ur.beg + ur.n;
  const int64_t r0 = beg + (int64_t)chunk * RPB;
  if (r0 >= end) return;
  const int64_t r1 = (end - r0 < RPB) ? end : r0 + RPB;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l = lane % LPR;
  const int gw = lane / LPR;
  const int n_off = os.n;

  const char* kbase = static_cast<const char*>(a.keys) + r0 * L::kRowBytes;
  const int32_t* pbase = a.pos + r0;
  const uint32_t last = (uint32_t)(r1 - r0 - 1);
  const uint32_t wave_row = (uint32_t)(wave * ROWS_WAVE + gw);
  KT kb[M];
  int32_t pb[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t row = min(wave_row + m * GPW, last);
    kb[m] = L::load(kbase, row, l);
    pb[m] = load_pos(pbase, row);
  }

  // the offset table, the histogram, and this lane's constants
  for (int i = threadIdx.x; i < n_off * F; i += kMaxThreads) {
    const int o = i / F, f = i - o * F;
    const uint32_t dl = os.delta[o];
    const float rev = band_phase(dl, (float)dl, bc.step[f] & 0x7FFFFFu, bc.resid[f]);
    tab[o][f] = make_float2(__builtin_amdgcn_cosf(rev), __builtin_amdgcn_sinf(rev));
  }
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < kHistBins; i += kMaxThreads) lhist[i] = 0u;
  }
  uint32_t step[4];
  float resid[4];
  float cre[4], cim[4];
  {
    const float4* mp = reinterpret_cast<const float4*>(a.mu + ((size_t)unit * F + 4 * l) * 2);
    const float4 m0 = mp[0], m1 = mp[1];
    cre[0] = m0.x; cim[0] = m0.y; cre[1] = m0.z; cim[1] = m0.w;
    cre[2] = m1.x; cim[2] = m1.y; cre[3] = m1.z; cim[3] = m1.w;
#pragma unroll
    for (int j = 0; j < 4; ++j) { step[j] = bc.step[4 * l + j] & 0x7FFFFFu; resid[j] = bc.resid[4 * l + j]; }
  }
  CenterCoef<DT> cc;
  cc.init(cre, cim);
  const int32_t t = a.t_now[unit];
  __syncthreads();

  for (int it = 0; it < ITERS; ++it) {
    KT kc[M];
    int32_t pc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) { kc[m] = kb[m]; pc[m] = pb[m]; }
    const uint32_t base = wave_row + (uint32_t)(it * ROWS_ITER);
    if (it + 1 < ITERS) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint32_t row = min(base + ROWS_ITER + m * GPW, last);
        kb[m] = L::load(kbase, row, l);
        pb[m] = load_pos(pbase, row);
      }
    }
    // per row and band: the center term rotated by the distance, (P, Q)
    float P[M][4], Q[M][4];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t dl = (uint32_t)(t - pc[m]);
      const float df = (float)dl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float rev = band_phase(dl, df, step[j], resid[j]);
        const float sn = __builtin_amdgcn_sinf(rev);
        const float cs = __builtin_amdgcn_cosf(rev);
        float x, y;
        cc.xy(kc[m], j, x, y);
        P[m][j] = fmaf(x, cs, -(y * sn));
        Q[m][j] = fmaf(x, sn, y * cs);
      }
    }
    // offsets outer: one table read serves the M rows of this lane
    float best[M];
#pragma unroll
    for (int m = 0; m < M; ++m) best[m] = -__builtin_inff();
    for (int o = 0; o < n_off; ++o) {
      const float4 w01 = *reinterpret_cast<const float4*>(&tab[o][4 * l]);
      const float4 w23 = *reinterpret_cast<const float4*>(&tab[o][4 * l + 2]);
#pragma unroll
      for (int m = 0; m < M; ++m) best[m] = fmaxf(best[m], group_sum<LPR>(band_terms(P[m], Q[m], w01, w23)));
    }
    if (l < M) {
      float v = best[0];
#pragma unroll
      for (int m = 1; m < M; ++m) v = (l == m) ? best[m] : v;
      const uint32_t row = base - gw + l * GPW + gw;
      if (row <= last) {
        a.scores[r0 + row] = v;
        if constexpr (HIST) atomicAdd(&lhist[order_key(v) >> kHistShift], 1u);
      }
    }
  }

  if constexpr (HIST) {
    __syncthreads();
    uint32_t* gh = a.hist + (size_t)unit * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kMaxThreads) {
      const uint32_t c = lhist[i];
      if (c) atomicAdd(&gh[i], c);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// d = 128: the offset loop as a matrix product on the matrix cores
// ---------------------------------------------------------------------------------------------
//
// For one row, S(delta_o) = sum_f P_f cos(w_f delta_o) - Q_f sin(w_f delta_o) is the product of
// the row [P_0..P_63, Q_0..Q_63] with column o of W = [cos(w_f delta_o); -sin(w_f delta_o)]:
// 16 rows x 128 x 16 offsets per v_mfma_f32_16x16x32_bf16 tile (K = 32 per instruction, four
// steps). Each operand is split into bf16 hi + lo (x = hi + lo + O(2^-16 x)) and the product is
// hi*hi + hi*lo + lo*hi, accumulated in fp32. A wave writes its 16 rows' P, Q (hi and lo) to an
// LDS tile in the lane layout the instruction takes (lane L: row L % 16, k = 8 (L / 16) + i), and
// holds W in registers for the whole workgroup. Offsets past the last repeat it (the maximum
// does not change). The result tile gives lane L offset L % 16 of rows 4 (L / 16) + i; a DPP
// maximum over the 16 lanes of each row group finishes the row.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4m __attribute__((ext_vector_type(4)));

constexpr int kMfmaRowsPerBlock = 512;
constexpr int kTileStride = 136;  // bf16 per LDS tile row: 128 + 8 (16 bytes of padding against bank conflicts)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2m __attribute__((ext_vector_type(2)));

// x = hi + lo with hi, lo bf16 (round to nearest even both times)
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}
// the same for a pair (one packed conversion each for hi and lo)
__device__ __forceinline__ void split_bf16x2(float x0, float x1, bf16x2& hi, bf16x2& lo) {
  const f32x2m v = {x0, x1};
  hi = __builtin_convertvector(v, bf16x2);
  lo = __builtin_convertvector(v - __builtin_convertvector(hi, f32x2m), bf16x2);
}

template <int DT, int LAYOUT, bool HIST, int NT>  // NT: tiles of 16 offsets
__global__ __launch_bounds__(kMaxThreads) void score_max_mfma_kernel(ScoreArgs a, int chunks_per_unit, BandConst bc,
                                                                     OffsetSet os) {
  constexpr int D = 128, F = 64, LPR = 16, GPW = 4, M = 4;
  constexpr int ROWS_WAVE = GPW * M;  // 16: one matrix tile of rows
  constexpr int WAVES = kMaxThreads / 64;
  constexpr int ROWS_ITER = ROWS_WAVE * WAVES;
  constexpr int RPB = kMfmaRowsPerBlock;
  constexpr int ITERS = RPB / ROWS_ITER;
  static_assert(RPB % ROWS_ITER == 0, "rows per block");
  using L = RowLoad<DT, LAYOUT, D>;
  using KT = typename L::T;

  __shared__ __align__(16) float2 tab[kMaxOffsets][F];                  // (cos, sin)(omega_f delta)
  __shared__ __align__(16) __bf16 tile[WAVES][2][ROWS_WAVE][kTileStride];  // per wave: hi, lo
  __shared__ uint32_t lhist[HIST ? kHistBins : 1];

  const int unit = blockIdx.x / chunks_per_unit;
  const int chunk = blockIdx.x - unit * chunks_per_unit;
  const dev::UnitRows ur = dev::unit_rows(a.row_off, unit, a.total_rows, a.max_rows);
  const int64_t beg = ur.beg, end = ur.beg + ur.n;
  const int64_t r0 = beg + (int64_t)chunk * RPB;
  if (r0 >= end) return;
  const int64_t r1 = (end - r0 < RPB) ? end : r0 + RPB;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l = lane % LPR;   // setup layout: bands 4l .. 4l+3 of rows m*GPW + gw
  const int gw = lane / LPR;
  const int mc = lane & 15;   // matrix layout: row (A) or offset column (B, result) ...
  const int mq = lane >> 4;   // ... and k block 8*mq .. 8*mq+7
  const int n_off = os.n;

  const char* kbase = static_cast<const char*>(a.keys) + r0 * L::kRowBytes;
  const int32_t* pbase = a.pos + r0;
  const uint32_t last = (uint32_t)(r1 - r0 - 1);
  const uint32_t wave_row = (uint32_t)(wave * ROWS_WAVE + gw);
  KT kb[M];
  int32_t pb[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t row = min(wave_row + m * GPW, last);
    kb[m] = L::load(kbase, row, l);
    pb[m] = load_pos(pbase, row);
  }

  // the offset table, the histogram, and this lane's constants
  for (int i = threadIdx.x; i < n_off * F; i += kMaxThreads) {
    const int o = i / F, f = i - o * F;
    const uint32_t dl = os.delta[o];
    const float rev = band_phase(dl, (float)dl, bc.step[f] & 0x7FFFFFu, bc.resid[f]);
    tab[o][f] = make_float2(__builtin_amdgcn_cosf(rev), __builtin_amdgcn_sinf(rev));
  }
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < kHistBins; i += kMaxThreads) lhist[i] = 0u;
  }
  uint32_t step[4];
  float resid[4];
  float cre[4], cim[4];
  {
    const float4* mp = reinterpret_cast<const float4*>(a.mu + ((size_t)unit * F + 4 * l) * 2);
    const float4 m0 = mp[0], m1 = mp[1];
    cre[0] = m0.x; cim[0] = m0.y; cre[1] = m0.z; cim[1] = m0.w;
    cre[2] = m1.x; cim[2] = m1.y; cre[3] = m1.z; cim[3] = m1.w;
#pragma unroll
    for (int j = 0; j < 4; ++j) { step[j] = bc.step[4 * l + j] & 0x7FFFFFu; resid[j] = bc.resid[4 * l + j]; }
  }
  CenterCoef<DT> cc;
  cc.init(cre, cim);
  const int32_t t = a.t_now[unit];
  __syncthreads();

  // W in registers: tile tt, step s: column o = 16 tt + mc (the last offset past n_off), rows
  // k = 32 s + 8 mq + i: cos(w_k delta_o) for k < 64, -sin(w_{k-64} delta_o) above
  bf16x8 whi[NT][4], wlo[NT][4];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int o = min(16 * tt + mc, n_off - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = 32 * s + 8 * mq + i;
        const float2 cs = tab[o][k & 63];
        __bf16 h, lo;
        split_bf16(k < 64 ? cs.x : -cs.y, h, lo);
        whi[tt][s][i] = h;
        wlo[tt][s][i] = lo;
      }
    }
  }

  __bf16* th = &tile[wave][0][0][0];
  __bf16* tl = &tile[wave][1][0][0];
  for (int it = 0; it < ITERS; ++it) {
    KT kc[M];
    int32_t pc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) { kc[m] = kb[m]; pc[m] = pb[m]; }
    const uint32_t base = (uint32_t)(it * ROWS_ITER + wave * ROWS_WAVE);  // the wave's first row
    if (it + 1 < ITERS) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint32_t row = min(wave_row + (uint32_t)((it + 1) * ROWS_ITER) + m * GPW, last);
        kb[m] = L::load(kbase, row, l);
        pb[m] = load_pos(pbase, row);
      }
    }
    // per row and band: (P, Q), split, into the wave's tile (row m*GPW + gw; k = 4l + j, 64 + 4l + j)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t dl = (uint32_t)(t - pc[m]);
      const float df = (float)dl;
      float P[4], Q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float rev = band_phase(dl, df, step[j], resid[j]);
        const float sn = __builtin_amdgcn_sinf(rev);
        const float cs = __builtin_amdgcn_cosf(rev);
        float x, y;
        cc.xy(kc[m], j, x, y);
        P[j] = fmaf(x, cs, -(y * sn));
        Q[j] = fmaf(x, sn, y * cs);
      }
      bf16x2 ph0, ph1, pl0, pl1, qh0, qh1, ql0, ql1;
      split_bf16x2(P[0], P[1], ph0, pl0);
      split_bf16x2(P[2], P[3], ph1, pl1);
      split_bf16x2(Q[0], Q[1], qh0, ql0);
      split_bf16x2(Q[2], Q[3], qh1, ql1);
      const int rr = m * GPW + gw;
      *reinterpret_cast<bf16x4*>(th + rr * kTileStride + 4 * l) = bf16x4{ph0[0], ph0[1], ph1[0], ph1[1]};
      *reinterpret_cast<bf16x4*>(th + rr * kTileStride + 64 + 4 * l) = bf16x4{qh0[0], qh0[1], qh1[0], qh1[1]};
      *reinterpret_cast<bf16x4*>(tl + rr * kTileStride + 4 * l) = bf16x4{pl0[0], pl0[1], pl1[0], pl1[1]};
      *reinterpret_cast<bf16x4*>(tl + rr * kTileStride + 64 + 4 * l) = bf16x4{ql0[0], ql0[1], ql1[0], ql1[1]};
    }
    // the tile is this wave's own: its LDS operations run in order; keep the compiler's order too
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4m acc[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = f32x4m{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(th + mc * kTileStride + 32 * s + 8 * mq);
      const bf16x8 alo = *reinterpret_cast<const bf16x8*>(tl + mc * kTileStride + 32 * s + 8 * mq);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, whi[tt][s], acc[tt], 0, 0, 0);
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, wlo[tt][s], acc[tt], 0, 0, 0);
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, whi[tt][s], acc[tt], 0, 0, 0);
      }
    }
    // the next iteration rewrites the tile only after these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane L: offset column mc of rows 4 mq + i; maximum over the offsets, then over the 16 lanes
    float best[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[0][i];
#pragma unroll
      for (int tt = 1; tt < NT; ++tt) v = fmaxf(v, acc[tt][i]);
      best[i] = group_max16(v);
    }
    if (mc < 4) {
      const float v = mc == 0 ? best[0] : mc == 1 ? best[1] : mc == 2 ? best[2] : best[3];
      const uint32_t row = base + 4 * mq + mc;
      if (row <= last) {
        a.scores[r0 + row] = v;
        if constexpr (HIST) atomicAdd(&lhist[order_key(v) >> kHistShift], 1u);
      }
    }
  }

  if constexpr (HIST) {
    __syncthreads();
    uint32_t* gh = a.hist + (size_t)unit * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kMaxThreads) {
      const uint32_t c = lhist[i];
      if (c) atomicAdd(&gh[i], c);
    }
  }
}

template <int DT, int LAYOUT, int NT>
hipError_t launch_mfma(const ScoreArgs& a, const BandConst& bc, const OffsetSet& os, hipStream_t s) {
  constexpr int RPB = kMfmaRowsPerBlock;
  const int64_t chunks = (a.max_rows + RPB - 1) / RPB;
  const int64_t grid = chunks * a.n_units;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b(kMaxThreads);
  if (a.hist) hipLaunchKernelGGL((score_max_mfma_kernel<DT, LAYOUT, true, NT>), g, b, 0, s, a, (int)chunks, bc, os);
  else hipLaunchKernelGGL((score_max_mfma_kernel<DT, LAYOUT, false, NT>), g, b, 0, s, a, (int)chunks, bc, os);
  return hipGetLastError();
}

template <int DT, int LAYOUT, int D>
hipError_t launch_t(const ScoreArgs& a, const BandConst& bc, const OffsetSet& os, hipStream_t s) {
  constexpr int RPB = max_rows_per_block<D>();
  const int64_t chunks = (a.max_rows + RPB - 1) / RPB;
  const int64_t grid = chunks * a.n_units;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b(kMaxThreads);
  if (a.hist) hipLaunchKernelGGL((score_max_kernel<DT, LAYOUT, D, true>), g, b, 0, s, a, (int)chunks, bc, os);
  else hipLaunchKernelGGL((score_max_kernel<DT, LAYOUT, D, false>), g, b, 0, s, a, (int)chunks, bc, os);
  return hipGetLastError();
}

template <int DT, int LAYOUT>
hipError_t launch_d(const ScoreArgs& a, const BandConst& bc, const OffsetSet& os, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_t<DT, LAYOUT, 64>(a, bc, os, s);
    case 128:  // the matrix-core form
      return os.n <= 16 ? launch_mfma<DT, LAYOUT, 1>(a, bc, os, s) : launch_mfma<DT, LAYOUT, 2>(a, bc, os, s);
    case 256: return launch_t<DT, LAYOUT, 256>(a, bc, os, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_score_max(const ScoreArgs& a, const BandConst& bc, const OffsetSet& os, hipStream_t s) {
  if (a.dtype == kDtBf16) {
    return a.layout == kInterleaved ? launch_d<kDtBf16, kInterleaved>(a, bc, os, s)
                                    : launch_d<kDtBf16, kHalfSplit>(a, bc, os, s);
  }
  return a.layout == kInterleaved ? launch_d<kDtF32, kInterleaved>(a, bc, os, s)
                                  : launch_d<kDtF32, kHalfSplit>(a, bc, os, s);
}

}  // namespace tri
