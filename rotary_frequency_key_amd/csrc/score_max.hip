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
// a row add each offset's terms with DPP and keep the running maximum; with 16 lanes per row
// (d = 128) whole groups of 16 offsets are reduced together (a reduce-scatter across the lanes).
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
    int o0 = 0;
    if constexpr (LPR == 16) {
      // whole groups of 16 offsets: lane l's slot k holds offset 16c + ((k + l) mod 16), so that
      // four row_ror steps (8, 4, 2, 1) leave in each lane the row sum of one offset, 15 DPP adds
      // for 16 offsets instead of 64; the maximum over the lanes is taken once at the end.
      for (; o0 + 16 <= n_off; o0 += 16) {
        float acc[M][16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int o = o0 + ((k + l) & 15);
          const float4 w01 = *reinterpret_cast<const float4*>(&tab[o][4 * l]);
          const float4 w23 = *reinterpret_cast<const float4*>(&tab[o][4 * l + 2]);
#pragma unroll
          for (int m = 0; m < M; ++m) acc[m][k] = band_terms(P[m], Q[m], w01, w23);
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[m][k] += dpp_f<0x128>(acc[m][k + 8]);  // row_ror:8
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[m][k] += dpp_f<0x124>(acc[m][k + 4]);  // row_ror:4
#pragma unroll
          for (int k = 0; k < 2; ++k) acc[m][k] += dpp_f<0x122>(acc[m][k + 2]);  // row_ror:2
          acc[m][0] += dpp_f<0x121>(acc[m][1]);                                  // row_ror:1
          best[m] = fmaxf(best[m], acc[m][0]);
        }
      }
    }
    for (int o = o0; o < n_off; ++o) {  // the rest one at a time, every lane gets the row sum
      const float4 w01 = *reinterpret_cast<const float4*>(&tab[o][4 * l]);
      const float4 w23 = *reinterpret_cast<const float4*>(&tab[o][4 * l + 2]);
#pragma unroll
      for (int m = 0; m < M; ++m) best[m] = fmaxf(best[m], group_sum<LPR>(band_terms(P[m], Q[m], w01, w23)));
    }
    if constexpr (LPR == 16) {
#pragma unroll
      for (int m = 0; m < M; ++m) best[m] = group_max16(best[m]);
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
    case 128: return launch_t<DT, LAYOUT, 128>(a, bc, os, s);
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
