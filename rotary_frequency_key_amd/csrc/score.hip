// Score kernel of libtri for gfx950 (CDNA4, wave64).
//
// Streams every key once: 16 lanes per 128-d row (4 rotary bands per lane), one 16-byte load
// per lane per row. Per band: the rotation phase in 23-bit fixed point plus a binary32
// residual, hardware sine and cosine in revolutions, two-term bf16 dot products with the
// offset-averaged center; the 16 partial sums of a row are added with DPP. Optionally adds a
// 12-bit top-digit histogram of the scores per unit (the first radix digit of the select).
//
// Score: "The future-offset average in TriAttention can be precomputed", sections "The same
// score, read as arrows in the plane" and "The averaging step": per key,
//     Re{ sum_f mu'_f conj(k_f) e^{i omega_f delta} }
//   = sum_f x_f cos(omega_f delta) - y_f sin(omega_f delta),
//     x_f = Re(mu'_f) Re(k_f) + Im(mu'_f) Im(k_f),  y_f = Im(mu'_f) Re(k_f) - Re(mu'_f) Im(k_f).
#include "score_device.h"
#include "stamps.h"

namespace tri {

TRI_STAMPS_BUFFER(g_stamps_score)

namespace {

using dev::kDtBf16;
using dev::kDtF32;
using dev::kHalfSplit;
using dev::kInterleaved;
using dev::order_key;
using namespace sdev;

// 512 threads and 1024 rows per workgroup (one per CU on one layer's 8 x 32768 keys), 2 rows per
// lane group per iteration and the loads of two iterations in flight: a smaller last iteration
// leaves less arithmetic exposed after the last load than 4 rows with one iteration ahead
// (measured 13.5-13.8 against 14.0-14.5 us for the 67 MB of keys with the histogram).
constexpr int kScoreThreads = 512;
constexpr int kRowsPerLoad = 2;  // rows per lane group per iteration

template <int D>
constexpr int score_rows_per_block() { return 1024; }


// ROT: the keys were rotated at their own positions (stored after the rotary embedding). Then
// conj(k_f) e^{i omega_f (t - p)} = conj(k_f e^{i omega_f p}) e^{i omega_f t}, so the score is
// Re{ sum_f (mu'_f e^{i omega_f t}) conj(krot_f) }: one coefficient vector per unit, a plain dot
// product per key, no positions and no per-key trigonometry ("The same score, read as arrows in
// the plane": the rotation is a multiplication, and rotations compose by adding angles).
template <int DT, int LAYOUT, int D, bool HIST, bool ROT>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a, int chunks_per_unit, BandConst bc) {
  constexpr int F = D / 2;
  constexpr int LPR = F / 4;                 // lanes per row, 4 bands each
  constexpr int GPW = 64 / LPR;              // row groups per wave
  constexpr int M = kRowsPerLoad;
  constexpr int ROWS_WAVE = GPW * M;         // rows per wave per iteration
  constexpr int ROWS_ITER = ROWS_WAVE * (kScoreThreads / 64);
  constexpr int RPB = score_rows_per_block<D>();
  constexpr int ITERS = RPB / ROWS_ITER;
  static_assert(RPB % ROWS_ITER == 0, "rows per block");
  using L = RowLoad<DT, LAYOUT, D>;
  using KT = typename L::T;

  __shared__ uint32_t lhist[HIST ? kHistBins : 1];

  TRI_STAMP(g_stamps_score, stamps::kScore, 0);
  const int bid = dev::xcd_block(blockIdx.x, gridDim.x);
  const int unit = bid / chunks_per_unit;
  const int chunk = bid - unit * chunks_per_unit;
  const dev::UnitRows ur = dev::unit_rows(a.row_off, unit, a.total_rows, a.max_rows);
  const int64_t beg = ur.beg, end = ur.beg + ur.n;
  const int64_t r0 = beg + (int64_t)chunk * RPB;
  if (r0 >= end) return;  // uniform across the block
  const int64_t r1 = (end - r0 < RPB) ? end : r0 + RPB;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l = lane % LPR;   // lane within the row group: bands 4l .. 4l+3
  const int gw = lane / LPR;  // row group within the wave

  // Rows are addressed relative to r0 with 32-bit offsets; rows past the end load the last
  // row of the chunk instead (always valid) and are never stored.
  const char* kbase = static_cast<const char*>(a.keys) + r0 * L::kRowBytes;
  const int32_t* pbase = ROT ? nullptr : a.pos + r0;
  const uint32_t last = (uint32_t)(r1 - r0 - 1);
  const uint32_t wave_row = (uint32_t)(wave * ROWS_WAVE + gw);
  KT kb[M], kn[M];
  int32_t pb[M], pn[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t row = min(wave_row + m * GPW, last);
    kb[m] = L::load(kbase, row, l);
    pb[m] = ROT ? 0 : load_pos(pbase, row);
  }
  if (ITERS > 1) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t row = min(wave_row + ROWS_ITER + m * GPW, last);
      kn[m] = L::load(kbase, row, l);
      pn[m] = ROT ? 0 : load_pos(pbase, row);
    }
  }

  if constexpr (HIST) {
    for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) lhist[i] = 0u;
  }

  // per-lane constants
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
  const int32_t t = a.t_now[unit];
  CenterCoef<DT> cc;
  if constexpr (ROT) {
    // mu'_f e^{i omega_f t}
    const uint32_t tl = (uint32_t)t;
    const float tf = (float)tl;
    float rre[4], rim[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float rev = band_phase(tl, tf, step[j], resid[j]);
      const float sn = __builtin_amdgcn_sinf(rev);
      const float cs = __builtin_amdgcn_cosf(rev);
      rre[j] = fmaf(cre[j], cs, -(cim[j] * sn));
      rim[j] = fmaf(cre[j], sn, cim[j] * cs);
    }
    cc.init(rre, rim);
  } else {
    cc.init(cre, cim);
  }

  if constexpr (HIST) __syncthreads();

#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    KT kc[M];
    int32_t pc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) { kc[m] = kb[m]; pc[m] = pb[m]; kb[m] = kn[m]; pb[m] = pn[m]; }
    const uint32_t base = wave_row + (uint32_t)(it * ROWS_ITER);
    if (it + 2 < ITERS) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint32_t row = min(base + 2 * ROWS_ITER + m * GPW, last);
        kn[m] = L::load(kbase, row, l);
        pn[m] = ROT ? 0 : load_pos(pbase, row);
      }
    }
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float s = 0.f;
      if constexpr (ROT) {
#pragma unroll
        for (int j = 0; j < 4; ++j) s += cc.x(kc[m], j);
      } else {
        const uint32_t dl = (uint32_t)(t - pc[m]);
        const float df = (float)dl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float rev = band_phase(dl, df, step[j], resid[j]);
          const float sn = __builtin_amdgcn_sinf(rev);
          const float cs = __builtin_amdgcn_cosf(rev);
          float x, y;
          cc.xy(kc[m], j, x, y);
          s = fmaf(x, cs, s);
          s = fmaf(-y, sn, s);
        }
      }
      acc[m] = group_sum<LPR>(s);
    }
    // lane l < M of each group stores row m = l: the wave's M*GPW rows are contiguous
    if (l < M) {
      float v = acc[0];
#pragma unroll
      for (int m = 1; m < M; ++m) v = (l == m) ? acc[m] : v;
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
    for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) {
      const uint32_t c = lhist[i];
      if (c) atomicAdd(&gh[i], c);
    }
  }
  TRI_STAMP(g_stamps_score, stamps::kScore, 1);
}

// Row order inside an iteration: wave w owns rows [w*ROWS_WAVE, (w+1)*ROWS_WAVE); load m of row
// group gw reads row m*GPW + gw, so one load instruction covers GPW consecutive rows and the
// M*GPW rows a wave stores are consecutive.

template <int DT, int LAYOUT, int D>
hipError_t launch_score_t(const ScoreArgs& a, const BandConst& bc, hipStream_t s) {
  constexpr int RPB = score_rows_per_block<D>();
  const int64_t chunks = (a.max_rows + RPB - 1) / RPB;
  const int64_t grid = chunks * a.n_units;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b(kScoreThreads);
  if (a.rotated) {
    if (a.hist) hipLaunchKernelGGL((score_kernel<DT, LAYOUT, D, true, true>), g, b, 0, s, a, (int)chunks, bc);
    else hipLaunchKernelGGL((score_kernel<DT, LAYOUT, D, false, true>), g, b, 0, s, a, (int)chunks, bc);
  } else {
    if (a.hist) hipLaunchKernelGGL((score_kernel<DT, LAYOUT, D, true, false>), g, b, 0, s, a, (int)chunks, bc);
    else hipLaunchKernelGGL((score_kernel<DT, LAYOUT, D, false, false>), g, b, 0, s, a, (int)chunks, bc);
  }
  return hipGetLastError();
}

template <int DT, int LAYOUT>
hipError_t launch_score_d(const ScoreArgs& a, const BandConst& bc, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_score_t<DT, LAYOUT, 64>(a, bc, s);
    case 128: return launch_score_t<DT, LAYOUT, 128>(a, bc, s);
    case 256: return launch_score_t<DT, LAYOUT, 256>(a, bc, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, const BandConst& bc, hipStream_t s) {
  if (a.dtype == kDtBf16) {
    return a.layout == kInterleaved ? launch_score_d<kDtBf16, kInterleaved>(a, bc, s)
                                    : launch_score_d<kDtBf16, kHalfSplit>(a, bc, s);
  }
  return a.layout == kInterleaved ? launch_score_d<kDtF32, kInterleaved>(a, bc, s)
                                  : launch_score_d<kDtF32, kHalfSplit>(a, bc, s);
}

}  // namespace tri
