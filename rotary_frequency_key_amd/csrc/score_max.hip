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

// ROT: keys stored after the rotary rotation at their positions; conj(k) e^{i w (t - p + delta)}
// = conj(k_rot) e^{i w (t + delta)}, so the same evaluation with every position taken as 0.
template <int DT, int LAYOUT, int D, bool HIST, bool ROT>
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
  const int32_t* pbase = ROT ? nullptr : a.pos + r0;
  const uint32_t last = (uint32_t)(r1 - r0 - 1);
  const uint32_t wave_row = (uint32_t)(wave * ROWS_WAVE + gw);
  KT kb[M];
  int32_t pb[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t row = min(wave_row + m * GPW, last);
    kb[m] = L::load(kbase, row, l);
    pb[m] = ROT ? 0 : load_pos(pbase, row);
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
        pb[m] = ROT ? 0 : load_pos(pbase, row);
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
// Rotations compose by adding angles, so band f's term at offset delta_o factors into a part of
// the key and a part of the unit:
//     E[q_f] conj(k_f) e^{i w_f (Delta + delta_o)} = A_f W_fo,
//     A_f = conj(k_f) e^{i w_f Delta},  W_fo = E[q_f] e^{i w_f delta_o},
// and S(delta_o) = sum_f Re A_f Re W_fo - Im A_f Im W_fo is the product of the key's row
// [Re A, Im A] (128 values) with column o of [Re W; -Im W]. One v_mfma_f32_16x16x32_bf16 takes
// 16 offsets (operand A, W transposed) x 32 values of k x 16 keys (operand B); four steps cover
// k. Each operand is split into bf16 hi + lo (x = hi + lo + O(2^-16 x)) and the product is
// hi*hi + hi*lo + lo*hi, accumulated in fp32.
// Operand B is computed where it is used: lane L holds key L % 16 and, at step s, the k values
// 8 (L / 16) + i. The sum over k does not depend on the order of k, which is chosen so that these
// are the lane's bands 16 h + 4 (L / 16) + j, four contiguous pieces of its key row: value i of
// step s is band n = 8 (s & 1) + i of that list (n = 4 h + j), its real part for s < 2 and its
// imaginary part for s >= 2. W's columns use the same order; the waves of a workgroup build W once
// in LDS and each keeps it in registers. bf16 interleaved keys are loaded contiguously (1 KB per
// instruction) and pass through a per-wave LDS region into that layout; loaded in it directly,
// one instruction would read 64 bytes from each of 16 rows. Offsets past the last repeat it (the maximum does not
// change). The result gives lane L key L % 16 at offsets 16 t + 4 (L / 16) + i of tile t: the
// maximum over those, then over the key's four lanes (two lane swaps), finishes the key.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4m __attribute__((ext_vector_type(4)));

constexpr int kMfmaRowsPerBlock = 512;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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
  constexpr int D = 128, F = 64;
  constexpr int WAVES = kMaxThreads / 64;
  constexpr int ROWS_ITER = 16 * WAVES;  // a wave takes one tile of 16 rows per iteration
  constexpr int RPB = kMfmaRowsPerBlock;
  constexpr int ITERS = RPB / ROWS_ITER;
  static_assert(RPB % ROWS_ITER == 0, "rows per block");
  using L = RowLoad<DT, LAYOUT, D>;
  using KT = typename L::T;

  __shared__ __align__(16) bf16x8 wsh[NT][4][2][64];  // W for each lane: [tile][step][hi, lo][lane]
  // bf16 interleaved keys: tiles loaded contiguously (1 KB per instruction), staged per wave
  constexpr bool STAGE = DT == kDtBf16 && LAYOUT == kInterleaved;
  constexpr uint32_t TSTRIDE = 256 + 16;
  __shared__ __align__(16) char tile[STAGE ? WAVES : 1][STAGE ? 16 * TSTRIDE : 16];
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
  const int mc = lane & 15;  // key row of the wave's tile; offset of an offset tile
  const int mq = lane >> 4;  // bands 16 h + 4 mq + j (h, j < 4): element n = 4 h + j of this lane
  const int n_off = os.n;

  const char* kbase = static_cast<const char*>(a.keys) + r0 * L::kRowBytes;
  const int32_t* pbase = a.pos + r0;
  const uint32_t last = (uint32_t)(r1 - r0 - 1);
  const uint32_t wave_row = (uint32_t)(wave * 16 + mc);
  KT kb[4];
  u32x4 kr[4];  // STAGE: the lane's 16 bytes at g * 1024 + 16 lane of the wave's 16 rows
  int32_t pb;
  auto load_next = [&](int j) {
    const uint32_t row = min(wave_row + (uint32_t)(j * ROWS_ITER), last);
    if constexpr (STAGE) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t byte = (uint32_t)(g * 1024 + 16 * lane);
        const uint32_t r = min((uint32_t)(j * ROWS_ITER + wave * 16) + byte / 256u, last);
        kr[g] = ld_stream<u32x4>(kbase, r * 256u + byte % 256u);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h) kb[h] = L::load(kbase, row, 4 * h + mq);
    }
    pb = load_pos(pbase, row);
  };
  load_next(0);

  if constexpr (HIST) {
    for (int i = threadIdx.x; i < kHistBins; i += kMaxThreads) lhist[i] = 0u;
  }
  uint32_t step[16];
  float resid[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    const int b = 16 * (n >> 2) + 4 * mq + (n & 3);
    step[n] = bc.step[b] & 0x7FFFFFu;
    resid[n] = bc.resid[b];
  }
  const int32_t t = a.t_now[unit];

  // W = E[q_f] e^{i w_f delta_o}, operand A of the product: lane L holds offset o = 16 tt + mc
  // (the last offset past n_off) and, at step s, k = 8 mq + i: band n = 8 (s & 1) + i of this
  // lane, real part for s < 2, minus the imaginary part for s >= 2. Wave w builds tile w / 2,
  // bands n = 8 (w & 1) + i (steps w & 1 and 2 + (w & 1)) for every lane, in LDS.
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {  // unrolled so that the band index is a constant
    if (wave >= 2 * NT || (wave & 1) != hh) continue;
    const int tt = wave >> 1;
    const int o = min(16 * tt + mc, n_off - 1);
    const uint32_t dlo = os.delta[o];
    const float dfo = (float)dlo;
    float mre[8], mim[8];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float4* mp = reinterpret_cast<const float4*>(a.mu + ((size_t)unit * F + 16 * (2 * hh + g) + 4 * mq) * 2);
      const float4 m0 = mp[0], m1 = mp[1];
      mre[4 * g + 0] = m0.x; mim[4 * g + 0] = m0.y; mre[4 * g + 1] = m0.z; mim[4 * g + 1] = m0.w;
      mre[4 * g + 2] = m1.x; mim[4 * g + 2] = m1.y; mre[4 * g + 3] = m1.z; mim[4 * g + 3] = m1.w;
    }
    bf16x8 rh, rl, ih, il;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = 8 * hh + i;
      const float rev = band_phase(dlo, dfo, step[n], resid[n]);
      const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
      const float wr = fmaf(mre[i], cs, -(mim[i] * sn));
      const float wi = fmaf(mre[i], sn, mim[i] * cs);
      __bf16 h, lo;
      split_bf16(wr, h, lo);
      rh[i] = h;
      rl[i] = lo;
      split_bf16(-wi, h, lo);
      ih[i] = h;
      il[i] = lo;
    }
    wsh[tt][hh][0][lane] = rh;
    wsh[tt][hh][1][lane] = rl;
    wsh[tt][2 + hh][0][lane] = ih;
    wsh[tt][2 + hh][1][lane] = il;
  }
  __syncthreads();

  bf16x8 whi[NT][4], wlo[NT][4];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      whi[tt][st] = wsh[tt][st][0][lane];
      wlo[tt][st] = wsh[tt][st][1][lane];
    }

  // a row's score is stored one iteration late, halfway through the next tile, after the wait for
  // that tile's loads: the memory counter takes loads and stores in issue order, so a wait for a
  // load never has to wait for a store issued just before it
  float v_prev = 0.f;
  bool mine_prev = false;
  uint32_t row_prev = 0;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    KT kc[4];
    if constexpr (STAGE) {
      char* tw = tile[wave];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t byte = (uint32_t)(g * 1024 + 16 * lane);
        *reinterpret_cast<u32x4*>(tw + (byte / 256u) * TSTRIDE + byte % 256u) = kr[g];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(tw + mc * TSTRIDE + (4 * h + mq) * 16);
        kc[h] = KT{{v.x, v.y, v.z, v.w}};
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h) kc[h] = kb[h];
    }
    const int32_t pc = pb;
    if (it + 1 < ITERS) load_next(it + 1);
    __builtin_amdgcn_sched_barrier(0);  // the next tile's loads stay in flight during this one
    // operand B: conj(k_f) e^{i w_f Delta} of row mc, k laid out as in W
    const uint32_t dl = (uint32_t)(t - pc);
    const float df = (float)dl;
    f32x4m acc[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = f32x4m{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float ar[8], ai[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int n = 8 * hh + i;
        const float rev = band_phase(dl, df, step[n], resid[n]);
        const float sn = __builtin_amdgcn_sinf(rev);
        const float cs = __builtin_amdgcn_cosf(rev);
        float x, y;
        if constexpr (DT == kDtBf16) {
          const uint32_t w = kc[n >> 2].b[n & 3];
          x = __uint_as_float(w << 16);
          y = __uint_as_float(w & 0xFFFF0000u);
        } else {
          x = kc[n >> 2].re[n & 3];
          y = kc[n >> 2].im[n & 3];
        }
        ar[i] = fmaf(x, cs, y * sn);
        ai[i] = fmaf(x, sn, -(y * cs));
      }
      bf16x8 rhi, rlo, ihi, ilo;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        bf16x2 h2, l2;
        split_bf16x2(ar[i], ar[i + 1], h2, l2);
        rhi[i] = h2[0]; rhi[i + 1] = h2[1]; rlo[i] = l2[0]; rlo[i + 1] = l2[1];
        split_bf16x2(ai[i], ai[i + 1], h2, l2);
        ihi[i] = h2[0]; ihi[i + 1] = h2[1]; ilo[i] = l2[0]; ilo[i + 1] = l2[1];
      }
      if (hh == 1 && mine_prev) a.scores[r0 + row_prev] = v_prev;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(whi[tt][hh], rhi, acc[tt], 0, 0, 0);
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wlo[tt][hh], rhi, acc[tt], 0, 0, 0);
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(whi[tt][hh], rlo, acc[tt], 0, 0, 0);
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(whi[tt][2 + hh], ihi, acc[tt], 0, 0, 0);
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wlo[tt][2 + hh], ihi, acc[tt], 0, 0, 0);
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(whi[tt][2 + hh], ilo, acc[tt], 0, 0, 0);
      }
    }
    // lane L: row mc at offsets 16 tt + 4 mq + i; maximum over those, then over the four k blocks
    float v = acc[0][0];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) v = fmaxf(v, acc[tt][i]);
    {  // lanes L, L ^ 16, L ^ 32, L ^ 48 hold the same row: swap 16-lane rows, then halves
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      v = fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
    }
    const uint32_t row = (uint32_t)(it * ROWS_ITER) + wave_row;
    const bool mine = mq == 0 && row <= last;
    if constexpr (HIST) {
      if (mine) atomicAdd(&lhist[order_key(v) >> kHistShift], 1u);
    }
    v_prev = v;
    mine_prev = mine;
    row_prev = row;
  }
  if (mine_prev) a.scores[r0 + row_prev] = v_prev;

  if constexpr (HIST) {
    __syncthreads();
    uint32_t* gh = a.hist + (size_t)unit * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kMaxThreads) {
      const uint32_t c = lhist[i];
      if (c) atomicAdd(&gh[i], c);
    }
  }
}

// Keys stored after the rotary rotation (k_rot = k e^{i w p}; "The same score, read as arrows in
// the plane": rotations compose by adding angles): conj(k_f) e^{i w_f (t - p + delta)} =
// conj(k_rot_f) e^{i w_f (t + delta)}. With P_fo = E[q_f] e^{i w_f (t + delta_o)}, one value per
// unit, band and offset, and k_rot_f = x_f + i y_f,
//     S(delta_o) = sum_f Re(P_fo) x_f + Im(P_fo) y_f,
// the product of the key row itself (128 values in memory order) with W[e][o] = Re or Im of
// P_{f(e), o}, e the element of the row and f(e) its band. There is no per-key trigonometry: bf16
// keys are exact bf16 operands (W split into hi + lo: two products per step), fp32 keys are split
// like W (three). Lane L holds key L % 16 and, at step s, elements 32 s + 8 (L / 16) + i of it:
// one 16-byte piece of the row for bf16, two for fp32. Loaded in that layout, one instruction would
// read 64 bytes from each of 16 rows; the tiles are loaded contiguously instead (1 KB per
// instruction) and pass through a per-wave LDS region into the operand layout. W, the result and
// the stores are as in score_max_mfma_kernel.
template <int DT, int LAYOUT, bool HIST, int NT>  // NT: tiles of 16 offsets
__global__ __launch_bounds__(kMaxThreads) void score_max_rot_mfma_kernel(ScoreArgs a, int chunks_per_unit,
                                                                         BandConst bc, OffsetSet os) {
  constexpr int D = 128, F = 64;
  constexpr int WAVES = kMaxThreads / 64;
  constexpr int ROWS_ITER = 16 * WAVES;
  constexpr int RPB = kMfmaRowsPerBlock;
  constexpr int ITERS = RPB / ROWS_ITER;
  static_assert(RPB % ROWS_ITER == 0, "rows per block");
  constexpr int EB = DT == kDtBf16 ? 2 : 4;  // bytes per element
  constexpr uint32_t ROW_BYTES = D * EB;
  constexpr int PIECES = 8 * EB / 16;        // 16-byte pieces per 8 elements
  constexpr int PF = 3;                      // tiles of loads in flight ahead of the one in use
  static_assert(ITERS > PF, "tiles per wave");

  __shared__ __align__(16) bf16x8 wsh[NT][4][2][64];  // W for each lane: [tile][step][hi, lo][lane]
  constexpr uint32_t TSTRIDE = ROW_BYTES + 16;  // LDS bytes per staged row (16 of padding)
  __shared__ __align__(16) char tile[WAVES][16 * TSTRIDE];  // each wave's 16 rows, staged
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
  const int mc = lane & 15;  // key row of the wave's tile; offset of an offset tile
  const int mq = lane >> 4;  // elements 32 s + 8 mq + i of the row at step s
  const int n_off = os.n;

  const char* kbase = static_cast<const char*>(a.keys) + r0 * (int64_t)ROW_BYTES;
  const uint32_t last = (uint32_t)(r1 - r0 - 1);
  const uint32_t wave_row = (uint32_t)(wave * 16 + mc);
  // a ring of PF + 1 tiles in registers (the loop is unrolled): tile it in use, it + 1 .. it + PF
  // in flight; with one tile ahead a CU keeps too few bytes in flight to cover the memory latency
  // loads are contiguous: instruction g of a tile covers 1 KB, lane L the 16 bytes at
  // g * 1024 + 16 L of the wave's 16 rows; the tile then goes through LDS into the operand layout
  constexpr int LPT = 16 * ROW_BYTES / 1024;  // load instructions per tile
  u32x4 kq[PF + 1][LPT];
  auto load_tile = [&](int j, int slot) {
#pragma unroll
    for (int g = 0; g < LPT; ++g) {
      const uint32_t byte = (uint32_t)(g * 1024 + 16 * lane);
      const uint32_t row = min((uint32_t)(j * ROWS_ITER + wave * 16) + byte / ROW_BYTES, last);
      kq[slot][g] = ld_stream<u32x4>(kbase, row * ROW_BYTES + byte % ROW_BYTES);
    }
  };
#pragma unroll
  for (int j = 0; j < PF; ++j) load_tile(j, j);
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < kHistBins; i += kMaxThreads) lhist[i] = 0u;
  }

  // W, operand A: lane L holds offset o = 16 tt + mc (the last offset past n_off) and, at step s,
  // W[32 s + 8 mq + i][o]. Wave w builds tile w / 2, steps 2 (w & 1) and 2 (w & 1) + 1, in LDS.
  const uint32_t t = (uint32_t)a.t_now[unit];
  if (wave < 2 * NT) {
    const int tt = wave >> 1;
    const int o = min(16 * tt + mc, n_off - 1);
    const uint32_t dlo = os.delta[o];
    const float2* mu2 = reinterpret_cast<const float2*>(a.mu) + (size_t)unit * F;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int st = 2 * (wave & 1) + s2;
      bf16x8 h8, l8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = 32 * st + 8 * mq + i;
        const int f = LAYOUT == kInterleaved ? e >> 1 : e & 63;
        const bool im = LAYOUT == kInterleaved ? (e & 1) != 0 : e >= 64;
        const uint32_t step = bc.step[f] & 0x7FFFFFu;
        const float resid = bc.resid[f];
        const float rt = band_phase(t, (float)t, step, resid);
        const float rd = band_phase(dlo, (float)dlo, step, resid);
        const float ct = __builtin_amdgcn_cosf(rt), snt = __builtin_amdgcn_sinf(rt);
        const float cd = __builtin_amdgcn_cosf(rd), snd = __builtin_amdgcn_sinf(rd);
        const float er = fmaf(ct, cd, -(snt * snd)), ei = fmaf(ct, snd, snt * cd);  // e^{i w (t + delta)}
        const float2 m = mu2[f];
        const float w = im ? fmaf(m.x, ei, m.y * er) : fmaf(m.x, er, -(m.y * ei));
        __bf16 h, lo;
        split_bf16(w, h, lo);
        h8[i] = h;
        l8[i] = lo;
      }
      wsh[tt][st][0][lane] = h8;
      wsh[tt][st][1][lane] = l8;
    }
  }
  __syncthreads();

  bf16x8 whi[NT][4], wlo[NT][4];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      whi[tt][st] = wsh[tt][st][0][lane];
      wlo[tt][st] = wsh[tt][st][1][lane];
    }

  // scores stored one iteration late, halfway through the next tile (as in score_max_mfma_kernel)
  float v_prev = 0.f;
  bool mine_prev = false;
  uint32_t row_prev = 0;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    if (it + PF < ITERS) load_tile(it + PF, (it + PF) % (PF + 1));
    // stage the tile, then read it in the operand layout (the wave's own region: its LDS
    // operations run in order; the fences keep the compiler's order too)
    char* tw = tile[wave];
#pragma unroll
    for (int g = 0; g < LPT; ++g) {
      const uint32_t byte = (uint32_t)(g * 1024 + 16 * lane);
      *reinterpret_cast<u32x4*>(tw + (byte / ROW_BYTES) * TSTRIDE + byte % ROW_BYTES) = kq[it % (PF + 1)][g];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    u32x4 kc[4][PIECES];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int q = 0; q < PIECES; ++q)
        kc[st][q] = *reinterpret_cast<const u32x4*>(tw + mc * TSTRIDE + (32 * st + 8 * mq) * EB + 16 * q);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_sched_barrier(0);  // the next tile's loads stay in flight during this one
    f32x4m acc[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = f32x4m{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (st == 2 && mine_prev) a.scores[r0 + row_prev] = v_prev;
      if constexpr (DT == kDtBf16) {
        const bf16x8 kv = __builtin_bit_cast(bf16x8, kc[st][0]);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(whi[tt][st], kv, acc[tt], 0, 0, 0);
          acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wlo[tt][st], kv, acc[tt], 0, 0, 0);
        }
      } else {
        bf16x8 khi, klo;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            bf16x2 h2, l2;
            split_bf16x2(__uint_as_float(kc[st][q][j]), __uint_as_float(kc[st][q][j + 1]), h2, l2);
            khi[4 * q + j] = h2[0]; khi[4 * q + j + 1] = h2[1];
            klo[4 * q + j] = l2[0]; klo[4 * q + j + 1] = l2[1];
          }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(whi[tt][st], khi, acc[tt], 0, 0, 0);
          acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wlo[tt][st], khi, acc[tt], 0, 0, 0);
          acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(whi[tt][st], klo, acc[tt], 0, 0, 0);
        }
      }
    }
    // lane L: row mc at offsets 16 tt + 4 mq + i; maximum over those, then over the four k blocks
    float v = acc[0][0];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) v = fmaxf(v, acc[tt][i]);
    {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      v = fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
    }
    const uint32_t row = (uint32_t)(it * ROWS_ITER) + wave_row;
    const bool mine = mq == 0 && row <= last;
    if constexpr (HIST) {
      if (mine) atomicAdd(&lhist[order_key(v) >> kHistShift], 1u);
    }
    v_prev = v;
    mine_prev = mine;
    row_prev = row;
  }
  if (mine_prev) a.scores[r0 + row_prev] = v_prev;

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
  if (a.rotated) {
    if (a.hist)
      hipLaunchKernelGGL((score_max_rot_mfma_kernel<DT, LAYOUT, true, NT>), g, b, 0, s, a, (int)chunks, bc, os);
    else
      hipLaunchKernelGGL((score_max_rot_mfma_kernel<DT, LAYOUT, false, NT>), g, b, 0, s, a, (int)chunks, bc, os);
  } else if (a.hist) {
    hipLaunchKernelGGL((score_max_mfma_kernel<DT, LAYOUT, true, NT>), g, b, 0, s, a, (int)chunks, bc, os);
  } else {
    hipLaunchKernelGGL((score_max_mfma_kernel<DT, LAYOUT, false, NT>), g, b, 0, s, a, (int)chunks, bc, os);
  }
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
  if (a.rotated) {
    if (a.hist) hipLaunchKernelGGL((score_max_kernel<DT, LAYOUT, D, true, true>), g, b, 0, s, a, (int)chunks, bc, os);
    else hipLaunchKernelGGL((score_max_kernel<DT, LAYOUT, D, false, true>), g, b, 0, s, a, (int)chunks, bc, os);
  } else if (a.hist) {
    hipLaunchKernelGGL((score_max_kernel<DT, LAYOUT, D, true, false>), g, b, 0, s, a, (int)chunks, bc, os);
  } else {
    hipLaunchKernelGGL((score_max_kernel<DT, LAYOUT, D, false, false>), g, b, 0, s, a, (int)chunks, bc, os);
  }
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
