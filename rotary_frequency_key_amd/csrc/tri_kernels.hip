// Device kernels of libtri for gfx950 (CDNA4, wave64) and their launchers.
//
//  score_kernel    streams the keys once, 16 lanes per 128-d row, one 16-byte load per lane
//                  per row; per band: fixed-point rotation phase, hardware sine/cosine in
//                  revolutions, two-term bf16 dot products with mu'; DPP row reduction.
//                  Optionally folds a 12-bit top-digit histogram of the scores per unit.
//  select_kernel   one workgroup per unit: radix select of the B-th largest order key
//                  (12 + 10 + 10 bits), then one ordered pass that emits kept row indices
//                  ascending with the lower-index tie rule.
//  compact_kernel  gathers the kept K/V rows (16-byte loads/stores) and positions.
//
// Score definition: "The future-offset average in TriAttention can be precomputed", sections
// "The same score, read as arrows in the plane" and "The averaging step": per key,
//     Re{ sum_f mu'_f conj(k_f) e^{i omega_f delta} }
//   = sum_f x_f cos(omega_f delta) - y_f sin(omega_f delta),
//     x_f = Re(mu'_f) Re(k_f) + Im(mu'_f) Im(k_f),  y_f = Im(mu'_f) Re(k_f) - Re(mu'_f) Im(k_f).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tri_internal.h"

namespace tri {
namespace {

constexpr int kDtF32 = 0;
constexpr int kDtBf16 = 1;
constexpr int kInterleaved = 0;
constexpr int kHalfSplit = 1;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t pack_bf16(uint32_t lo, uint32_t hi) {
  return (lo & 0xFFFFu) | (hi << 16);
}

// lo(k)*lo(c) + hi(k)*hi(c) + acc, bf16 pairs, binary32 accumulate (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2(uint32_t k, uint32_t c, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k),
                                         __builtin_bit_cast(bf16x2_t, c), acc, false);
}

// lo(k)*lo(c) + hi(k)*hi(c) from a zero accumulator (VOP3P form, inline constant 0)
__device__ __forceinline__ float dot2_z(uint32_t k, uint32_t c) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(k), "v"(c));
  return r;
}

// low 32 bits of a * b for a, b < 2^24 (full-rate 24-bit multiply)
__device__ __forceinline__ uint32_t mul_u24(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_mul_u32_u24 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Total order on binary32 scores as unsigned integers: larger score -> larger key;
// -0.0 and +0.0 map to one key; every NaN maps to 0, below -inf (0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t b = __float_as_uint(s);
  const uint32_t mag = b & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return 0u;
  if (mag == 0u) return 0x80000000u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LPR lanes (LPR = 8, 16 or 32); every lane gets its group's sum.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_f<0x141>(v);  // row_half_mirror: pairs quads 0<->1, 2<->3 within 8 lanes
  if constexpr (LPR >= 16) v += dpp_f<0x140>(v);  // row_mirror: the two halves of a 16-row
  if constexpr (LPR >= 32) {
    // swap 16-lane rows within each 32-lane half (ds_swizzle bit mode, xor 0x10)
    v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  }
  return v;
}

// ---------------------------------------------------------------------------------------------
// score
// ---------------------------------------------------------------------------------------------

// Loads this lane's 4 bands of one row and returns, per band, the pair (Re k, Im k).
// bf16: one dword per band holding (re, im) as a bf16 pair (re in the low half).
// f32: two floats per band.
template <int DT, int LAYOUT, int D>
struct RowLoad;

template <int D>
struct RowLoad<kDtBf16, kInterleaved, D> {
  struct T { uint32_t b[4]; };
  static constexpr int kRowBytes = D * 2;
  static __device__ __forceinline__ T load(const char* base, uint32_t row, int l) {
    const uint4 v = *reinterpret_cast<const uint4*>(base + row * kRowBytes + l * 16);
    return T{{v.x, v.y, v.z, v.w}};
  }
  static __device__ __forceinline__ T zero() { return T{{0u, 0u, 0u, 0u}}; }
};

template <int D>
struct RowLoad<kDtBf16, kHalfSplit, D> {
  struct T { uint32_t b[4]; };
  static constexpr int kRowBytes = D * 2;
  static __device__ __forceinline__ T load(const char* base, uint32_t row, int l) {
    const char* r = base + row * kRowBytes;
    const uint2 re = *reinterpret_cast<const uint2*>(r + l * 8);
    const uint2 im = *reinterpret_cast<const uint2*>(r + D + l * 8);
    return T{{(re.x & 0xFFFFu) | (im.x << 16), (re.x >> 16) | (im.x & 0xFFFF0000u),
              (re.y & 0xFFFFu) | (im.y << 16), (re.y >> 16) | (im.y & 0xFFFF0000u)}};
  }
  static __device__ __forceinline__ T zero() { return T{{0u, 0u, 0u, 0u}}; }
};

template <int D>
struct RowLoad<kDtF32, kInterleaved, D> {
  struct T { float re[4], im[4]; };
  static constexpr int kRowBytes = D * 4;
  static __device__ __forceinline__ T load(const char* base, uint32_t row, int l) {
    const float4* r = reinterpret_cast<const float4*>(base + row * kRowBytes + l * 32);
    const float4 a = r[0], b = r[1];
    return T{{a.x, a.z, b.x, b.z}, {a.y, a.w, b.y, b.w}};
  }
  static __device__ __forceinline__ T zero() { return T{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}; }
};

template <int D>
struct RowLoad<kDtF32, kHalfSplit, D> {
  struct T { float re[4], im[4]; };
  static constexpr int kRowBytes = D * 4;
  static __device__ __forceinline__ T load(const char* base, uint32_t row, int l) {
    const char* r = base + row * kRowBytes;
    const float4 a = *reinterpret_cast<const float4*>(r + l * 16);
    const float4 b = *reinterpret_cast<const float4*>(r + D * 2 + l * 16);
    return T{{a.x, a.y, a.z, a.w}, {b.x, b.y, b.z, b.w}};
  }
  static __device__ __forceinline__ T zero() { return T{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}; }
};

// The unit's offset-averaged center for this lane's 4 bands, in the form the band product uses.
template <int DT>
struct CenterCoef;

template <>
struct CenterCoef<kDtBf16> {
  // x = dot2(k, (a, b)), y = dot2(k, (b, -a)), each with a two-term bf16 split hi + lo of (a, b)
  uint32_t xh[4], xl[4], yh[4], yl[4];
  __device__ __forceinline__ void init(const float* re, const float* im) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t ah = bf16_rne(re[j]), bh = bf16_rne(im[j]);
      const uint32_t al = bf16_rne(re[j] - bf16_to_f32(ah)), bl = bf16_rne(im[j] - bf16_to_f32(bh));
      xh[j] = pack_bf16(ah, bh);
      xl[j] = pack_bf16(al, bl);
      yh[j] = pack_bf16(bh, ah ^ 0x8000u);
      yl[j] = pack_bf16(bl, al ^ 0x8000u);
    }
  }
  template <class T>
  __device__ __forceinline__ void xy(const T& k, int j, float& x, float& y) const {
    x = dot2(k.b[j], xh[j], dot2_z(k.b[j], xl[j]));
    y = dot2(k.b[j], yh[j], dot2_z(k.b[j], yl[j]));
  }
};

template <>
struct CenterCoef<kDtF32> {
  float a[4], b[4];
  __device__ __forceinline__ void init(const float* re, const float* im) {
#pragma unroll
    for (int j = 0; j < 4; ++j) { a[j] = re[j]; b[j] = im[j]; }
  }
  template <class T>
  __device__ __forceinline__ void xy(const T& k, int j, float& x, float& y) const {
    x = fmaf(a[j], k.re[j], b[j] * k.im[j]);
    y = fmaf(b[j], k.re[j], -(a[j] * k.im[j]));
  }
};

constexpr int kScoreThreads = 256;
constexpr int kRowsPerLoad = 4;  // rows per lane group in flight per iteration

template <int D>
constexpr int score_rows_per_block() { return 512; }

template <int DT, int LAYOUT, int D, bool HIST>
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

  const int unit = blockIdx.x / chunks_per_unit;
  const int chunk = blockIdx.x - unit * chunks_per_unit;
  int64_t beg = a.row_off[unit], end = a.row_off[unit + 1];
  beg = beg < 0 ? 0 : (beg > a.total_rows ? a.total_rows : beg);
  end = end < beg ? beg : (end > a.total_rows ? a.total_rows : end);
  if (end - beg > a.max_rows) end = beg + a.max_rows;
  const int64_t r0 = beg + (int64_t)chunk * RPB;
  if (r0 >= end) return;  // uniform across the block
  const int64_t r1 = (end - r0 < RPB) ? end : r0 + RPB;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l = lane % LPR;   // lane within the row group: bands 4l .. 4l+3
  const int gw = lane / LPR;  // row group within the wave

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
  CenterCoef<DT> cc;
  cc.init(cre, cim);
  const int32_t t = a.t_now[unit];

  if constexpr (HIST) __syncthreads();

  // Rows are addressed relative to r0 with 32-bit offsets; rows past the end load the last
  // row of the chunk instead (always valid) and are never stored.
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
    pb[m] = pbase[row];
  }

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
        pb[m] = pbase[row];
      }
    }
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t dl = (uint32_t)(t - pc[m]);
      const float df = (float)dl;
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t prod = mul_u24(dl, step[j]);
        const float one_frac = __uint_as_float((prod & 0x7FFFFFu) | 0x3F800000u);
        const float rev = fmaf(df, resid[j], one_frac);  // revolutions (+1, harmless)
        const float sn = __builtin_amdgcn_sinf(rev);
        const float cs = __builtin_amdgcn_cosf(rev);
        float x, y;
        cc.xy(kc[m], j, x, y);
        s = fmaf(x, cs, s);
        s = fmaf(-y, sn, s);
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
  if (a.hist)
    hipLaunchKernelGGL((score_kernel<DT, LAYOUT, D, true>), dim3((unsigned)grid), dim3(kScoreThreads), 0, s,
                       a, (int)chunks, bc);
  else
    hipLaunchKernelGGL((score_kernel<DT, LAYOUT, D, false>), dim3((unsigned)grid), dim3(kScoreThreads), 0, s,
                       a, (int)chunks, bc);
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

// ---------------------------------------------------------------------------------------------
// select
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum over the block; *total receives the block sum. sh: >= NT/64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sh[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    uint32_t w = lane < NW ? sh[lane] : 0u;
    w = wave_incl_scan(w);
    if (lane < NW) sh[lane] = w;
  }
  __syncthreads();
  const uint32_t base = wid ? sh[wid - 1] : 0u;
  *total = sh[NW - 1];
  __syncthreads();
  return base + inc - v;
}

// In h[0..nb): find bin b with above(b) < rank <= above(b) + h[b], above(b) = sum of bins > b.
// Requires sum(h) >= rank >= 1. Returns b; *above_out = above(b).
template <int NT>
__device__ uint32_t find_bin(const uint32_t* h, int nb, uint32_t rank, uint32_t* sh, uint32_t* found,
                             uint32_t* above_out) {
  const int per = nb / NT;  // nb is a multiple of NT
  const int top = nb - 1 - (int)threadIdx.x * per;
  uint32_t loc = 0;
  for (int q = 0; q < per; ++q) loc += h[top - q];
  uint32_t tot;
  uint32_t c = block_excl_scan<NT>(loc, sh, &tot);
  for (int q = 0; q < per; ++q) {
    const uint32_t hb = h[top - q];
    if (c < rank && rank <= c + hb) { found[0] = (uint32_t)(top - q); found[1] = c; }
    c += hb;
  }
  __syncthreads();
  const uint32_t b = found[0];
  *above_out = found[1];
  __syncthreads();
  return b;
}

constexpr int kSelectThreads = 1024;

__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectArgs a) {
  constexpr int NT = kSelectThreads;
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t sh[NT / 64];
  __shared__ uint32_t found[2];

  const int u = blockIdx.x;
  if (threadIdx.x == 0) { found[0] = 0u; found[1] = 0u; }
  int64_t beg = a.row_off[u], end = a.row_off[u + 1];
  beg = beg < 0 ? 0 : (beg > a.total_rows ? a.total_rows : beg);
  end = end < beg ? beg : (end > a.total_rows ? a.total_rows : end);
  if (end - beg > a.max_rows) end = beg + a.max_rows;
  const int n = (int)(end - beg);
  const int m = a.B < n ? a.B : n;
  int32_t* out = a.kept_idx + (int64_t)u * a.B;
  uint32_t* gh = a.hist ? a.hist + (size_t)u * kHistBins : nullptr;
  const float* s = a.scores + beg;

  if (m == n || m == 0) {  // keep every row, or none
    for (int j = threadIdx.x; j < a.B; j += NT) out[j] = j < m ? j : -1;
    if (threadIdx.x == 0) a.kept_cnt[u] = m;
    if (a.hist_ready)
      for (int i = threadIdx.x; i < kHistBins; i += NT) gh[i] = 0u;
    return;
  }

  // digit 1: bits 31..20
  if (a.hist_ready) {
    for (int i = threadIdx.x; i < kHistBins; i += NT) { h[i] = gh[i]; gh[i] = 0u; }
  } else {
    for (int i = threadIdx.x; i < kHistBins; i += NT) h[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) atomicAdd(&h[order_key(s[i]) >> 20], 1u);
  }
  __syncthreads();
  uint32_t rank = (uint32_t)m, above;
  const uint32_t b0 = find_bin<NT>(h, kHistBins, rank, sh, found, &above);
  rank -= above;

  // digit 2: bits 19..10 of keys whose digit 1 is b0
  for (int i = threadIdx.x; i < 1024; i += NT) h[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t k = order_key(s[i]);
    if ((k >> 20) == b0) atomicAdd(&h[(k >> 10) & 1023u], 1u);
  }
  __syncthreads();
  const uint32_t b1 = find_bin<NT>(h, 1024, rank, sh, found, &above);
  rank -= above;
  const uint32_t pre = (b0 << 10) | b1;  // bits 31..10

  // digit 3: bits 9..0 of keys whose bits 31..10 are pre
  for (int i = threadIdx.x; i < 1024; i += NT) h[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t k = order_key(s[i]);
    if ((k >> 10) == pre) atomicAdd(&h[k & 1023u], 1u);
  }
  __syncthreads();
  const uint32_t b2 = find_bin<NT>(h, 1024, rank, sh, found, &above);
  rank -= above;
  const uint32_t T = (pre << 10) | b2;  // order key of the B-th largest score
  const uint32_t need = rank;           // keys equal to T that are kept (the lowest indices)

  // ordered emission: slot of a kept key = (# greater keys before it) + (# kept ties before it)
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < n; base += NT) {
    const int i = base + threadIdx.x;
    const uint32_t k = i < n ? order_key(s[i]) : 0u;
    const uint32_t gt = (i < n && k > T) ? 1u : 0u;
    const uint32_t eq = (i < n && k == T) ? 1u : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan<NT>((gt << 16) | eq, sh, &tot);
    const uint32_t G = run_gt + (ex >> 16), E = run_eq + (ex & 0xFFFFu);
    // slots stay below m by construction; the bound also holds for a stale histogram
    const uint32_t slot = G + (E < need ? E : need);
    if ((gt || (eq && E < need)) && slot < (uint32_t)m) out[slot] = i;
    run_gt += tot >> 16;
    run_eq += tot & 0xFFFFu;
  }
  for (int j = m + threadIdx.x; j < a.B; j += NT) out[j] = -1;
  if (threadIdx.x == 0) a.kept_cnt[u] = m;
}

// ---------------------------------------------------------------------------------------------
// compact
// ---------------------------------------------------------------------------------------------

constexpr int kCompactThreads = 256;
constexpr int kCompactRows = 64;  // kept rows per block

template <int CPR>  // 16-byte chunks per row
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(CompactArgs a, int blocks_per_unit) {
  const int u = blockIdx.x / blocks_per_unit;
  const int b = blockIdx.x - u * blocks_per_unit;
  int64_t beg = a.row_off[u], end = a.row_off[u + 1];
  beg = beg < 0 ? 0 : (beg > a.total_rows ? a.total_rows : beg);
  end = end < beg ? beg : (end > a.total_rows ? a.total_rows : end);
  const int64_t n = end - beg;
  int cnt = a.kept_cnt[u];
  cnt = cnt < 0 ? 0 : (cnt > a.B ? a.B : cnt);
  const int j0 = b * kCompactRows;
  const uint4* K = static_cast<const uint4*>(a.K);
  const uint4* V = static_cast<const uint4*>(a.V);
  uint4* Ko = static_cast<uint4*>(a.K_out);
  uint4* Vo = static_cast<uint4*>(a.V_out);
  for (int q = threadIdx.x; q < kCompactRows * CPR; q += kCompactThreads) {
    const int j = j0 + q / CPR;
    const int c = q % CPR;
    if (j >= cnt) break;
    const int32_t src = a.kept_idx[(int64_t)u * a.B + j];
    if (src < 0 || src >= n) continue;
    const int64_t srow = beg + src;
    const int64_t drow = (int64_t)u * a.B + j;
    Ko[drow * CPR + c] = K[srow * CPR + c];
    Vo[drow * CPR + c] = V[srow * CPR + c];
    if (c == 0 && a.pos_out) a.pos_out[drow] = a.pos[srow];
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

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)a.n_units), dim3(kSelectThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const int64_t bpu = (a.B + kCompactRows - 1) / kCompactRows;
  const int64_t grid = bpu * a.n_units;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  switch (a.row_bytes / 16) {
    case 8: hipLaunchKernelGGL(compact_kernel<8>, dim3((unsigned)grid), dim3(kCompactThreads), 0, s, a, (int)bpu); break;
    case 16: hipLaunchKernelGGL(compact_kernel<16>, dim3((unsigned)grid), dim3(kCompactThreads), 0, s, a, (int)bpu); break;
    case 32: hipLaunchKernelGGL(compact_kernel<32>, dim3((unsigned)grid), dim3(kCompactThreads), 0, s, a, (int)bpu); break;
    case 64: hipLaunchKernelGGL(compact_kernel<64>, dim3((unsigned)grid), dim3(kCompactThreads), 0, s, a, (int)bpu); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tri
