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
#include "tri_device.h"

namespace tri {
namespace {

using dev::kDtBf16;
using dev::kDtF32;
using dev::kHalfSplit;
using dev::kInterleaved;
using dev::order_key;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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
  template <class T>
  __device__ __forceinline__ float x(const T& k, int j) const {
    return dot2(k.b[j], xh[j], dot2_z(k.b[j], xl[j]));
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
  template <class T>
  __device__ __forceinline__ float x(const T& k, int j) const {
    return fmaf(a[j], k.re[j], b[j] * k.im[j]);
  }
};

constexpr int kScoreThreads = 512;
constexpr int kRowsPerLoad = 4;  // rows per lane group in flight per iteration

template <int D>
constexpr int score_rows_per_block() { return 512; }

// The rotation phase of band j at distance dl, in revolutions (+1, which sine and cosine in
// revolutions ignore): ((dl * step) mod 2^23) / 2^23 + dl * resid, for dl < 2^24.
__device__ __forceinline__ float band_phase(uint32_t dl, float df, uint32_t step, float resid) {
  const uint32_t prod = mul_u24(dl, step);
  const float one_frac = __uint_as_float((prod & 0x7FFFFFu) | 0x3F800000u);
  return fmaf(df, resid, one_frac);
}

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

  const int unit = blockIdx.x / chunks_per_unit;
  const int chunk = blockIdx.x - unit * chunks_per_unit;
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
  KT kb[M];
  int32_t pb[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t row = min(wave_row + m * GPW, last);
    kb[m] = L::load(kbase, row, l);
    pb[m] = ROT ? 0 : pbase[row];
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
        pb[m] = ROT ? 0 : pbase[row];
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
