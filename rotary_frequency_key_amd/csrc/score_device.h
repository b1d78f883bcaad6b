// Device helpers of the score kernels (score.hip, score_max.hip): key-row loads, the center in
// the form the band product uses, the band phase and the row reduction.
#pragma once

#include "tri_device.h"

namespace tri {
namespace sdev {

using dev::kDtBf16;
using dev::kDtF32;
using dev::kHalfSplit;
using dev::kInterleaved;

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

// Streaming loads: every key is read once, so the loads carry the non-temporal hint (measured
// on the 8 x 32768 workload with the keys rotating over 536 MB: 13.7 vs 16.1 us per score launch).
// The address is a wave-uniform base plus a zero-extended 32-bit offset, so that the load takes
// the scalar-base form.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <class V>
__device__ __forceinline__ V ld_stream(const char* base, uint32_t off) {
  return __builtin_nontemporal_load(reinterpret_cast<const V*>(base + (uint64_t)off));
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
    const u32x4 v = ld_stream<u32x4>(base, row * kRowBytes + l * 16);
    return T{{v.x, v.y, v.z, v.w}};
  }
  static __device__ __forceinline__ T zero() { return T{{0u, 0u, 0u, 0u}}; }
};

template <int D>
struct RowLoad<kDtBf16, kHalfSplit, D> {
  struct T { uint32_t b[4]; };
  static constexpr int kRowBytes = D * 2;
  static __device__ __forceinline__ T load(const char* base, uint32_t row, int l) {
    const u32x2 re = ld_stream<u32x2>(base, row * kRowBytes + l * 8);
    const u32x2 im = ld_stream<u32x2>(base, row * kRowBytes + D + l * 8);
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
    const f32x4 a = ld_stream<f32x4>(base, row * kRowBytes + l * 32);
    const f32x4 b = ld_stream<f32x4>(base, row * kRowBytes + l * 32 + 16);
    return T{{a.x, a.z, b.x, b.z}, {a.y, a.w, b.y, b.w}};
  }
  static __device__ __forceinline__ T zero() { return T{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}; }
};

template <int D>
struct RowLoad<kDtF32, kHalfSplit, D> {
  struct T { float re[4], im[4]; };
  static constexpr int kRowBytes = D * 4;
  static __device__ __forceinline__ T load(const char* base, uint32_t row, int l) {
    const f32x4 a = ld_stream<f32x4>(base, row * kRowBytes + l * 16);
    const f32x4 b = ld_stream<f32x4>(base, row * kRowBytes + D * 2 + l * 16);
    return T{{a.x, a.y, a.z, a.w}, {b.x, b.y, b.z, b.w}};
  }
  static __device__ __forceinline__ T zero() { return T{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}; }
};

// The key's position (read once, like the key).
__device__ __forceinline__ int32_t load_pos(const int32_t* base, uint32_t row) {
  return ld_stream<int32_t>(reinterpret_cast<const char*>(base), row * 4u);
}

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

// The rotation phase of band j at distance dl, in revolutions (+1, which sine and cosine in
// revolutions ignore): ((dl * step) mod 2^23) / 2^23 + dl * resid, for dl < 2^24.
__device__ __forceinline__ float band_phase(uint32_t dl, float df, uint32_t step, float resid) {
  const uint32_t prod = mul_u24(dl, step);
  const float one_frac = __uint_as_float((prod & 0x7FFFFFu) | 0x3F800000u);
  return fmaf(df, resid, one_frac);
}

}  // namespace sdev
}  // namespace tri
