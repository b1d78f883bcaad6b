// Device helpers shared by the libtri kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tri_internal.h"

namespace tri {
namespace dev {

constexpr int kDtF32 = 0;
constexpr int kDtBf16 = 1;
constexpr int kInterleaved = 0;
constexpr int kHalfSplit = 1;

// Total order on binary32 scores as unsigned integers: larger score -> larger key;
// -0.0 and +0.0 map to one key; every NaN maps to 0, below -inf (0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t b = __float_as_uint(s);
  const uint32_t mag = b & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return 0u;
  if (mag == 0u) return 0x80000000u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Rows [beg, end) of unit u, clamped to [0, total_rows) and to max_rows rows.
struct UnitRows {
  int64_t beg, n;
};

__device__ __forceinline__ UnitRows unit_rows(const int64_t* row_off, int u, int64_t total_rows,
                                              int64_t max_rows) {
  int64_t beg = row_off[u], end = row_off[u + 1];
  beg = beg < 0 ? 0 : (beg > total_rows ? total_rows : beg);
  end = end < beg ? beg : (end > total_rows ? total_rows : end);
  if (end - beg > max_rows) end = beg + max_rows;
  return UnitRows{beg, end - beg};
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// DPP lane move: lanes whose source is out of range, or whose row is masked off, read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: Hillis-Steele within each row of
// 16 lanes (row_shr 1, 2, 4, 8), then row 0's total into rows 1 and 3 (row_bcast:15) and row 1's
// into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
  v += dpp_u<0x111>(v);        // row_shr:1
  v += dpp_u<0x112>(v);        // row_shr:2
  v += dpp_u<0x114>(v);        // row_shr:4
  v += dpp_u<0x118>(v);        // row_shr:8
  v += dpp_u<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
  v += dpp_u<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
  return v;
}

// Value of lane 63 (the wave total after an inclusive scan), uniform.
__device__ __forceinline__ uint32_t wave_last(uint32_t v) { return (uint32_t)__builtin_amdgcn_readlane((int)v, 63); }

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Exclusive prefix sum over a block of NT threads; *total receives the block sum.
// sh: >= NT/64 words of LDS. Contains __syncthreads(); call from every thread.
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

// Exclusive prefix sum over a block of NT threads with DPP wave scans and two barriers.
// sh: >= 2 * NT/64 words of LDS. *total receives the block sum. Call from every thread.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan_dpp(uint32_t v, uint32_t* sh, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan_dpp(v);
  if (lane == 63) sh[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    uint32_t w = lane < NW ? sh[lane] : 0u;
    w = wave_incl_scan_dpp(w);
    if (lane < NW) sh[NW + lane] = w;
  }
  __syncthreads();
  *total = sh[2 * NW - 1];
  return (wid ? sh[NW + wid - 1] : 0u) + inc - v;
}

// Two exclusive prefix sums over a block of NT threads sharing two barriers. sh: >= 4 * NT/64
// words of LDS. *ta, *tb receive the block sums. Call from every thread.
template <int NT>
__device__ __forceinline__ void block_excl_scan2_dpp(uint32_t a, uint32_t b, uint32_t* sh, uint32_t* ea,
                                                     uint32_t* eb, uint32_t* ta, uint32_t* tb) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t ia = wave_incl_scan_dpp(a), ib = wave_incl_scan_dpp(b);
  if (lane == 63) { sh[wid] = ia; sh[NW + wid] = ib; }
  __syncthreads();
  if (wid == 0) {
    uint32_t x = lane < NW ? sh[lane] : 0u, y = lane < NW ? sh[NW + lane] : 0u;
    x = wave_incl_scan_dpp(x);
    y = wave_incl_scan_dpp(y);
    if (lane < NW) { sh[2 * NW + lane] = x; sh[3 * NW + lane] = y; }
  }
  __syncthreads();
  *ta = sh[3 * NW - 1];
  *tb = sh[4 * NW - 1];
  *ea = (wid ? sh[2 * NW + wid - 1] : 0u) + ia - a;
  *eb = (wid ? sh[3 * NW + wid - 1] : 0u) + ib - b;
}

template <int NT>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* sh) {
  uint32_t tot;
  block_excl_scan<NT>(v, sh, &tot);
  return tot;
}

// In h[0..nb) (nb a multiple of NT): the bin b with above(b) < rank <= above(b) + h[b],
// above(b) = sum of the bins above b. Requires 1 <= rank <= sum(h). h may be global or LDS.
// found: 2 words of LDS. Returns b; *above_out = above(b).
template <int NT, class H>
__device__ uint32_t find_bin(const H* h, int nb, uint32_t rank, uint32_t* sh, uint32_t* found,
                             uint32_t* above_out) {
  const int per = nb / NT;
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

// Workgroup index for grids of at most kXcdRemapMaxGrid workgroups, remapped so that consecutive
// indices run on one XCD: workgroup i is dispatched to XCD i mod 8, and index
// (i mod 8) * (G / 8) + i / 8 (plus the remainder's share) gives each XCD one contiguous block of
// the grid. With unit-major grids, a unit's workgroups then share an L2 in every kernel of the
// pass, so the next kernel finds the scores, histogram and candidates it reads in that L2. Such a
// grid runs in one wave, so no XCD gets more than its share of it. Larger grids keep launch
// order, in which neighbouring workgroups stream neighbouring rows.
constexpr int kXcdRemapMaxGrid = 512;
__device__ __forceinline__ int xcd_block(int i, int G) {
  if (G > kXcdRemapMaxGrid) return i;
  const int x = i & 7, l = i >> 3, per = G >> 3, extra = G & 7;
  return x * per + (x < extra ? x : extra) + l;
}

}  // namespace dev
}  // namespace tri
