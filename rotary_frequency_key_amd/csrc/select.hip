// Top-B select of libtri for gfx950: keep the B highest scores of each unit, equal scores by
// lower row index, kept row indices written in ascending order; optionally gather the kept K/V
// rows and positions in the same pass.
//
// "The future-offset average in TriAttention can be precomputed", introduction: when the cache
// must be trimmed every key is scored and the highest-scoring ones are kept; the TriAttention
// README sets how many are kept per cache (the KV budget).
//
// Scores are compared as 32-bit order keys (dev::order_key). The B-th largest key T is found by
// radix select: bits 31..20 from the unit's top-digit histogram (added by the score kernel, or
// built here), then bits 19..10 and 9..0 among the keys whose top digit is the threshold's
// ("candidates"). Kept rows: key > T, and the `need` lowest-index rows with key == T.
//
//  threshold_kernel  one workgroup (1024 threads) per unit: one pass over the unit's scores
//                    counts, per chunk of rows, the keys above the threshold's top digit and
//                    collects the candidates in LDS; the last two digits are resolved among the
//                    candidates and per-chunk kept counts become per-chunk output offsets, all
//                    with block-wide DPP scans. Leaves the unit's histogram at zero.
//  emit_kernel       one workgroup (1024 threads, one row each) per chunk: re-reads the chunk,
//                    writes each kept row's index at  offset(chunk) + (rows kept before it in
//                    the chunk)  and, when fused, copies the chunk's kept rows, four 16-byte
//                    pieces of K and of V per thread per round, so that even a chunk whose rows
//                    are all kept takes four rounds.
#include "tri_device.h"

namespace tri {
namespace {

using dev::order_key;
using dev::wave_incl_scan_dpp;

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t readlane(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

struct WsPtrs {
  uint32_t* hist;
  UnitState* state;
  uint32_t* chunk_off;
  uint32_t* chunk_eq;
};

__device__ __forceinline__ WsPtrs ws_ptrs(const SelectArgs& a) {
  char* ws = reinterpret_cast<char*>(a.ws);
  return WsPtrs{reinterpret_cast<uint32_t*>(ws + a.lay.hist), reinterpret_cast<UnitState*>(ws + a.lay.state),
                reinterpret_cast<uint32_t*>(ws + a.lay.chunk_off), reinterpret_cast<uint32_t*>(ws + a.lay.chunk_eq)};
}

// ---------------------------------------------------------------------------------------------
// threshold
// ---------------------------------------------------------------------------------------------

constexpr int kTN = 1024;              // threads
constexpr int kTW = kTN / 64;          // waves
constexpr int kTPer = 32;              // rows per lane per tile
constexpr int kWaveRows = kTPer * 64;  // 2048 rows per wave per tile
constexpr int kTTile = kTN * kTPer;    // 32768 rows per tile

struct ThrShared {
  uint32_t hist[kHistBins];       // histogram built here when the score kernel did not
  uint32_t cand_key[kCandCap];
  uint32_t cand_row[kCandCap];
  uint32_t rhist[1024];           // radix bins of digits 2 and 3
  uint32_t gt_b0[kMaxChunks];     // per chunk: keys whose top digit is above b0
  uint32_t cnt_gt[kMaxChunks];    // per chunk: candidates above T
  uint32_t cnt_eq[kMaxChunks];    // per chunk: candidates equal to T
  uint32_t sh[2 * kTW];
  uint32_t ncand, found_b, found_above;
};

__device__ __forceinline__ float load_at(const float* s, uint32_t row) {
  // uniform base + 32-bit byte offset (units are below 2^29 rows): one address register
  return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(s) + row * 4u);
}

// Keys of one tile for this lane: rows t0 + wave*2048 + j*64 + lane, j < 32. Rows at or past
// n (n >= 1) read row n-1; callers mask them by index.
__device__ __forceinline__ void load_tile(const float* s, uint32_t n, uint32_t t0, uint32_t (&k)[kTPer]) {
  const uint32_t last = n - 1;
  const uint32_t base = t0 + (threadIdx.x >> 6) * kWaveRows + (threadIdx.x & 63);
#pragma unroll
  for (int j = 0; j < kTPer; ++j) {
    const uint32_t r = base + j * 64;
    k[j] = order_key(load_at(s, r < last ? r : last));
  }
}

// Block-wide: thread t holds the counts v[0..PER) of bins top_t, top_t - 1, ... where
// top_t = nb - 1 - t*PER (bins descending with t). Finds the bin b with
// above(b) < rank <= above(b) + count(b); results via LDS, uniform.
template <int PER>
__device__ __forceinline__ uint32_t block_find_bin(ThrShared& L, const uint32_t (&v)[PER], int nb, uint32_t rank,
                                                   uint32_t* above_out) {
  uint32_t loc = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) loc += v[q];
  if (threadIdx.x == 0) { L.found_b = 0u; L.found_above = 0u; }
  uint32_t tot;
  uint32_t c = dev::block_excl_scan_dpp<kTN>(loc, L.sh, &tot);
  const int top = nb - 1 - (int)threadIdx.x * PER;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    if (c < rank && rank <= c + v[q]) { L.found_b = (uint32_t)(top - q); L.found_above = c; }
    c += v[q];
  }
  __syncthreads();
  *above_out = L.found_above;
  return L.found_b;
}

// Radix digit over LDS bins rhist[0..1024): one bin per thread.
__device__ __forceinline__ uint32_t rhist_find(ThrShared& L, uint32_t rank, uint32_t* above_out) {
  const uint32_t v[1] = {L.rhist[1023 - threadIdx.x]};
  return block_find_bin<1>(L, v, 1024, rank, above_out);
}

template <bool MULTI, bool READY>  // units above one tile; histogram added by the score kernel
__global__ __launch_bounds__(kTN) void threshold_kernel(SelectArgs a) {
  __shared__ ThrShared L;
  const int u = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int C = a.lay.chunks, cshift = a.lay.chunk_shift;
  const WsPtrs w = ws_ptrs(a);
  const dev::UnitRows ur = dev::unit_rows(a.row_off, u, a.total_rows, a.max_rows);
  const uint32_t n = (uint32_t)ur.n;
  const uint32_t m = (uint32_t)a.B < n ? (uint32_t)a.B : n;
  const float* s = a.scores + ur.beg;
  uint32_t* gh = w.hist + (size_t)u * kHistBins;
  UnitState* st = w.state + u;

  if (m == n || m == 0) {  // keep every row, or none
    if (threadIdx.x == 0) { st->mode = m == 0 ? kModeNone : kModeAll; st->m = m; }
    if (READY)
      for (int i = threadIdx.x; i < kHistBins; i += kTN) gh[i] = 0u;
    return;
  }

  // ---- loads first: this thread's 4 histogram bins (descending: 4095-4t .. 4092-4t) and
  // the first tile of keys
  uint32_t hb[4] = {0u, 0u, 0u, 0u};
  if (READY) {
    const uint4 h = reinterpret_cast<const uint4*>(gh)[(kHistBins / 4) - 1 - threadIdx.x];
    hb[0] = h.w; hb[1] = h.z; hb[2] = h.y; hb[3] = h.x;
  }
  uint32_t k[kTPer];
  if (!MULTI) load_tile(s, n, 0, k);
  if (threadIdx.x == 0) L.ncand = 0u;
  for (int i = threadIdx.x; i < C; i += kTN) { L.gt_b0[i] = 0u; L.cnt_gt[i] = 0u; L.cnt_eq[i] = 0u; }
  if (READY) {
    // back to rest: each thread clears the four bins it read (no other thread reads them)
    reinterpret_cast<uint4*>(gh)[(kHistBins / 4) - 1 - threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  } else {
    for (int i = threadIdx.x; i < kHistBins; i += kTN) L.hist[i] = 0u;
    __syncthreads();
    if (MULTI) {
      for (uint32_t i = threadIdx.x; i < n; i += kTN) atomicAdd(&L.hist[order_key(load_at(s, i)) >> kHistShift], 1u);
    } else {
      const uint32_t base = wave * kWaveRows + lane;
#pragma unroll
      for (int j = 0; j < kTPer; ++j)
        if (base + j * 64 < n) atomicAdd(&L.hist[k[j] >> kHistShift], 1u);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) hb[q] = L.hist[kHistBins - 1 - 4 * threadIdx.x - q];
  }

  // ---- digit 1
  uint32_t above0;
  const uint32_t b0 = block_find_bin<4>(L, hb, kHistBins, m, &above0);

  // ---- one pass: per-chunk counts of keys above bin b0, candidates (bin b0) into LDS. A wave's
  // 2048 rows of a tile lie in at most two chunks (chunk_rows >= 1024, aligned): steps 0..15
  // and steps 16..31.
  for (uint32_t t0 = 0; t0 < n; t0 += kTTile) {
    if (MULTI) load_tile(s, n, t0, k);
    const uint32_t wbase = t0 + wave * kWaveRows;
    uint32_t gt_lo = 0, gt_hi = 0, nc_l = 0;
#pragma unroll
    for (int j = 0; j < kTPer; ++j) {
      const bool in = wbase + j * 64 + lane < n;
      const uint32_t d = k[j] >> kHistShift;
      const uint32_t g = (in && d > b0) ? 1u : 0u;
      if (j < kTPer / 2) gt_lo += g; else gt_hi += g;
      nc_l += (in && d == b0) ? 1u : 0u;
    }
    const uint32_t lo_sum = dev::wave_last(wave_incl_scan_dpp(gt_lo));
    const uint32_t hi_sum = dev::wave_last(wave_incl_scan_dpp(gt_hi));
    const uint32_t c_inc = wave_incl_scan_dpp(nc_l);
    const uint32_t c_tot = dev::wave_last(c_inc);
    uint32_t cbase = 0;
    if (lane == 0) {
      if (lo_sum) atomicAdd(&L.gt_b0[wbase >> cshift], lo_sum);
      if (hi_sum) atomicAdd(&L.gt_b0[(wbase + kWaveRows / 2) >> cshift], hi_sum);
      if (c_tot) cbase = atomicAdd(&L.ncand, c_tot);
    }
    if (c_tot) {
      uint32_t p = readlane(cbase, 0) + c_inc - nc_l;
#pragma unroll
      for (int j = 0; j < kTPer; ++j) {
        const uint32_t r = wbase + j * 64 + lane;
        if (r < n && (k[j] >> kHistShift) == b0) {
          if (p < (uint32_t)kCandCap) { L.cand_key[p] = k[j]; L.cand_row[p] = r; }
          ++p;
        }
      }
    }
  }
  __syncthreads();
  const uint32_t nc = L.ncand;
  const bool in_lds = nc <= (uint32_t)kCandCap;

  // ---- digits 2 and 3 among the candidates (or, if they overflowed, among the scores)
  uint32_t r = m - above0, pre = b0;
  for (int digit = 0; digit < 2; ++digit) {
    const int sh = digit == 0 ? 10 : 0;
    L.rhist[threadIdx.x] = 0u;
    __syncthreads();
    if (in_lds) {
      for (uint32_t j = threadIdx.x; j < nc; j += kTN) {
        const uint32_t kk = L.cand_key[j];
        if ((kk >> (sh + 10)) == pre) atomicAdd(&L.rhist[(kk >> sh) & 1023u], 1u);
      }
    } else {
      for (uint32_t i = threadIdx.x; i < n; i += kTN) {
        const uint32_t kk = order_key(load_at(s, i));
        if ((kk >> (sh + 10)) == pre) atomicAdd(&L.rhist[(kk >> sh) & 1023u], 1u);
      }
    }
    __syncthreads();
    uint32_t above;
    const uint32_t b = rhist_find(L, r, &above);
    r -= above;
    pre = (pre << 10) | b;
  }
  const uint32_t T = pre, need = r;

  // ---- per chunk: candidates above T and equal to T
  if (in_lds) {
    for (uint32_t j = threadIdx.x; j < nc; j += kTN) {
      const uint32_t kk = L.cand_key[j];
      const uint32_t c = L.cand_row[j] >> cshift;
      if (kk > T) atomicAdd(&L.cnt_gt[c], 1u);
      else if (kk == T) atomicAdd(&L.cnt_eq[c], 1u);
    }
  } else {
    for (uint32_t i = threadIdx.x; i < n; i += kTN) {
      const uint32_t kk = order_key(load_at(s, i));
      if ((kk >> kHistShift) != b0) continue;
      if (kk > T) atomicAdd(&L.cnt_gt[i >> cshift], 1u);
      else if (kk == T) atomicAdd(&L.cnt_eq[i >> cshift], 1u);
    }
  }
  __syncthreads();

  // ---- per-chunk output offsets; ties at T are kept lowest chunks first. Thread t owns chunks
  // 2t and 2t+1.
  uint32_t e[2], kg[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = 2 * threadIdx.x + q;
    e[q] = c < C ? L.cnt_eq[c] : 0u;
    kg[q] = c < C ? L.gt_b0[c] + L.cnt_gt[c] : 0u;
  }
  uint32_t tot;
  uint32_t E = dev::block_excl_scan_dpp<kTN>(e[0] + e[1], L.sh, &tot);
  uint32_t kept[2];
  const uint32_t E_first = E;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t ties = E >= need ? 0u : (need - E < e[q] ? need - E : e[q]);
    kept[q] = kg[q] + ties;
    E += e[q];
  }
  uint32_t off = dev::block_excl_scan_dpp<kTN>(kept[0] + kept[1], L.sh, &tot);
  E = E_first;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = 2 * threadIdx.x + q;
    if (c < C) {
      w.chunk_off[(size_t)u * C + c] = off;
      w.chunk_eq[(size_t)u * C + c] = E;
    }
    off += kept[q];
    E += e[q];
  }
  if (threadIdx.x == 0) { st->T = T; st->need = need; st->mode = kModeThreshold; st->m = m; }
}

// ---------------------------------------------------------------------------------------------
// emit (and gather)
// ---------------------------------------------------------------------------------------------

constexpr int kEN = 1024;       // threads: one row of a 1024-row sub-chunk each
constexpr int kEW = kEN / 64;   // waves
constexpr int kSub = kEN;       // rows per sub-chunk

// Copy rows staged in LDS: src[j] (unit-local row) -> output slot lo + j, j < cnt. Each thread
// moves 4 pieces of K and of V per round, all loads issued before the stores.
struct Piece {
  uint4 k, v;
  uint32_t q;
};

// Staged rows are unit-local indices below n; one that is not (only with an inconsistent
// workspace) is read as row n-1 and never stored.
template <int CPR>
__device__ __forceinline__ Piece load_piece(const uint4* __restrict__ K, const uint4* __restrict__ V, int64_t beg,
                                            uint32_t n, const uint32_t* src, uint32_t q, uint32_t total) {
  const uint32_t qc = q < total ? q : total - 1;  // past the end: load the last piece again
  Piece p;
  p.q = q;
  const uint32_t sr = src[qc / CPR];
  const int64_t srow = beg + (sr < n ? sr : n - 1);
  p.k = K[srow * CPR + qc % CPR];
  p.v = V[srow * CPR + qc % CPR];
  return p;
}

template <int CPR>
__device__ __forceinline__ void store_piece(const SelectArgs& a, uint4* __restrict__ Ko, uint4* __restrict__ Vo,
                                            int64_t beg, uint32_t n, const uint32_t* src, int64_t out0,
                                            const Piece& p, uint32_t total) {
  if (p.q >= total) return;
  const uint32_t j = p.q / CPR, part = p.q % CPR;
  if (src[j] >= n) return;
  Ko[(out0 + j) * CPR + part] = p.k;
  Vo[(out0 + j) * CPR + part] = p.v;
  if (part == 0 && a.pos_out) a.pos_out[out0 + j] = a.pos[beg + src[j]];
}

template <int CPR>
__device__ __forceinline__ void gather_staged(const SelectArgs& a, int u, int64_t beg, uint32_t n,
                                              const uint32_t* src, uint32_t lo, uint32_t cnt) {
  const uint4* __restrict__ K = static_cast<const uint4*>(a.K);
  const uint4* __restrict__ V = static_cast<const uint4*>(a.V);
  uint4* __restrict__ Ko = static_cast<uint4*>(a.K_out);
  uint4* __restrict__ Vo = static_cast<uint4*>(a.V_out);
  const uint32_t total = cnt * CPR;
  const int64_t out0 = (int64_t)u * a.B + lo;
  for (uint32_t q0 = threadIdx.x; q0 < total; q0 += 4 * kEN) {
    const Piece p0 = load_piece<CPR>(K, V, beg, n, src, q0, total);
    const Piece p1 = load_piece<CPR>(K, V, beg, n, src, q0 + kEN, total);
    const Piece p2 = load_piece<CPR>(K, V, beg, n, src, q0 + 2 * kEN, total);
    const Piece p3 = load_piece<CPR>(K, V, beg, n, src, q0 + 3 * kEN, total);
    store_piece<CPR>(a, Ko, Vo, beg, n, src, out0, p0, total);
    store_piece<CPR>(a, Ko, Vo, beg, n, src, out0, p1, total);
    store_piece<CPR>(a, Ko, Vo, beg, n, src, out0, p2, total);
    store_piece<CPR>(a, Ko, Vo, beg, n, src, out0, p3, total);
  }
}

template <int CPR>  // 16-byte pieces per K/V row; 0: no gather
__global__ __launch_bounds__(kEN) void emit_kernel(SelectArgs a) {
  __shared__ uint32_t wcnt[kEW];
  __shared__ uint32_t staged[kSub];  // unit-local rows kept in the current sub-chunk, in slot order
  const int C = a.lay.chunks, CH = a.lay.chunk_rows;
  const int u = blockIdx.x / C, c = blockIdx.x - u * C;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const WsPtrs w = ws_ptrs(a);
  const dev::UnitRows ur = dev::unit_rows(a.row_off, u, a.total_rows, a.max_rows);
  const uint32_t n = (uint32_t)ur.n;
  const uint32_t i0 = (uint32_t)c * CH;
  const float* sc = a.scores + ur.beg;
  // this thread's first key, issued together with the unit state
  const uint32_t r_first = i0 + threadIdx.x;
  const float s_first = r_first < n ? load_at(sc, r_first) : 0.f;
  const UnitState* st = w.state + u;
  const uint32_t mode = st->mode, m = st->m;
  const uint32_t T = st->T, need = st->need;
  const uint32_t off = w.chunk_off[(size_t)u * C + c];
  const uint32_t E0 = w.chunk_eq[(size_t)u * C + c];
  int32_t* out = a.kept_idx + (int64_t)u * a.B;
  if (c == 0) {
    for (uint32_t j = m + threadIdx.x; j < (uint32_t)a.B; j += kEN) out[j] = -1;
    if (threadIdx.x == 0) a.kept_cnt[u] = (int32_t)m;
  }
  if (i0 >= n || mode == kModeNone) return;
  const uint32_t i1 = n - i0 < (uint32_t)CH ? n : i0 + CH;

  if (mode == kModeAll) {  // slot = row
    for (uint32_t t0 = i0; t0 < i1; t0 += kSub) {
      const uint32_t cnt = i1 - t0 < (uint32_t)kSub ? i1 - t0 : (uint32_t)kSub;
      if (threadIdx.x < cnt) { out[t0 + threadIdx.x] = (int32_t)(t0 + threadIdx.x); staged[threadIdx.x] = t0 + threadIdx.x; }
      if constexpr (CPR > 0) {
        __syncthreads();
        gather_staged<CPR>(a, u, ur.beg, n, staged, t0, cnt);
        __syncthreads();
      }
    }
    return;
  }

  const uint32_t ties0 = E0 < need ? E0 : need;  // ties kept before this chunk
  uint32_t run_g = 0, run_e = E0;                 // greater keys / ties before the sub-chunk
  for (uint32_t t0 = i0; t0 < i1; t0 += kSub) {
    const uint32_t r = t0 + threadIdx.x;
    const bool in = r < i1;
    const uint32_t k = order_key(t0 == i0 ? s_first : load_at(sc, in ? r : i1 - 1));  // i1 > i0 here
    const bool gt = in && k > T, eq = in && k == T;
    const uint64_t mg = __ballot(gt), me = __ballot(eq);
    __syncthreads();
    if (lane == 0) wcnt[wave] = ((uint32_t)__popcll(mg) << 16) | (uint32_t)__popcll(me);
    __syncthreads();
    uint32_t pg = run_g, pe = run_e, tg = 0, te = 0;
#pragma unroll
    for (int v = 0; v < kEW; ++v) {
      const uint32_t x = wcnt[v];
      if (v < wave) { pg += x >> 16; pe += x & 0xFFFFu; }
      tg += x >> 16;
      te += x & 0xFFFFu;
    }
    const uint32_t sub0 = run_g + (run_e < need ? run_e : need) - ties0;  // kept before the sub-chunk
    const uint32_t G_ = pg + lanes_below(mg), E_ = pe + lanes_below(me);
    if (gt || (eq && E_ < need)) {
      const uint32_t local = G_ + (E_ < need ? E_ : need) - ties0;  // kept before it in the chunk
      if (off + local < m) out[off + local] = (int32_t)r;
      if (local - sub0 < (uint32_t)kSub) staged[local - sub0] = r;
    }
    run_g += tg;
    run_e += te;
    if constexpr (CPR > 0) {
      const uint32_t sub1 = run_g + (run_e < need ? run_e : need) - ties0;
      uint32_t cnt = sub1 - sub0;
      if (off + sub0 >= m) cnt = 0;
      else if (off + sub1 > m) cnt = m - off - sub0;
      if (cnt > (uint32_t)kSub) cnt = kSub;
      __syncthreads();
      gather_staged<CPR>(a, u, ur.beg, n, staged, off + sub0, cnt);
    }
  }
}

template <int CPR>
void launch_emit(const SelectArgs& a, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL(emit_kernel<CPR>, dim3(grid), dim3(kEN), 0, s, a);
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.lay.chunks * a.n_units;  // one emit workgroup per chunk
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 tg((unsigned)a.n_units), tb(kTN);
  const bool multi = a.max_rows > kTTile;
  if (a.hist_ready) {
    if (multi) hipLaunchKernelGGL((threshold_kernel<true, true>), tg, tb, 0, s, a);
    else hipLaunchKernelGGL((threshold_kernel<false, true>), tg, tb, 0, s, a);
  } else {
    if (multi) hipLaunchKernelGGL((threshold_kernel<true, false>), tg, tb, 0, s, a);
    else hipLaunchKernelGGL((threshold_kernel<false, false>), tg, tb, 0, s, a);
  }
  if (a.K_out == nullptr) {
    launch_emit<0>(a, (unsigned)grid, s);
  } else {
    switch (a.row_bytes / 16) {
      case 8: launch_emit<8>(a, (unsigned)grid, s); break;
      case 16: launch_emit<16>(a, (unsigned)grid, s); break;
      case 32: launch_emit<32>(a, (unsigned)grid, s); break;
      case 64: launch_emit<64>(a, (unsigned)grid, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace tri
