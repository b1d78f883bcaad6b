// Top-B select of libtri for gfx950: keep the B highest scores of each unit, equal scores by
// lower row index, kept row indices written in ascending order; optionally gather the kept K/V
// rows and positions in the same pass.
//
// "The future-offset average in TriAttention can be precomputed", introduction: when the cache
// must be trimmed every key is scored and the highest-scoring ones are kept; the TriAttention
// README sets how many are kept per cache (the KV budget).
//
// Scores are compared as 32-bit order keys (dev::order_key). The B-th largest key T is found by
// radix select: bits 31..20 from the unit's top-digit histogram (added by the score kernel, or by
// hist_kernel here), then bits 19..10 and 9..0 among the keys whose top digit is the threshold's
// ("candidates"). Kept rows: key > T, and the `need` lowest-index rows with key == T.
//
// Three arrangements of the same select, chosen on the host from the unit count and max_rows
// (all give the same bits):
//
//  * Units of up to 64Ki rows, 48 units or more with 384 groups of 64 output slots or more (a few
//    layers or more in one call):
//      topb_kernel -> compact_kernel
//    One workgroup per unit with the keys in registers; from a few dozen units on, many units'
//    selects run at once, and the other arrangement's resolve in every output workgroup costs
//    more.
//  * Otherwise, units of up to 2^18 rows whose output slots make at most kFinishMaxWorkgroups
//    groups of 64 in all (a few layers' heads, budgets of a few thousand):
//      cand_kernel -> finish_kernel
//    A unit is spread over many workgroups: one workgroup sees only a fraction of the HBM
//    bandwidth and one CU's VALU, so a per-unit pass over 32k scores in one workgroup, or a
//    dense run of kept rows gathered by one workgroup, would set the time of the whole call.
//  * Everything else (longer units, or many slots): cand_kernel -> resolve_kernel -> emit_kernel.
//  The in-place pass uses topb_kernel (up to 64Ki rows) or cand/resolve/mark_kernel, then
//  move_kernel.
//
//  hist_kernel     (standalone select only) top-digit histogram, 4096 rows per workgroup.
//  cand_kernel     512 threads per chunk of 1024 rows (or one granule, if larger), or 256 per up
//                  to 16 consecutive chunks of a unit when the grid is large: finds the threshold's
//                  top digit b0 from the histogram, counts per granule the keys above it and
//                  writes each chunk's candidates, packed, to the chunk's own region.
//  finish_kernel   one workgroup per 64 output slots: resolves digits 2 and 3 from the unit's
//                  candidates itself, finds the granules whose kept rows land in its slots, and
//                  writes and gathers those rows.
//  resolve_kernel  one workgroup per unit: clears the histogram, stages the candidates in LDS,
//                  resolves digits 2 and 3, and turns per-granule kept counts into per-granule
//                  output offsets and counts of ties before each granule (block-wide DPP scans).
//                  (Resolving in the candidate kernel's last workgroup per unit would need an
//                  agent-scope release in every workgroup, an L2 writeback each, which costs far
//                  more here than the kernel boundary.)
//  emit_kernel     one wave per granule (64 rows unless units are very long) writes each kept
//                  row's index at  offset(granule) + (rows kept before it in the granule). When
//                  fused, a granule has a second wave: the first copies the kept K rows and the
//                  positions, the second the V rows, up to 8 loads of 16 bytes per lane in flight
//                  (a dense run of kept rows is spread over many waves, not one CU).
//  topb_kernel     one 1024-thread workgroup per unit, all three digits over keys held in
//                  registers; writes the kept indices (or the in-place lists) itself.
#include "stamps.h"
#include "tri_device.h"

namespace tri {

TRI_STAMPS_BUFFER(g_stamps_select)

namespace {

using dev::order_key;

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

struct WsPtrs {
  uint32_t* hist;
  UnitState* state;
  uint32_t* wg_cnt;
  uint32_t* cand;
  uint32_t* gran_gt;
  uint32_t* gran_off;
  uint32_t* gran_eq;
};

__device__ __forceinline__ WsPtrs ws_ptrs(const SelectArgs& a) {
  char* ws = reinterpret_cast<char*>(a.ws);
  return WsPtrs{reinterpret_cast<uint32_t*>(ws + a.lay.hist),     reinterpret_cast<UnitState*>(ws + a.lay.state),
                reinterpret_cast<uint32_t*>(ws + a.lay.wg_cnt),   reinterpret_cast<uint32_t*>(ws + a.lay.cand),
                reinterpret_cast<uint32_t*>(ws + a.lay.gran_gt),  reinterpret_cast<uint32_t*>(ws + a.lay.gran_off),
                reinterpret_cast<uint32_t*>(ws + a.lay.gran_eq)};
}

__device__ __forceinline__ float load_at(const float* s, uint32_t row) {
  // uniform base + 32-bit byte offset (units are below 2^29 rows): one address register
  return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(s) + row * 4u);
}

// Block-wide radix-bin search. Thread t holds the counts v[0..PER) of bins top_t, top_t - 1, ...
// with top_t = nb - 1 - t*PER (bins descending with t). Returns the bin b with
// above(b) < rank <= above(b) + count(b), above(b) = sum of the bins above b; *above_out =
// above(b). Uniform; bin 0 and 0 if no bin qualifies (only with inconsistent counts).
// sh: 2*NT/64 words, found: 2 words of LDS. Call from every thread.
template <int NT, int PER>
__device__ __forceinline__ uint32_t block_find(const uint32_t (&v)[PER], int nb, uint32_t rank, uint32_t* sh,
                                               uint32_t* found, uint32_t* above_out) {
  uint32_t loc = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) loc += v[q];
  if (threadIdx.x == 0) { found[0] = 0u; found[1] = 0u; }
  uint32_t tot;
  uint32_t c = dev::block_excl_scan_dpp<NT>(loc, sh, &tot);
  const int top = nb - 1 - (int)threadIdx.x * PER;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    if (c < rank && rank <= c + v[q]) { found[0] = (uint32_t)(top - q); found[1] = c; }
    c += v[q];
  }
  __syncthreads();
  *above_out = found[1];
  return found[0];
}

// ---------------------------------------------------------------------------------------------
// histogram (standalone select; the fused pass takes it from the score kernel)
// ---------------------------------------------------------------------------------------------

constexpr int kHN = 256;
constexpr int kHPer = 16;
constexpr int kHRows = kHN * kHPer;

__global__ __launch_bounds__(kHN) void hist_kernel(SelectArgs a, int hpu) {
  __shared__ uint32_t lh[kHistBins];
  const int u = blockIdx.x / hpu, c = blockIdx.x - u * hpu;
  const dev::UnitRows ur = dev::unit_rows(a.row_off, u, a.total_rows, a.max_rows);
  const uint32_t n = (uint32_t)ur.n, r0 = (uint32_t)c * kHRows;
  if (r0 >= n) return;
  const float* s = a.scores + ur.beg;
  const uint32_t last = n - 1;
  uint32_t k[kHPer];
#pragma unroll
  for (int j = 0; j < kHPer; ++j) {
    const uint32_t r = r0 + j * kHN + threadIdx.x;
    k[j] = order_key(load_at(s, r < last ? r : last));
  }
  for (int i = threadIdx.x; i < kHistBins; i += kHN) lh[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kHPer; ++j)
    if (r0 + j * kHN + threadIdx.x < n) atomicAdd(&lh[k[j] >> kHistShift], 1u);
  __syncthreads();
  uint32_t* gh = ws_ptrs(a).hist + (size_t)u * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kHN) {
    const uint32_t v = lh[i];
    if (v) atomicAdd(&gh[i], v);
  }
}

// ---------------------------------------------------------------------------------------------
// candidates
// ---------------------------------------------------------------------------------------------

// Threads per candidate workgroup: 512 (2 rows each per 1024-row tile) when a workgroup takes one
// chunk, where the launch is latency-bound and more threads shorten the histogram scan; 256 (4
// rows each) when it takes several, where the per-tile block scan over fewer waves costs less.
constexpr int kCTile = 1 << kCandRowsShift;  // rows per tile

// Keys of rows t0 + j*NT + threadIdx.x (j < PER); rows at or past r1 (> t0) read row r1 - 1.
template <int NT, int PER>
__device__ __forceinline__ void load_cand_tile(const float* s, uint32_t r1, uint32_t t0, uint32_t (&k)[PER]) {
  const uint32_t last = r1 - 1;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t r = t0 + j * NT + threadIdx.x;
    k[j] = order_key(load_at(s, r < last ? r : last));
  }
}

// Each workgroup takes cpw consecutive candidate workgroups' worth of rows ("chunks", 2^cand_shift
// rows each) of one unit, finds b0 once, and writes each chunk's candidates, count and granule
// counts as its own. Several chunks per workgroup cut the histogram reads and block scans where
// the grid is large; one keeps the launch short where it is not. Tiles are software-pipelined:
// the next tile's scores are loaded before the current one is counted.
template <int kCN>
__global__ __launch_bounds__(kCN) void cand_kernel(SelectArgs a, int cpw) {
  constexpr int kCW = kCN / 64;           // waves
  constexpr int kCPer = kCTile / kCN;     // rows per thread per tile
  static_assert(kCPer * kCN == kCTile, "a tile is one chunk");
  constexpr int kGpwMax = 1 << (kCandRowsShift - kGranMinShift);  // granules per chunk, at most
  __shared__ uint32_t sh[2 * kCW];
  __shared__ uint32_t found[2];
  __shared__ uint32_t lgt[2][kGpwMax];  // keys above b0 per granule, by chunk parity
  TRI_STAMP(g_stamps_select, stamps::kCand, 0);
  const int WPU = a.lay.cand_wgs, gshift = a.lay.gran_shift, cshift = a.lay.cand_shift;
  const int wgpu = (WPU + cpw - 1) / cpw;  // workgroups per unit
  const int bid = dev::xcd_block(blockIdx.x, gridDim.x);
  const int u = bid / wgpu, cg = bid - u * wgpu;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const dev::UnitRows ur = dev::unit_rows(a.row_off, u, a.total_rows, a.max_rows);
  const uint32_t n = (uint32_t)ur.n;
  const uint32_t m = (uint32_t)a.B < n ? (uint32_t)a.B : n;
  if (m == n || m == 0) return;  // every row kept, or none: no threshold
  const uint32_t nch = ((n - 1) >> cshift) + 1;  // chunks of this unit
  const uint32_t c0 = (uint32_t)cg * (uint32_t)cpw;
  if (c0 >= nch) return;
  const uint32_t c1 = nch - c0 > (uint32_t)cpw ? c0 + (uint32_t)cpw : nch;
  const uint32_t R0 = c0 << cshift, R1 = (c1 << cshift) < n ? (c1 << cshift) : n;  // this workgroup's rows
  const WsPtrs w = ws_ptrs(a);
  const float* s = a.scores + ur.beg;
  const uint32_t gpw = 1u << (cshift - gshift);  // granules per chunk (<= kGpwMax)

  // loads first: kBPT histogram bins per thread (4095 - kBPT*t downwards) and the first tile
  constexpr int kBPT = kHistBins / kCN;  // histogram bins per thread
  uint32_t hb[kBPT];
  {
    const uint4* gh4 = reinterpret_cast<const uint4*>(w.hist + (size_t)u * kHistBins);
#pragma unroll
    for (int q = 0; q < kBPT / 4; ++q) {
      const uint4 h = gh4[(kHistBins / 4) - 1 - (kBPT / 4) * threadIdx.x - q];
      hb[4 * q] = h.w; hb[4 * q + 1] = h.z; hb[4 * q + 2] = h.y; hb[4 * q + 3] = h.x;
    }
  }
  uint32_t k[kCPer];
  load_cand_tile<kCN, kCPer>(s, R1, R0, k);
  if (threadIdx.x < 2 * kGpwMax) lgt[threadIdx.x / kGpwMax][threadIdx.x % kGpwMax] = 0u;

  uint32_t above0;
  const uint32_t b0 = block_find<kCN, kBPT>(hb, kHistBins, m, sh, found, &above0);  // (synchronises)

  uint32_t c = c0, par = 0;
  uint32_t r0 = R0, r1 = R1 - R0 > (1u << cshift) ? R0 + (1u << cshift) : R1;  // the current chunk
  uint32_t* cout = w.cand + (((size_t)u * WPU + c) << cshift);
  uint32_t cbase = 0;
  for (uint32_t t0 = R0; t0 < R1; t0 += kCTile) {
    uint32_t kn[kCPer] = {};
    if (t0 + kCTile < R1) load_cand_tile<kCN, kCPer>(s, R1, t0 + kCTile, kn);
    uint32_t ncl = 0;
#pragma unroll
    for (int j = 0; j < kCPer; ++j) {
      const uint32_t row0 = t0 + j * kCN + wave * 64;  // a wave's 64 rows: one granule
      const bool in = row0 + lane < r1;
      const uint32_t d = k[j] >> kHistShift;
      const uint64_t mg = __ballot(in && d > b0);
      if (lane == 0 && mg) atomicAdd(&lgt[par][(row0 - r0) >> gshift], popc64(mg));
      ncl += (in && d == b0) ? 1u : 0u;
    }
    uint32_t ctot;
    uint32_t p = cbase + dev::block_excl_scan_dpp<kCN>(ncl, sh, &ctot);
    if (ncl) {
#pragma unroll
      for (int j = 0; j < kCPer; ++j) {
        const uint32_t r = t0 + j * kCN + threadIdx.x;
        if (r < r1 && (k[j] >> kHistShift) == b0) cout[p++] = ((k[j] & 0xFFFFFu) << 12) | (r >> gshift);
      }
    }
    cbase += ctot;
    if (t0 + kCTile >= r1) {  // the chunk is done: its granule counts and candidate count
      __syncthreads();
      if (threadIdx.x < gpw) {
        const uint32_t g = (r0 >> gshift) + threadIdx.x;
        if (g < (uint32_t)a.lay.grans) w.gran_gt[(size_t)u * a.lay.grans + g] = lgt[par][threadIdx.x];
        lgt[par][threadIdx.x] = 0u;  // for chunk c + 2, which counts after the next chunk's barrier
      }
      if (threadIdx.x == 0) w.wg_cnt[(size_t)u * WPU + c] = cbase;
      ++c;
      par ^= 1u;
      r0 = r1;
      r1 = R1 - r0 > (1u << cshift) ? r0 + (1u << cshift) : R1;
      cout += (size_t)1 << cshift;
      cbase = 0;
    }
#pragma unroll
    for (int j = 0; j < kCPer; ++j) k[j] = kn[j];
  }
  if (threadIdx.x == 0 && c0 == 0) { w.state[u].b0 = b0; w.state[u].above0 = above0; }
  TRI_STAMP(g_stamps_select, stamps::kCand, 1);
}

// ---------------------------------------------------------------------------------------------
// resolve
// ---------------------------------------------------------------------------------------------

constexpr int kRN = 1024;
constexpr int kRW = kRN / 64;
constexpr int kRPer = kMaxGran / kRN;  // granules (and candidate workgroups) per thread
constexpr int kPre = 8;                // candidates each thread loads with the first loads
constexpr int kTieList = 1024;         // candidates whose top 22 bits are T's, kept in a list
static_assert(kRPer * kRN == kMaxGran, "granules per thread");
static_assert(kPre * (kRN / 8) <= (1 << kCandRowsShift), "preload stays inside a workgroup region");

struct ResShared {
  uint32_t sh[4 * kRW];
  uint32_t found[2];
  uint32_t nlist;
  uint32_t cand[kCandCap];         // packed candidates: low 20 key bits << 12 | granule
  uint32_t rhist[2][1024];         // radix bins of digits 2 and 3
  uint32_t wgoff[kMaxGran + 1];    // first candidate of each candidate workgroup
  uint32_t cnt[kMaxGran];          // per granule: candidates above T (low 16 bits), equal (high 16)
  uint32_t list[kTieList];         // candidates sharing T's digits 1 and 2
};

// Digit-3 bin, granule and "above" tests of a packed candidate: bits 31..22 are digit 2, bits
// 21..12 digit 3, bits 11..0 the granule.
__device__ __forceinline__ uint32_t cand_d2(uint32_t p) { return p >> 22; }
__device__ __forceinline__ uint32_t cand_d3(uint32_t p) { return (p >> 12) & 1023u; }

// One workgroup per unit: digits 2 and 3 of T among the candidates, then per-granule output
// offsets and counts of ties before each granule. Leaves the unit's histogram at zero.
// The candidates are loaded with the first loads (each of the unit's candidate workgroups gets
// 1024/nwg threads that load kPre of its candidates each; more are fetched afterwards), placed
// in LDS behind their workgroup's prefix and counted by digit 2 as they are placed; the digit-3
// pass also counts, per granule, the candidates whose digit 2 is above T's.
__global__ __launch_bounds__(kRN) void resolve_kernel(SelectArgs a) {
  __shared__ ResShared L;
  const int u = blockIdx.x;
  const int NG = a.lay.grans, WPU = a.lay.cand_wgs, gshift = a.lay.gran_shift, cshift = a.lay.cand_shift;
  const WsPtrs w = ws_ptrs(a);
  const dev::UnitRows ur = dev::unit_rows(a.row_off, u, a.total_rows, a.max_rows);
  const uint32_t n = (uint32_t)ur.n;
  const uint32_t m = (uint32_t)a.B < n ? (uint32_t)a.B : n;
  UnitState* st = w.state + u;

  // the unit's histogram back to rest (the candidate kernel has read it)
  static_assert(kHistBins == 4 * kRN, "one uint4 of bins per thread");
  reinterpret_cast<uint4*>(w.hist + (size_t)u * kHistBins)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  if (m == n || m == 0) {
    if (threadIdx.x == 0) { st->mode = m == 0 ? kModeNone : kModeAll; st->m = m; }
    return;
  }
  const uint32_t b0 = st->b0, above0 = st->above0;
  const uint32_t ngu = ((n - 1) >> gshift) + 1;  // granules of this unit
  const uint32_t nwg = ((n - 1) >> cshift) + 1;  // candidate workgroups of this unit
  const uint32_t* cin = w.cand + (((size_t)u * WPU) << cshift);

  // loads: this thread's granules and candidate workgroups 4t..4t+3, and its share of the
  // candidates of workgroup cw = t / tpw (entries ci + k*tpw, inside the region whatever the count)
  uint32_t lg = 0;
  while ((1u << lg) < nwg) ++lg;
  const uint32_t tpw = lg > 10 ? 0u : ((kRN >> lg) < kRN / 8 ? (kRN >> lg) : kRN / 8);  // threads per workgroup
  const uint32_t cw = tpw ? threadIdx.x / tpw : 0u, ci = tpw ? threadIdx.x % tpw : 0u;
  const bool pre_ok = tpw != 0 && cw < nwg;
  uint32_t pv[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) pv[k] = pre_ok ? cin[((size_t)cw << cshift) + ci + k * tpw] : 0u;
  uint32_t ggt[kRPer], wc[kRPer];
#pragma unroll
  for (int q = 0; q < kRPer; ++q) {
    const uint32_t i = kRPer * threadIdx.x + q;
    ggt[q] = i < ngu ? w.gran_gt[(size_t)u * NG + i] : 0u;
    wc[q] = i < nwg ? w.wg_cnt[(size_t)u * WPU + i] : 0u;
  }
  L.rhist[0][threadIdx.x] = 0u;
  L.rhist[1][threadIdx.x] = 0u;
#pragma unroll
  for (int q = 0; q < kRPer; ++q) L.cnt[kRPer * threadIdx.x + q] = 0u;
  if (threadIdx.x == 0) L.nlist = 0u;

  uint32_t nc;
  uint32_t wex = dev::block_excl_scan_dpp<kRN>(wc[0] + wc[1] + wc[2] + wc[3], L.sh, &nc);
  const bool in_lds = nc <= (uint32_t)kCandCap;
#pragma unroll
  for (int q = 0; q < kRPer; ++q) {
    const uint32_t i = kRPer * threadIdx.x + q;
    if (i < nwg) L.wgoff[i] = wex;
    wex += wc[q];
  }
  if (threadIdx.x == 0) L.wgoff[nwg] = nc;
  __syncthreads();

  uint32_t r = m - above0;
  uint32_t pre, T, need;
  if (in_lds) {
    // ---- place the candidates, counting digit 2
    if (pre_ok) {
      const uint32_t base = L.wgoff[cw], cnt_w = L.wgoff[cw + 1] - base;
#pragma unroll
      for (int k = 0; k < kPre; ++k) {
        const uint32_t i = ci + k * tpw;
        if (i < cnt_w) {
          L.cand[base + i] = pv[k];
          atomicAdd(&L.rhist[0][cand_d2(pv[k])], 1u);
        }
      }
    }
    // candidates past the preloaded share: the same threads go on; with more than 1024
    // candidate workgroups, one thread per workgroup takes all of them
    if (tpw) {
      if (cw < nwg) {
        const uint32_t base = L.wgoff[cw], cnt_w = L.wgoff[cw + 1] - base;
        for (uint32_t i = tpw * kPre + ci; i < cnt_w; i += tpw) {
          const uint32_t v = cin[((size_t)cw << cshift) + i];
          L.cand[base + i] = v;
          atomicAdd(&L.rhist[0][cand_d2(v)], 1u);
        }
      }
    } else {
      for (uint32_t c = threadIdx.x; c < nwg; c += kRN) {
        const uint32_t base = L.wgoff[c], cnt_w = L.wgoff[c + 1] - base;
        for (uint32_t i = 0; i < cnt_w; ++i) {
          const uint32_t v = cin[((size_t)c << cshift) + i];
          L.cand[base + i] = v;
          atomicAdd(&L.rhist[0][cand_d2(v)], 1u);
        }
      }
    }
    __syncthreads();
    // ---- digit 2
    uint32_t above;
    {
      const uint32_t v[1] = {L.rhist[0][1023 - threadIdx.x]};
      const uint32_t d2 = block_find<kRN, 1>(v, 1024, r, L.sh, L.found, &above);
      r -= above;
      pre = (b0 << 10) | d2;
    }
    // ---- digit 3 among the candidates with T's digit 2; the others above it are counted per
    // granule now
    const uint32_t d2 = pre & 1023u;
    for (uint32_t j = threadIdx.x; j < nc; j += kRN) {
      const uint32_t p = L.cand[j];
      const uint32_t dj = cand_d2(p);
      if (dj > d2) {
        atomicAdd(&L.cnt[p & 0xFFFu], 1u);
      } else if (dj == d2) {
        atomicAdd(&L.rhist[1][cand_d3(p)], 1u);
        const uint32_t slot = atomicAdd(&L.nlist, 1u);
        if (slot < (uint32_t)kTieList) L.list[slot] = p;
      }
    }
    __syncthreads();
    {
      const uint32_t v[1] = {L.rhist[1][1023 - threadIdx.x]};
      const uint32_t d3 = block_find<kRN, 1>(v, 1024, r, L.sh, L.found, &above);
      r -= above;
      pre = (pre << 10) | d3;
    }
    T = pre;
    need = r;
    // ---- the candidates with T's digit 2: above T or equal to it, per granule
    const uint32_t d3 = T & 1023u;
    const uint32_t nl = L.nlist;
    if (nl <= (uint32_t)kTieList) {
      for (uint32_t j = threadIdx.x; j < nl; j += kRN) {
        const uint32_t p = L.list[j];
        if (cand_d3(p) >= d3) atomicAdd(&L.cnt[p & 0xFFFu], cand_d3(p) > d3 ? 1u : 0x10000u);
      }
    } else {
      for (uint32_t j = threadIdx.x; j < nc; j += kRN) {
        const uint32_t p = L.cand[j];
        if (cand_d2(p) == d2 && cand_d3(p) >= d3) atomicAdd(&L.cnt[p & 0xFFFu], cand_d3(p) > d3 ? 1u : 0x10000u);
      }
    }
  } else {
    // ---- more candidates than LDS holds: three passes over the candidate words in the
    // workspace (digit 2, digit 3, then the per-granule counts), each thread over the same share
    // as above, the preloaded first ones from registers
    auto each_cand = [&](auto&& f) {
      if (tpw) {
        if (cw < nwg) {
          const uint32_t cnt_w = L.wgoff[cw + 1] - L.wgoff[cw];
#pragma unroll
          for (int k = 0; k < kPre; ++k)
            if (ci + k * tpw < cnt_w) f(pv[k]);
          for (uint32_t i = tpw * kPre + ci; i < cnt_w; i += tpw) f(cin[((size_t)cw << cshift) + i]);
        }
      } else {
        for (uint32_t c = threadIdx.x; c < nwg; c += kRN) {
          const uint32_t cnt_w = L.wgoff[c + 1] - L.wgoff[c];
          for (uint32_t i = 0; i < cnt_w; ++i) f(cin[((size_t)c << cshift) + i]);
        }
      }
    };
    each_cand([&](uint32_t p) { atomicAdd(&L.rhist[0][cand_d2(p)], 1u); });
    __syncthreads();
    uint32_t above;
    const uint32_t v2[1] = {L.rhist[0][1023 - threadIdx.x]};
    const uint32_t d2 = block_find<kRN, 1>(v2, 1024, r, L.sh, L.found, &above);
    r -= above;
    each_cand([&](uint32_t p) {
      if (cand_d2(p) == d2) atomicAdd(&L.rhist[1][cand_d3(p)], 1u);
    });
    __syncthreads();
    const uint32_t v3[1] = {L.rhist[1][1023 - threadIdx.x]};
    const uint32_t d3 = block_find<kRN, 1>(v3, 1024, r, L.sh, L.found, &above);
    r -= above;
    T = (((b0 << 10) | d2) << 10) | d3;
    need = r;
    const uint32_t lowT = T & 0xFFFFFu;
    each_cand([&](uint32_t p) {
      const uint32_t lk = p >> 12;
      if (lk >= lowT) atomicAdd(&L.cnt[p & 0xFFFu], lk > lowT ? 1u : 0x10000u);
    });
  }
  __syncthreads();

  // ---- per-granule output offsets: rows above T before the granule plus the ties kept before
  // it, min(ties before the granule, need) (ties are kept lowest rows first)
  uint32_t e[kRPer], kg[kRPer], se = 0, sg = 0;
#pragma unroll
  for (int q = 0; q < kRPer; ++q) {
    const uint32_t i = kRPer * threadIdx.x + q;
    const uint32_t cc = i < ngu ? L.cnt[i] : 0u;
    e[q] = cc >> 16;
    kg[q] = ggt[q] + (cc & 0xFFFFu);
    se += e[q];
    sg += kg[q];
  }
  uint32_t E, G, tE, tG;
  dev::block_excl_scan2_dpp<kRN>(se, sg, L.sh, &E, &G, &tE, &tG);
#pragma unroll
  for (int q = 0; q < kRPer; ++q) {
    const uint32_t i = kRPer * threadIdx.x + q;
    if (i < ngu) {
      w.gran_off[(size_t)u * NG + i] = G + (E < need ? E : need);
      w.gran_eq[(size_t)u * NG + i] = E;
    }
    G += kg[q];
    E += e[q];
  }
  if (threadIdx.x == 0) { st->T = T; st->need = need; st->mode = kModeThreshold; st->m = m; }
}

// ---------------------------------------------------------------------------------------------
// finish: resolve and emit in one kernel (units of at most kFinishMaxRows rows)
// ---------------------------------------------------------------------------------------------
//
// One workgroup of 1024 threads per 64 output slots of a unit. Every workgroup of a unit
// resolves T itself from the unit's candidates (a few thousand words, read by all of them, with
// no communication between workgroups) and turns the per-granule counts (keys above the top
// digit from the candidate kernel, candidates above or equal to T) into each granule's first
// output slot. The granules whose kept rows fall into its 64 slots (at most 64 of them) are then
// read again, one wave each, to place every kept row at its slot; the workgroup writes those
// slots' indices and positions and gathers their K/V rows. Work per workgroup is bounded by its
// slots, so kept rows that crowd into a few granules (high scores at nearby positions) are still
// copied by many workgroups.
// With more than kCandCap candidates (thousands of keys sharing T's top 12 bits), digits 2 and 3
// and the per-granule counts come from the candidate words in the workspace, streamed in three
// passes.

constexpr int64_t kFinishMaxRows = int64_t(1) << 18;  // 64-row granules, at most 256 candidate workgroups
constexpr int kFinSlots = 64;                         // output slots per workgroup
// Every finish workgroup resolves its unit's threshold again; beyond about 4096 finish
// workgroups in all the repeated resolves cost more than the separate resolve kernel and its
// boundary. Measured crossovers: units of 32768 rows with B = 2048 (32 finish workgroups per
// unit): equal at 160 units, 2% slower at 200; units of 65536 rows with B = 4096: 2.5% slower at
// 96 units. 2048 units of 132096 rows with B = 12000 took 33.1 ms per pass with finish_kernel
// and 17.1 ms with candidates, resolve and emit.
constexpr int64_t kFinishMaxWorkgroups = 4096;
constexpr int kFinMaxCandWgs = kFinishMaxRows >> kCandRowsShift;

struct FinShared {
  uint32_t sh[4 * kRW];
  uint32_t found[2];
  uint32_t nsel;
  uint32_t cand[kCandCap];              // packed candidates: low 20 key bits << 12 | granule
  uint32_t rhist[2][1024];              // radix bins of digits 2 and 3
  uint32_t wgoff[kFinMaxCandWgs + 1];   // first candidate of each candidate workgroup
  uint32_t cnt[kMaxGran];               // per granule: candidates above T (low 16 bits), equal (high 16)
  uint32_t gsel[kFinSlots];             // granules with kept rows in this workgroup's slots,
  uint32_t goff[kFinSlots];             //   their first kept row's slot
  uint32_t geq[kFinSlots];              //   and the keys equal to T before them
  uint32_t krow[kFinSlots];             // row of each of this workgroup's slots
};

// Copy of a workgroup's kept K and V rows to consecutive output rows: piece q (16 bytes) is part
// q % CPR of output row q / CPR, whose source row (from the unit's first row) is krow[q / CPR],
// clamped to lim. Every load of a step is issued before its stores.
template <int CPR>
struct PieceCopy {
  static constexpr int kShift = CPR == 8 ? 3 : CPR == 16 ? 4 : CPR == 32 ? 5 : 6;
  static constexpr uint32_t kRowBytes = CPR * 16;
  const char* __restrict__ srcK;
  const char* __restrict__ srcV;
  char* __restrict__ dstK;
  char* __restrict__ dstV;
  const uint32_t* krow;  // LDS
  uint32_t per, lim;     // pieces per tensor; last row of the unit

  __device__ __forceinline__ size_t src(uint32_t q) const {
    const uint32_t kr = krow[q >> kShift];
    return (size_t)(kr < lim ? kr : lim) * kRowBytes + (q & (CPR - 1)) * 16u;
  }
  __device__ __forceinline__ uint4 ld(const char* p, size_t o) const { return *reinterpret_cast<const uint4*>(p + o); }
  __device__ __forceinline__ void st(char* p, uint32_t q, const uint4& v) const {
    *reinterpret_cast<uint4*>(p + q * 16u) = v;  // output row q / CPR, part q % CPR
  }
  // per <= 1024: one piece of K and one of V per thread
  __device__ __forceinline__ void run1() const {
    const uint32_t q = threadIdx.x;
    const size_t o = src(q < per ? q : per - 1);
    const uint4 k = ld(srcK, o), v = ld(srcV, o);
    if (q < per) { st(dstK, q, k); st(dstV, q, v); }
  }
  // any count: two pieces of each per thread in flight
  __device__ __forceinline__ void run2() const {
    for (uint32_t q0 = 0; q0 < per; q0 += 2 * kRN) {  // uniform trip count
      const uint32_t qa = q0 + threadIdx.x, qb = qa + kRN;
      const size_t oa = src(qa < per ? qa : per - 1), ob = src(qb < per ? qb : per - 1);
      const uint4 ka = ld(srcK, oa), va = ld(srcV, oa), kb = ld(srcK, ob), vb = ld(srcV, ob);
      if (qa < per) { st(dstK, qa, ka); st(dstV, qa, va); }
      if (qb < per) { st(dstK, qb, kb); st(dstV, qb, vb); }
    }
  }
};

template <int CPR>  // 16-byte pieces per K/V row; 0: no gather
__global__ __launch_bounds__(kRN) void finish_kernel(SelectArgs a, int wpu) {
  __shared__ FinShared L;
  TRI_STAMP(g_stamps_select, stamps::kFinish, stamps::kFinStart);
  const int NG = a.lay.grans;
  const int bid = dev::xcd_block(blockIdx.x, gridDim.x);
  const int u = bid / wpu, c = bid - u * wpu;
  const uint32_t t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const WsPtrs w = ws_ptrs(a);
  // First loads, all issued before the unit's length is known (which they would otherwise wait
  // for): the unit's state, a share of the candidates of candidate workgroup cw = t / tpw (entries
  // ci + k*tpw), the candidate counts and the per-granule counts above the top digit, each for a
  // unit of max_rows rows and inside the unit's regions of the workspace; what lies past the
  // unit's own length is masked below.
  const uint32_t mr1 = a.max_rows > 0 ? (uint32_t)(a.max_rows - 1) : 0u;  // (the regions hold one group at least)
  const uint32_t nwg_max = (mr1 >> kCandRowsShift) + 1;  // <= kFinMaxCandWgs
  const uint32_t ngu_max = (mr1 >> kGranMinShift) + 1;   // <= kMaxGran
  const UnitState* st = w.state + u;
  const uint32_t b0 = st->b0, above0 = st->above0;
  const uint32_t* cin = w.cand + (((size_t)u * a.lay.cand_wgs) << kCandRowsShift);
  uint32_t lg = 0;
  while ((1u << lg) < nwg_max) ++lg;
  const uint32_t tpw = (kRN >> lg) < kRN / 8 ? (kRN >> lg) : kRN / 8;  // threads per workgroup (>= 4)
  const uint32_t cw = t / tpw, ci = t % tpw;
  uint32_t pv[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) pv[k] = cw < nwg_max ? cin[((size_t)cw << kCandRowsShift) + ci + k * tpw] : 0u;
  uint32_t wc = t < nwg_max ? w.wg_cnt[(size_t)u * a.lay.cand_wgs + t] : 0u;
  uint32_t ggt[kRPer];
#pragma unroll
  for (int q = 0; q < kRPer; ++q) {
    const uint32_t i = kRPer * t + q;
    ggt[q] = i < ngu_max ? w.gran_gt[(size_t)u * NG + i] : 0u;
  }
  const dev::UnitRows ur = dev::unit_rows(a.row_off, u, a.total_rows, a.max_rows);
  const uint32_t n = (uint32_t)ur.n;
  const uint32_t m = (uint32_t)a.B < n ? (uint32_t)a.B : n;
  int32_t* out = a.kept_idx + (int64_t)u * a.B;
  if (c == 0) {  // the unit's histogram back to rest (the candidate kernel has read it), padding, count
    static_assert(kHistBins == 4 * kRN, "one uint4 of bins per thread");
    reinterpret_cast<uint4*>(w.hist + (size_t)u * kHistBins)[t] = make_uint4(0u, 0u, 0u, 0u);
    for (uint32_t j = m + t; j < (uint32_t)a.B; j += kRN) out[j] = -1;
    if (t == 0) a.kept_cnt[u] = (int32_t)m;
  }
  const uint32_t s0 = (uint32_t)c * kFinSlots;
  if (s0 >= m) return;
  const uint32_t ns = m - s0 < (uint32_t)kFinSlots ? m - s0 : (uint32_t)kFinSlots;  // this workgroup's slots
  const float* s = a.scores + ur.beg;

  if (m == n) {  // every row kept: slot = row
    if (t < ns) L.krow[t] = s0 + t;
    __syncthreads();
  } else {
    const uint32_t nwg = ((n - 1) >> kCandRowsShift) + 1;  // candidate workgroups of this unit (<= nwg_max)
    const uint32_t ngu = ((n - 1) >> kGranMinShift) + 1;   // granules of this unit (<= ngu_max)
    const bool pre_ok = cw < nwg;
    if (t >= nwg) wc = 0u;
#pragma unroll
    for (int q = 0; q < kRPer; ++q) {
      const uint32_t i = kRPer * t + q;
      if (i >= ngu) ggt[q] = 0u;
      L.cnt[i] = 0u;
    }
    L.rhist[0][t] = 0u;
    L.rhist[1][t] = 0u;
    if (t == 0) L.nsel = 0u;
    uint32_t nc;
    const uint32_t wex = dev::block_excl_scan_dpp<kRN>(wc, L.sh, &nc);
    if (t < nwg) L.wgoff[t] = wex;
    if (t == 0) L.wgoff[nwg] = nc;
    __syncthreads();
    TRI_STAMP(g_stamps_select, stamps::kFinish, stamps::kFinLoads);

    uint32_t r = m - above0, above, T, need;
    if (nc <= (uint32_t)kCandCap) {
      // ---- place the candidates, counting digit 2
      if (pre_ok) {
        const uint32_t base = L.wgoff[cw], cnt_w = L.wgoff[cw + 1] - base;
#pragma unroll
        for (int k = 0; k < kPre; ++k) {
          const uint32_t i = ci + k * tpw;
          if (i < cnt_w) {
            L.cand[base + i] = pv[k];
            atomicAdd(&L.rhist[0][cand_d2(pv[k])], 1u);
          }
        }
        for (uint32_t i = tpw * kPre + ci; i < cnt_w; i += tpw) {
          const uint32_t v = cin[((size_t)cw << kCandRowsShift) + i];
          L.cand[base + i] = v;
          atomicAdd(&L.rhist[0][cand_d2(v)], 1u);
        }
      }
      __syncthreads();
      const uint32_t v2[1] = {L.rhist[0][1023 - t]};
      const uint32_t d2 = block_find<kRN, 1>(v2, 1024, r, L.sh, L.found, &above);
      r -= above;
      for (uint32_t j = t; j < nc; j += kRN) {
        const uint32_t p = L.cand[j];
        if (cand_d2(p) == d2) atomicAdd(&L.rhist[1][cand_d3(p)], 1u);
      }
      __syncthreads();
      const uint32_t v3[1] = {L.rhist[1][1023 - t]};
      const uint32_t d3 = block_find<kRN, 1>(v3, 1024, r, L.sh, L.found, &above);
      T = (((b0 << 10) | d2) << 10) | d3;
      need = r - above;
      // candidates above T and equal to it, per granule
      const uint32_t lowT = T & 0xFFFFFu;
      for (uint32_t j = t; j < nc; j += kRN) {
        const uint32_t p = L.cand[j], lk = p >> 12;
        if (lk >= lowT) atomicAdd(&L.cnt[p & 0xFFFu], lk > lowT ? 1u : 0x10000u);
      }
    } else {
      // ---- more candidates than LDS holds: three passes over the candidate words in the
      // workspace (digit 2, digit 3, then the per-granule counts), each thread over its share of
      // one candidate workgroup's words, the preloaded first ones from registers. (Re-reading
      // the unit's scores instead cost every one of the unit's workgroups a pass over all of
      // them: 103 us against 13 us for a pass over 4 units of 132096 rows.)
      auto each_cand = [&](auto&& f) {
        if (!pre_ok) return;
        const uint32_t cnt_w = L.wgoff[cw + 1] - L.wgoff[cw];
#pragma unroll
        for (int k = 0; k < kPre; ++k)
          if (ci + k * tpw < cnt_w) f(pv[k]);
        for (uint32_t i = tpw * kPre + ci; i < cnt_w; i += tpw) f(cin[((size_t)cw << kCandRowsShift) + i]);
      };
      each_cand([&](uint32_t p) { atomicAdd(&L.rhist[0][cand_d2(p)], 1u); });
      __syncthreads();
      const uint32_t v2[1] = {L.rhist[0][1023 - t]};
      const uint32_t d2 = block_find<kRN, 1>(v2, 1024, r, L.sh, L.found, &above);
      r -= above;
      each_cand([&](uint32_t p) {
        if (cand_d2(p) == d2) atomicAdd(&L.rhist[1][cand_d3(p)], 1u);
      });
      __syncthreads();
      const uint32_t v3[1] = {L.rhist[1][1023 - t]};
      const uint32_t d3 = block_find<kRN, 1>(v3, 1024, r, L.sh, L.found, &above);
      T = (((b0 << 10) | d2) << 10) | d3;
      need = r - above;
      const uint32_t lowT = T & 0xFFFFFu;
      each_cand([&](uint32_t p) {
        const uint32_t lk = p >> 12;
        if (lk >= lowT) atomicAdd(&L.cnt[p & 0xFFFu], lk > lowT ? 1u : 0x10000u);
      });
    }
    __syncthreads();
    TRI_STAMP(g_stamps_select, stamps::kFinish, stamps::kFinResolved);

    // ---- each granule's first slot; list the granules with kept rows in [s0, s0 + ns)
    uint32_t kgt[kRPer], keq[kRPer], sg = 0, se = 0;
#pragma unroll
    for (int q = 0; q < kRPer; ++q) {
      const uint32_t cc = L.cnt[kRPer * t + q];
      kgt[q] = ggt[q] + (cc & 0xFFFFu);
      keq[q] = cc >> 16;
      sg += kgt[q];
      se += keq[q];
    }
    uint32_t G, E, tg, te;
    dev::block_excl_scan2_dpp<kRN>(sg, se, L.sh, &G, &E, &tg, &te);
#pragma unroll
    for (int q = 0; q < kRPer; ++q) {
      const uint32_t first = G + (E < need ? E : need);
      const uint32_t E1 = E + keq[q];
      const uint32_t end = G + kgt[q] + (E1 < need ? E1 : need);
      if (end > first && first < s0 + ns && end > s0) {
        const uint32_t i = atomicAdd(&L.nsel, 1u);
        if (i < (uint32_t)kFinSlots) {  // always, with a consistent workspace
          L.gsel[i] = kRPer * t + q;
          L.goff[i] = first;
          L.geq[i] = E;
        }
      }
      G += kgt[q];
      E = E1;
    }
    __syncthreads();
    TRI_STAMP(g_stamps_select, stamps::kFinish, stamps::kFinListed);

    // ---- the listed granules' rows, one wave per granule: every kept row to its slot
    const uint32_t nsel = L.nsel < (uint32_t)kFinSlots ? L.nsel : (uint32_t)kFinSlots;
    constexpr int kGW = kFinSlots / kRW;  // granules per wave, at most
    uint32_t kk[kGW];
#pragma unroll
    for (int i = 0; i < kGW; ++i) {
      const uint32_t j = (uint32_t)(i * kRW + wave);
      const uint32_t row = j < nsel ? (L.gsel[j] << kGranMinShift) + lane : 0u;
      kk[i] = order_key(load_at(s, row < n ? row : n - 1));
    }
#pragma unroll
    for (int i = 0; i < kGW; ++i) {
      const uint32_t j = (uint32_t)(i * kRW + wave);
      if (j >= nsel) break;  // uniform
      const uint32_t row = (L.gsel[j] << kGranMinShift) + lane;
      const bool in = row < n;
      const bool gt = in && kk[i] > T, eq = in && kk[i] == T;
      const bool keep = gt || (eq && L.geq[j] + lanes_below(__ballot(eq)) < need);
      const uint32_t slot = L.goff[j] + lanes_below(__ballot(keep));
      if (keep && slot >= s0 && slot < s0 + ns) L.krow[slot - s0] = row;
    }
    __syncthreads();
    TRI_STAMP(g_stamps_select, stamps::kFinish, stamps::kFinPlaced);
  }

  // ---- this workgroup's slots: indices, positions, K/V rows
  const uint32_t my_row = t < ns ? (L.krow[t] < n ? L.krow[t] : n - 1) : 0u;
  const int64_t obase = (int64_t)u * a.B + s0;
  if constexpr (CPR > 0) {
    constexpr int64_t RB = CPR * 16;
    const int32_t pos_v = a.pos_out ? a.pos[ur.beg + my_row] : 0;  // in range for every thread
    const PieceCopy<CPR> cp{static_cast<const char*>(a.K) + ur.beg * RB, static_cast<const char*>(a.V) + ur.beg * RB,
                            static_cast<char*>(a.K_out) + obase * RB, static_cast<char*>(a.V_out) + obase * RB,
                            L.krow, ns * CPR, n - 1};
    if (cp.per <= (uint32_t)kRN) cp.run1();
    else cp.run2();
    if (a.pos_out && t < ns) a.pos_out[obase + t] = pos_v;
  }
  if (t < ns) out[s0 + t] = (int32_t)my_row;
  TRI_STAMP(g_stamps_select, stamps::kFinish, stamps::kFinEnd);
}

template <int CPR>
hipError_t launch_finish(const SelectArgs& a, hipStream_t s) {
  const int64_t mm = a.B < a.max_rows ? a.B : a.max_rows;
  const int64_t wpu = mm > 0 ? (mm + kFinSlots - 1) / kFinSlots : 1;
  const int64_t grid = (int64_t)a.n_units * wpu;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(finish_kernel<CPR>, dim3((unsigned)grid), dim3(kRN), 0, s, a, (int)wpu);
  return hipSuccess;
}

// ---------------------------------------------------------------------------------------------
// emit (and gather)
// ---------------------------------------------------------------------------------------------

constexpr int kEN = 256;       // four waves, one granule each, no block-level synchronisation
constexpr int kEW = kEN / 64;

// Copy of one step's kept rows of one tensor (K or V). Addresses are a wave-uniform base (the
// step's first row, the step's first output slot) plus a 32-bit byte offset below 64 rows * row
// bytes.
template <int CPR>
struct RowCopy {
  static constexpr int kShift = CPR == 8 ? 3 : CPR == 16 ? 4 : CPR == 32 ? 5 : 6;
  static constexpr uint32_t kRowBytes = CPR * 16;
  const char* __restrict__ src;  // row t0 of the unit
  char* __restrict__ dst;        // output slot s0
  uint32_t rows;                 // lane j < kc: (j-th kept row) - t0
  uint32_t total, room;          // pieces (kc * CPR); output slots left

  // piece q of the kept rows (q clamped to total - 1): row j = q / CPR, 16-byte part q % CPR.
  // Call with every lane active (the row index comes from lane j).
  __device__ __forceinline__ uint4 load(uint32_t q) const {
    const uint32_t qc = q < total ? q : total - 1;
    const uint32_t rj = (uint32_t)__shfl((int)rows, (int)(qc >> kShift), 64);
    return *reinterpret_cast<const uint4*>(src + rj * kRowBytes + (qc & (CPR - 1)) * 16u);
  }
  __device__ __forceinline__ void store(uint32_t q, const uint4& v) const {
    if (q >= total || (q >> kShift) >= room) return;
    *reinterpret_cast<uint4*>(dst + q * 16u) = v;  // slot j = q / CPR, part q % CPR
  }
  // all pieces in batches of NB per lane: every load of a batch is issued before its stores
  template <int NB>
  __device__ __forceinline__ void run() const {
    const uint32_t lane = threadIdx.x & 63;
    for (uint32_t q0 = 0; q0 < total; q0 += NB * 64) {  // uniform trip count
      uint4 p[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) p[i] = load(q0 + i * 64 + lane);
#pragma unroll
      for (int i = 0; i < NB; ++i) store(q0 + i * 64 + lane, p[i]);
    }
  }
};

// With the gather, each granule has two waves that both scan it: the first writes the kept
// indices and positions and copies the K rows, the second copies the V rows.
template <int CPR>
constexpr int waves_per_granule() { return CPR > 0 ? 2 : 1; }

template <int CPR>  // 16-byte pieces per K/V row; 0: no gather
__global__ __launch_bounds__(kEN) void emit_kernel(SelectArgs a) {
  constexpr int WPG = waves_per_granule<CPR>();
  constexpr int GPB = kEW / WPG;  // granules per workgroup
  const int NG = a.lay.grans, gshift = a.lay.gran_shift;
  const int EPU = (NG + GPB - 1) / GPB;
  const int u = blockIdx.x / EPU, c = blockIdx.x - u * EPU;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const bool second = WPG == 2 && (wave & 1);  // the V wave of its granule
  const WsPtrs w = ws_ptrs(a);
  const dev::UnitRows ur = dev::unit_rows(a.row_off, u, a.total_rows, a.max_rows);
  const uint32_t n = (uint32_t)ur.n;
  const uint32_t g = (uint32_t)(c * GPB + wave / WPG);
  const uint32_t gc = g < (uint32_t)NG ? g : (uint32_t)NG - 1;
  const uint32_t i0 = g << gshift;
  const float* sc = a.scores + ur.beg;
  // everything this wave reads up front, unconditionally (in-bounds; unused in modes all/none)
  const UnitState* st = w.state + u;
  const uint32_t mode = st->mode, m = st->m, T = st->T, need = st->need;
  const uint32_t goff = w.gran_off[(size_t)u * NG + gc];
  const uint32_t geq = w.gran_eq[(size_t)u * NG + gc];
  const uint32_t r_first = i0 + lane;
  const float s_first = r_first < n ? load_at(sc, r_first) : 0.f;
  int32_t* out = a.kept_idx + (int64_t)u * a.B;
  if (c == 0 && wave == 0) {
    for (uint32_t j = m + lane; j < (uint32_t)a.B; j += 64) out[j] = -1;
    if (lane == 0) a.kept_cnt[u] = (int32_t)m;
  }
  if (g >= (uint32_t)NG || i0 >= n || mode == kModeNone) return;  // whole wave
  const uint32_t i1 = n - i0 > (1u << gshift) ? i0 + (1u << gshift) : n;
  const bool all = mode == kModeAll;
  const uint32_t off = all ? i0 : goff;
  const uint32_t E0 = all ? 0u : geq;
  const uint32_t ties0 = E0 < need ? E0 : need;  // ties kept before this granule
  const int64_t obase = (int64_t)u * a.B;

  uint32_t run_g = 0, run_e = E0;  // keys above T / ties before the current step
  for (uint32_t t0 = i0; t0 < i1; t0 += 64) {
    const uint32_t r = t0 + lane;
    const bool in = r < i1;
    bool keep;
    uint32_t s0;  // output slot of the step's first kept row
    if (all) {
      keep = in;
      s0 = t0;
    } else {
      const uint32_t k = order_key(t0 == i0 ? s_first : load_at(sc, in ? r : i1 - 1));
      const bool gt = in && k > T, eq = in && k == T;
      const uint64_t mg = __ballot(gt), me = __ballot(eq);
      keep = gt || (eq && run_e + lanes_below(me) < need);
      s0 = off + run_g + (run_e < need ? run_e : need) - ties0;
      run_g += popc64(mg);
      run_e += popc64(me);
    }
    const uint64_t mk = __ballot(keep);
    const uint32_t kc = popc64(mk);
    if (kc == 0) continue;
    // kept rows to lanes 0..kc-1 in row order (a permutation: the others fill lanes kc..63)
    const uint32_t dst = keep ? lanes_below(mk) : kc + lanes_below(~mk);
    const uint32_t rows = (uint32_t)__builtin_amdgcn_ds_permute((int)(dst << 2), (int)r);
    const uint32_t room = s0 < m ? m - s0 : 0u;  // slots left (all of them, with a consistent workspace)
    if (!second && lane < kc && lane < room) {
      out[s0 + lane] = (int32_t)rows;
      if (CPR > 0 && a.pos_out) a.pos_out[obase + s0 + lane] = a.pos[ur.beg + rows];
    }
    if constexpr (CPR > 0) {
      constexpr int64_t RB = CPR * 16;
      const RowCopy<CPR> cp{static_cast<const char*>(second ? a.V : a.K) + (ur.beg + t0) * RB,
                            static_cast<char*>(second ? a.V_out : a.K_out) + (obase + s0) * RB, rows - t0,
                            kc * CPR, room};
      // pieces per lane: kc * CPR / 64, at most CPR; batches of at most 8 keep the VGPRs (and
      // so the waves resident per SIMD) where a full batch of 16 would not pay for itself
      if (cp.total <= 4 * 64) cp.template run<4>();
      else cp.template run<8>();
    }
  }
}

template <int CPR>
hipError_t launch_emit(const SelectArgs& a, hipStream_t s) {
  constexpr int GPB = kEW / waves_per_granule<CPR>();
  const int64_t grid = (int64_t)a.n_units * ((a.lay.grans + GPB - 1) / GPB);
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(emit_kernel<CPR>, dim3((unsigned)grid), dim3(kEN), 0, s, a);
  return hipSuccess;
}

// ---------------------------------------------------------------------------------------------
// in-place pass: freed slots and the kept rows that fill them
// ---------------------------------------------------------------------------------------------
//
// After the select, unit u keeps m rows. In place, the kept rows must end up in the unit's first
// m slots. A kept row below m stays where it is; every slot below m whose row is dropped is
// freed, and the kept rows at or beyond m fill the freed slots: the highest such row the lowest
// free slot, the next highest the next, and so on. Only those rows move (at most
// min(m, N_u - m)), so a steady-state pass over a cache of B + chunk rows copies at most one
// chunk of rows instead of the B rows a full compaction would.
//
// mark_kernel: one wave per granule. With r's kept rank q(r) (kept rows before r):
//   freed slot s < m   is the (s - q(s))-th freed slot
//   kept row r >= m    is the (m - 1 - q(r))-th kept row counted from the last
// and the wave holding row m records moves = m - q(m), the number of either.
// move_kernel: the j-th freed slot receives the j-th kept row from the last (K, V, position);
// sources are at or beyond m and destinations below it, so no row is both read and written.

__global__ __launch_bounds__(kEN) void mark_kernel(SelectArgs a, uint32_t* hole, uint32_t* mover, uint32_t hcap) {
  const int NG = a.lay.grans, gshift = a.lay.gran_shift;
  const int EPU = (NG + kEW - 1) / kEW;
  const int u = blockIdx.x / EPU, c = blockIdx.x - u * EPU;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const WsPtrs w = ws_ptrs(a);
  const dev::UnitRows ur = dev::unit_rows(a.row_off, u, a.total_rows, a.max_rows);
  const uint32_t n = (uint32_t)ur.n;
  const uint32_t g = (uint32_t)(c * kEW + wave);
  const uint32_t gc = g < (uint32_t)NG ? g : (uint32_t)NG - 1;
  const uint32_t i0 = g << gshift;
  const float* sc = a.scores + ur.beg;
  UnitState* st = w.state + u;
  const uint32_t mode = st->mode, m = st->m, T = st->T, need = st->need;
  const uint32_t off = w.gran_off[(size_t)u * NG + gc];
  const uint32_t E0 = w.gran_eq[(size_t)u * NG + gc];
  const uint32_t r_first = i0 + lane;
  const float s_first = r_first < n ? load_at(sc, r_first) : 0.f;
  if (c == 0 && wave == 0 && lane == 0) {
    a.kept_cnt[u] = (int32_t)m;
    if (mode != kModeThreshold) st->moves = 0u;  // every row kept, or none: nothing moves
  }
  if (g >= (uint32_t)NG || i0 >= n || mode != kModeThreshold) return;  // whole wave
  const uint32_t i1 = n - i0 > (1u << gshift) ? i0 + (1u << gshift) : n;
  const uint32_t ties0 = E0 < need ? E0 : need;
  uint32_t* hl = hole + (size_t)u * hcap;
  uint32_t* ml = mover + (size_t)u * hcap;

  uint32_t run_g = 0, run_e = E0;
  for (uint32_t t0 = i0; t0 < i1; t0 += 64) {
    const uint32_t r = t0 + lane;
    const bool in = r < i1;
    const uint32_t k = order_key(t0 == i0 ? s_first : load_at(sc, in ? r : i1 - 1));
    const bool gt = in && k > T, eq = in && k == T;
    const uint64_t mg = __ballot(gt), me = __ballot(eq);
    const bool keep = gt || (eq && run_e + lanes_below(me) < need);
    const uint32_t s0 = off + run_g + (run_e < need ? run_e : need) - ties0;  // kept rank of the step's first kept row
    run_g += popc64(mg);
    run_e += popc64(me);
    const uint64_t mk = __ballot(keep);
    const uint32_t q = s0 + lanes_below(mk);  // kept rows before r
    if (in && r < m && !keep) {
      const uint32_t j = r - q;
      if (j < hcap) hl[j] = r;
    }
    if (in && r >= m && keep) {
      const uint32_t j = m - 1 - q;
      if (j < hcap) ml[j] = r;
    }
    if (t0 <= m && m - t0 < 64u && m < i1 && lane == 0) {  // the step holding row m (m < n here)
      const uint32_t below = m - t0;  // lanes of rows before m
      const uint64_t before = below ? (mk & (~0ull >> (64 - below))) : 0ull;
      st->moves = m - (s0 + popc64(before));
    }
  }
}

template <int CPR>
__global__ __launch_bounds__(256) void move_kernel(SelectArgs a, MoveArgs mv, int blocks_per_unit) {
  constexpr int ROWS = 256 / CPR;
  const int u = blockIdx.x / blocks_per_unit, b = blockIdx.x - u * blocks_per_unit;
  const WsPtrs w = ws_ptrs(a);
  const dev::UnitRows ur = dev::unit_rows(a.row_off, u, a.total_rows, a.max_rows);
  const UnitState* st = w.state + u;
  const uint32_t h = st->moves;
  const uint32_t j = (uint32_t)(b * ROWS) + threadIdx.x / CPR;
  const uint32_t part = threadIdx.x % CPR;
  if (j >= h || j >= (uint32_t)mv.hcap) return;
  const uint32_t dst = mv.hole[(size_t)u * mv.hcap + j];
  const uint32_t src = mv.mover[(size_t)u * mv.hcap + j];
  if (dst >= ur.n || src >= ur.n) return;  // only with an inconsistent workspace
  const int64_t sp = (ur.beg + src) * CPR + part, dp = (ur.beg + dst) * CPR + part;
  // every load before the stores (a load issued after a store waits for that store too); the
  // source rows (at or beyond m) and the destinations (below m) are disjoint
  const bool with_pos = part == 0 && mv.pos != nullptr;
  const uint4 kv = static_cast<const uint4*>(mv.K)[sp];
  const uint4 vv = static_cast<const uint4*>(mv.V)[sp];
  const int32_t pv = with_pos ? mv.pos[ur.beg + src] : 0;
  static_cast<uint4*>(mv.K)[dp] = kv;
  static_cast<uint4*>(mv.V)[dp] = vv;
  if (with_pos) mv.pos[ur.beg + dst] = pv;
}

template <int CPR>
hipError_t launch_move(const SelectArgs& a, const MoveArgs& mv, hipStream_t s) {
  constexpr int ROWS = 256 / CPR;
  const int64_t bpu = (mv.hcap + ROWS - 1) / ROWS;
  const int64_t grid = bpu * a.n_units;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(move_kernel<CPR>, dim3((unsigned)grid), dim3(256), 0, s, a, mv, (int)bpu);
  return hipSuccess;
}

// ---------------------------------------------------------------------------------------------
// units of at most 64k rows: the whole select in one workgroup per unit
// ---------------------------------------------------------------------------------------------
//
// topb_kernel holds a unit's order keys in registers (KPT per thread; element j of thread t is
// row j*1024 + t, so element j of wave w is the 64-row granule 16j + w) and runs the three radix
// digits there: bits 31..20 from the histogram, 19..10 and 9..0 by LDS histograms over the keys
// that share the digits found so far. Per-granule counts of keys above and equal to T, one
// block scan of both, and every kept row's output slot follows: kept rows before its granule plus
// kept lanes below it. It writes the kept indices (or, for the in-place pass, the freed-slot and
// mover lists and the move count) itself, so the pass needs no candidate, resolve or emit kernel;
// the K/V rows are then gathered by the compaction kernel.

constexpr int kTN = 1024;
constexpr int kTW = kTN / 64;
constexpr int64_t kTopbMaxRows = 64 * kTN;
// tri_select_topb and tri_prune_pass use it from this many units on. Measured against candidates
// + finish on units of 32768 keys, B = 2048 (pass time per call): 8 units 33.6 against 26.9 us,
// 16 units 48.3 against 42.3, 24 units 60.7 against 59.2, 32 units 74.4-75.8 against 73.4-77.1,
// 64 units 128.3 against 138.6, 128 units 243.1 against 274.2, 192 units 376.2 against 406.9.
// With B = 256 (4 finish workgroups per unit) candidates + finish stay ahead a little longer:
// 48 units 86.5 against 88.3 us, 64 units 111.8 against 112.4, 128 units 215.8 against 211.0; with
// B = 8192 the one-workgroup select is ahead from 48 units (156.2 against 163.5). So it also needs
// kTopbMinFinishGroups output groups of 64 slots in all.
constexpr int kTopbMinUnits = 48;
constexpr int64_t kTopbMinFinishGroups = 384;

struct TopbShared {
  uint32_t sh[4 * kTW];
  uint32_t found[2];
  uint32_t rhist[2][1024];  // radix bins of digits 2 and 3
  uint32_t gt[kTN];         // per granule: keys above T, then kept rows before the granule
  uint32_t eq[kTN];         // per granule: keys equal to T, then those before the granule
};

struct InplaceOut {
  uint32_t* hole;
  uint32_t* mover;
  uint32_t hcap;
};

template <int KPT, bool INPLACE>
__global__ __launch_bounds__(kTN) void topb_kernel(SelectArgs a, InplaceOut io) {
  static_assert(KPT * kTN <= kTopbMaxRows && KPT * (kTN / 64) <= kTN, "one granule per thread");
  __shared__ TopbShared L;
  const int u = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const WsPtrs w = ws_ptrs(a);
  const dev::UnitRows ur = dev::unit_rows(a.row_off, u, a.total_rows, a.max_rows);
  const uint32_t n = (uint32_t)ur.n;
  const uint32_t m = (uint32_t)a.B < n ? (uint32_t)a.B : n;
  uint4* hist4 = reinterpret_cast<uint4*>(w.hist + (size_t)u * kHistBins);
  int32_t* out = a.kept_idx ? a.kept_idx + (int64_t)u * a.B : nullptr;
  static_assert(kHistBins == 4 * kTN, "one uint4 of bins per thread");

  if (m == n || m == 0) {  // every row kept, or none: no threshold
    hist4[t] = make_uint4(0u, 0u, 0u, 0u);
    if (out)
      for (uint32_t j = t; j < (uint32_t)a.B; j += kTN) out[j] = j < m ? (int32_t)j : -1;
    if (t == 0) {
      a.kept_cnt[u] = (int32_t)m;
      if constexpr (INPLACE) w.state[u].moves = 0u;
    }
    return;
  }

  // loads: 4 histogram bins (4095-4t down to 4092-4t) and the keys
  const uint4 h = hist4[kTN - 1 - t];
  const float* s = a.scores + ur.beg;
  uint32_t k[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {  // unconditional (rows past the unit read its last row): all in flight
    const uint32_t row = (uint32_t)j * kTN + t;
    k[j] = order_key(load_at(s, row < n ? row : n - 1));
  }
  L.rhist[0][t] = 0u;
  L.rhist[1][t] = 0u;

  // digit 1 from the histogram, then the histogram back to rest
  uint32_t above;
  const uint32_t hv[4] = {h.w, h.z, h.y, h.x};
  const uint32_t b0 = block_find<kTN, 4>(hv, kHistBins, m, L.sh, L.found, &above);
  hist4[kTN - 1 - t] = make_uint4(0u, 0u, 0u, 0u);
  uint32_t r = m - above;
  // digit 2 among the keys with T's digit 1
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if ((uint32_t)j * kTN + t < n && (k[j] >> 20) == b0) atomicAdd(&L.rhist[0][(k[j] >> 10) & 1023u], 1u);
  __syncthreads();
  const uint32_t v2[1] = {L.rhist[0][1023 - t]};
  const uint32_t p2 = (b0 << 10) | block_find<kTN, 1>(v2, 1024, r, L.sh, L.found, &above);
  r -= above;
  // digit 3 among the keys with T's digits 1 and 2
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if ((uint32_t)j * kTN + t < n && (k[j] >> 10) == p2) atomicAdd(&L.rhist[1][k[j] & 1023u], 1u);
  __syncthreads();
  const uint32_t v3[1] = {L.rhist[1][1023 - t]};
  const uint32_t T = (p2 << 10) | block_find<kTN, 1>(v3, 1024, r, L.sh, L.found, &above);
  const uint32_t need = r - above;  // keys equal to T that are kept, lowest rows first

  // per granule: keys above T and equal to it
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if ((uint32_t)j * kTN >= n) break;  // uniform
    const bool in = (uint32_t)j * kTN + t < n;
    const uint64_t mg = __ballot(in && k[j] > T), me = __ballot(in && k[j] == T);
    if (lane == 0) {
      L.gt[j * kTW + wave] = popc64(mg);
      L.eq[j * kTW + wave] = popc64(me);
    }
  }
  __syncthreads();
  const uint32_t ngr = (n + 63) >> 6;
  uint32_t G, E, tg, te;
  dev::block_excl_scan2_dpp<kTN>((uint32_t)t < ngr ? L.gt[t] : 0u, (uint32_t)t < ngr ? L.eq[t] : 0u, L.sh, &G, &E,
                                 &tg, &te);
  if ((uint32_t)t < ngr) {
    L.gt[t] = G + (E < need ? E : need);  // kept rows before granule t
    L.eq[t] = E;                          // keys equal to T before granule t
  }
  __syncthreads();

  // every kept row's slot: kept rows before its granule plus kept lanes below it
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if ((uint32_t)j * kTN >= n) break;  // uniform
    const uint32_t row = (uint32_t)j * kTN + t;
    const bool in = row < n;
    const bool gt = in && k[j] > T, eq = in && k[j] == T;
    const uint32_t g = (uint32_t)(j * kTW + wave);
    const uint32_t e0 = L.eq[g], off = L.gt[g];
    const bool keep = gt || (eq && e0 + lanes_below(__ballot(eq)) < need);
    const uint32_t q = off + lanes_below(__ballot(keep));  // kept rows before this row
    if (out && keep) out[q] = (int32_t)row;
    if constexpr (INPLACE) {
      if (in && row < m && !keep && row - q < io.hcap) io.hole[(size_t)u * io.hcap + row - q] = row;
      if (in && row >= m && keep && m - 1 - q < io.hcap) io.mover[(size_t)u * io.hcap + m - 1 - q] = row;
      if (row == m) w.state[u].moves = m - q;  // m < n here
    }
  }
  if (out)
    for (uint32_t j = m + t; j < (uint32_t)a.B; j += kTN) out[j] = -1;
  if (t == 0) a.kept_cnt[u] = (int32_t)m;
}

// Chunks per candidate workgroup: one while the candidate grid is small, where the launch is
// latency-bound and more workgroups finish sooner; past kCandWgTarget workgroups, chunks are
// merged (up to 16) so that each workgroup reads the unit's histogram and scans it once for
// several chunks.
constexpr int64_t kCandWgTarget = 16384;

int cand_chunks_per_wg(const SelectArgs& a) {
  int cpw = 1;
  while (cpw < 16 && (int64_t)a.n_units * ((a.lay.cand_wgs + cpw - 1) / cpw) > kCandWgTarget) cpw *= 2;
  return cpw;
}

hipError_t launch_cand(const SelectArgs& a, int cpw, hipStream_t s) {
  const int64_t grid = (int64_t)a.n_units * ((a.lay.cand_wgs + cpw - 1) / cpw);
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (cpw == 1) hipLaunchKernelGGL(cand_kernel<512>, dim3((unsigned)grid), dim3(512), 0, s, a, cpw);
  else hipLaunchKernelGGL(cand_kernel<256>, dim3((unsigned)grid), dim3(256), 0, s, a, cpw);
  return hipSuccess;
}

template <bool INPLACE>
hipError_t launch_topb(const SelectArgs& a, const InplaceOut& io, hipStream_t s) {
  const dim3 g((unsigned)a.n_units), b(kTN);
  if (a.max_rows <= 4 * kTN) hipLaunchKernelGGL((topb_kernel<4, INPLACE>), g, b, 0, s, a, io);
  else if (a.max_rows <= 8 * kTN) hipLaunchKernelGGL((topb_kernel<8, INPLACE>), g, b, 0, s, a, io);
  else if (a.max_rows <= 16 * kTN) hipLaunchKernelGGL((topb_kernel<16, INPLACE>), g, b, 0, s, a, io);
  else if (a.max_rows <= 32 * kTN) hipLaunchKernelGGL((topb_kernel<32, INPLACE>), g, b, 0, s, a, io);
  else hipLaunchKernelGGL((topb_kernel<64, INPLACE>), g, b, 0, s, a, io);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const int64_t U = a.n_units;
  const int64_t cand_grid = U * a.lay.cand_wgs;
  const int64_t hpu = (a.max_rows + kHRows - 1) / kHRows;
  if (cand_grid > 0x7FFFFFFF || U * hpu > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (U * ((a.lay.grans + kEW - 1) / kEW) * 2 > 0x7FFFFFFF) return hipErrorInvalidValue;  // emit grids
  if (a.K_out != nullptr && a.row_bytes != 128 && a.row_bytes != 256 && a.row_bytes != 512 && a.row_bytes != 1024)
    return hipErrorInvalidValue;
  if (!a.hist_ready && hpu > 0)
    hipLaunchKernelGGL(hist_kernel, dim3((unsigned)(U * hpu)), dim3(kHN), 0, s, a, (int)hpu);
  const int64_t mm = a.B < a.max_rows ? a.B : a.max_rows;
  const int64_t fin_wgs = (int64_t)a.n_units * (mm > 0 ? (mm + kFinSlots - 1) / kFinSlots : 1);
  if (a.max_rows <= kTopbMaxRows && a.n_units >= kTopbMinUnits && fin_wgs >= kTopbMinFinishGroups) {
    // one workgroup per unit: the units' selects fill the GPU
    hipError_t e = launch_topb<false>(a, InplaceOut{nullptr, nullptr, 0u}, s);
    if (e != hipSuccess || a.K_out == nullptr) return e;
    const CompactArgs c{a.K, a.V, a.pos, a.row_bytes, a.row_off, a.n_units, a.total_rows, a.kept_idx, a.kept_cnt,
                        a.B, a.K_out, a.V_out, a.pos_out};
    return launch_compact(c, s);
  }
  if (a.max_rows <= kFinishMaxRows && fin_wgs <= kFinishMaxWorkgroups) {
    hipError_t e = launch_cand(a, 1, s);
    if (e != hipSuccess) return e;
    switch (a.K_out == nullptr ? 0 : a.row_bytes / 16) {
      case 0: e = launch_finish<0>(a, s); break;
      case 8: e = launch_finish<8>(a, s); break;
      case 16: e = launch_finish<16>(a, s); break;
      case 32: e = launch_finish<32>(a, s); break;
      default: e = launch_finish<64>(a, s); break;
    }
    if (e != hipSuccess) return e;
    return hipGetLastError();
  }
  hipError_t e = launch_cand(a, cand_chunks_per_wg(a), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(resolve_kernel, dim3((unsigned)U), dim3(kRN), 0, s, a);
  if (a.K_out == nullptr) {
    e = launch_emit<0>(a, s);
  } else {
    switch (a.row_bytes / 16) {
      case 8: e = launch_emit<8>(a, s); break;
      case 16: e = launch_emit<16>(a, s); break;
      case 32: e = launch_emit<32>(a, s); break;
      default: e = launch_emit<64>(a, s); break;
    }
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_select_inplace(const SelectArgs& a, const MoveArgs& mv, hipStream_t s) {
  const int64_t U = a.n_units;
  const int64_t cand_grid = U * a.lay.cand_wgs;
  const int64_t mark_grid = U * ((a.lay.grans + kEW - 1) / kEW);
  if (cand_grid > 0x7FFFFFFF || mark_grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (mv.row_bytes != 128 && mv.row_bytes != 256 && mv.row_bytes != 512 && mv.row_bytes != 1024)
    return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  if (a.max_rows <= kTopbMaxRows) {
    e = launch_topb<true>(a, InplaceOut{mv.hole, mv.mover, (uint32_t)mv.hcap}, s);
    if (e != hipSuccess) return e;
  } else {
    e = launch_cand(a, cand_chunks_per_wg(a), s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(resolve_kernel, dim3((unsigned)U), dim3(kRN), 0, s, a);
    hipLaunchKernelGGL(mark_kernel, dim3((unsigned)mark_grid), dim3(kEN), 0, s, a, mv.hole, mv.mover, (uint32_t)mv.hcap);
  }
  switch (mv.row_bytes / 16) {
    case 8: e = launch_move<8>(a, mv, s); break;
    case 16: e = launch_move<16>(a, mv, s); break;
    case 32: e = launch_move<32>(a, mv, s); break;
    default: e = launch_move<64>(a, mv, s); break;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace tri
