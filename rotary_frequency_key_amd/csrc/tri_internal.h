// Internal declarations shared by the C entry points (tri_api.cpp) and the kernel launchers.
// Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tri {

constexpr int kMaxBands = 128;     // d <= 256 on the device path
constexpr int kHistBins = 4096;    // top radix digit: bits 31..20 of the order key
constexpr int kHistShift = 20;

// Select. Rows of a unit are cut into granules of 2^gran_shift rows (64, doubled until a unit of
// max_rows rows has at most kMaxGran of them); the emit kernel gives each granule one wave. The
// candidate kernel gives each workgroup 2^cand_shift rows (max(1024, granule)) and collects the
// keys whose top digit is the threshold's ("candidates"); the resolve kernel stages up to
// kCandCap of them in LDS (beyond that it reads them from the workspace once per pass over
// them). Per-granule counts are kept
// in 16 bits, so granules are at most 2^15 rows and units at most kMaxSelectRows rows.
constexpr int kGranMinShift = 6;
constexpr int kMaxGran = 4096;
constexpr int kCandRowsShift = 10;
constexpr int kCandCap = 4096;
constexpr int64_t kMaxSelectRows = int64_t(kMaxGran) << 15;

// Per-band rotation constants of tri_score. The phase of band f at distance delta is
// frac(delta * omega_f / 2pi) revolutions, evaluated as
//     ((delta * step[f]) mod 2^23) / 2^23  +  delta * resid[f]
// with step[f] = round(frac(omega_f / 2pi) * 2^23) and resid[f] the binary32 remainder.
struct BandConst {
  uint32_t step[kMaxBands];
  float resid[kMaxBands];
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Per-unit select state. b0/above0: written by the candidate kernel (the threshold's top digit
// and the count of keys in higher bins); T/need/mode/m: written by the resolve kernel.
struct UnitState {
  uint32_t T;       // order key of the B-th largest score
  uint32_t need;    // rows equal to T that are kept (the lowest indices)
  uint32_t mode;    // kModeThreshold / kModeAll / kModeNone
  uint32_t m;       // rows kept: min(B, N_u)
  uint32_t b0;      // top digit of T
  uint32_t above0;  // keys whose top digit is above b0
  uint32_t moves;   // in-place pass: kept rows at or beyond slot m (= slots freed below m)
  uint32_t pad;
};
constexpr uint32_t kModeThreshold = 0, kModeAll = 1, kModeNone = 2;

// Workspace: per-unit top-digit histograms [n_units][kHistBins] (zero at rest: the score kernel
// or the histogram kernel adds into them, the candidate kernel reads them, the resolve kernel
// clears them), then scratch that every call writes before it reads it: unit states,
// per-candidate-workgroup candidate counts, the candidates (one word per row: low 20 bits of the
// key above the granule index), and per granule the keys above the top digit, the output offset
// and the ties before it. The histograms come first so that tri_score's workspace is a prefix.
struct WsLayout {
  int gran_shift, grans;     // granule rows = 2^gran_shift; granules per unit (>= 1)
  int cand_shift, cand_wgs;  // candidate workgroup rows = 2^cand_shift; workgroups per unit (>= 1)
  size_t hist, state, wg_cnt, cand, gran_gt, gran_off, gran_eq, total;
};

inline size_t hist_bytes(int n_units) { return (size_t)n_units * kHistBins * 4; }

inline WsLayout ws_layout(int n_units, int64_t max_rows) {
  WsLayout L{};
  int gs = kGranMinShift;
  while ((int64_t(kMaxGran) << gs) < max_rows) ++gs;
  L.gran_shift = gs;
  const int64_t ng = (max_rows + (int64_t(1) << gs) - 1) >> gs;
  L.grans = ng < 1 ? 1 : (int)ng;
  const int cs = gs > kCandRowsShift ? gs : kCandRowsShift;
  L.cand_shift = cs;
  const int64_t nw = (max_rows + (int64_t(1) << cs) - 1) >> cs;
  L.cand_wgs = nw < 1 ? 1 : (int)nw;
  const size_t U = (size_t)n_units;
  size_t off = 0;
  L.hist = off;     off = align256(off + hist_bytes(n_units));
  L.state = off;    off = align256(off + U * sizeof(UnitState));
  L.wg_cnt = off;   off = align256(off + U * L.cand_wgs * 4);
  L.cand = off;     off = align256(off + (U * L.cand_wgs << cs) * 4);
  L.gran_gt = off;  off = align256(off + U * L.grans * 4);
  L.gran_off = off; off = align256(off + U * L.grans * 4);
  L.gran_eq = off;  off = align256(off + U * L.grans * 4);
  L.total = off;
  return L;
}

// In-place pass: the select workspace followed by the freed-slot list and the list of kept rows
// beyond slot m, hcap entries per unit (hcap >= min(B, max_rows - B), the most rows that move).
struct InplaceLayout {
  WsLayout sel;
  int64_t hcap;
  size_t hole, mover, total;
};

inline InplaceLayout inplace_layout(int n_units, int64_t max_rows, int B) {
  InplaceLayout L{};
  L.sel = ws_layout(n_units, max_rows);
  const int64_t spare = max_rows > B ? max_rows - B : 0;
  L.hcap = spare < B ? spare : B;
  if (L.hcap < 1) L.hcap = 1;
  size_t off = L.sel.total;
  L.hole = off;  off = align256(off + (size_t)n_units * L.hcap * 4);
  L.mover = off; off = align256(off + (size_t)n_units * L.hcap * 4);
  L.total = off;
  return L;
}

struct ScoreArgs {
  const void* keys;
  int dtype, layout, d;  // layout: band pairing only (TRI_BANDS_*)
  bool rotated;          // keys stored after the rotary rotation at their positions
  const int64_t* row_off;
  int n_units;
  int64_t total_rows, max_rows;
  const int32_t* pos;
  const int32_t* t_now;
  const float* mu;
  float* scores;
  uint32_t* hist;  // [n_units][kHistBins] or nullptr
};

// Select, optionally fused with the compaction (K_out != nullptr).
struct SelectArgs {
  const float* scores;
  const int64_t* row_off;
  int n_units;
  int64_t total_rows, max_rows;
  int B;
  int32_t* kept_idx;
  int32_t* kept_cnt;
  void* ws;         // workspace, laid out by `lay`
  WsLayout lay;
  bool hist_ready;  // the histograms hold the score kernel's counts
  const void* K;
  const void* V;
  const int32_t* pos;
  int row_bytes;
  void* K_out;
  void* V_out;
  int32_t* pos_out;
};

// In-place pass, after the threshold: freed slots below m and kept rows beyond it.
struct MoveArgs {
  void* K;
  void* V;
  int32_t* pos;  // or nullptr
  int row_bytes;
  uint32_t* hole;
  uint32_t* mover;
  int64_t hcap;
};

struct CompactArgs {
  const void* K;
  const void* V;
  const int32_t* pos;
  int row_bytes;
  const int64_t* row_off;
  int n_units;
  int64_t total_rows;
  const int32_t* kept_idx;
  const int32_t* kept_cnt;
  int B;
  void* K_out;
  void* V_out;
  int32_t* pos_out;
};

// Offset schedule of the max-over-offsets score (each 0 <= delta < 2^24).
constexpr int kMaxOffsets = 32;
struct OffsetSet {
  int n;
  uint32_t delta[kMaxOffsets];
};

hipError_t launch_score(const ScoreArgs& a, const BandConst& bc, hipStream_t s);
hipError_t launch_score_max(const ScoreArgs& a, const BandConst& bc, const OffsetSet& os, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);
// Zero fill of bytes (a multiple of 16) at p (16-byte aligned), as a kernel on s.
hipError_t launch_clear(void* p, size_t bytes, hipStream_t s);

// tri_prune_pass after its size query: every argument check with a workspace of ws_cap bytes at
// ws, then the launches; with clear_hist, the workspace's histograms are zero-filled first (one
// more launch), so it need not be in its rest state. With os (tri_prune_pass_max), the score is
// the maximum over those offsets and mu holds the raw centers.
int prune_pass_run(const void* K, const void* V, int dtype, int layout, int d, double theta, const int64_t* row_off,
                   int n_units, int64_t total_rows, int64_t max_rows, const int32_t* pos, const int32_t* t_now,
                   const float* mu, int B, float* scores, int32_t* kept_idx, int32_t* kept_cnt, void* K_out,
                   void* V_out, int32_t* pos_out, void* ws, size_t ws_cap, bool clear_hist, hipStream_t s,
                   const OffsetSet* os = nullptr);
// tri_prune_inplace after the score: threshold, then the freed slots filled with the kept rows
// beyond them (a.K_out etc. unused).
hipError_t launch_select_inplace(const SelectArgs& a, const MoveArgs& mv, hipStream_t s);

#ifdef TRI_STAMPS
// The timestamp buffer pointer of each stamping source file (the measurement build only).
hipError_t attach_g_stamps_score(void* p);
hipError_t attach_g_stamps_select(void* p);
#endif

}  // namespace tri
