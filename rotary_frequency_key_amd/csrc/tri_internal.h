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

// Select: candidates (keys in the threshold's top-digit bin) buffered in LDS up to kCandCap,
// beyond which the last two digits are counted from the scores directly. Units are cut into
// chunks of chunk_rows rows (a power of two >= 1024) so that no unit has more than kMaxChunks.
constexpr int kCandCap = 8192;
constexpr int kChunkMin = 1024;
constexpr int kMaxChunks = 2048;
// Output slots per workgroup of the emit / gather kernel.
constexpr int kSlots = 64;

// Per-band rotation constants of tri_score. The phase of band f at distance delta is
// frac(delta * omega_f / 2pi) revolutions, evaluated as
//     ((delta * step[f]) mod 2^23) / 2^23  +  delta * resid[f]
// with step[f] = round(frac(omega_f / 2pi) * 2^23) and resid[f] the binary32 remainder.
struct BandConst {
  uint32_t step[kMaxBands];
  float resid[kMaxBands];
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Per-unit result of the threshold kernel, read by the emit kernel.
struct UnitState {
  uint32_t T;     // order key of the B-th largest score
  uint32_t need;  // rows equal to T that are kept (the lowest indices)
  uint32_t mode;  // kModeThreshold / kModeAll / kModeNone
  uint32_t m;     // rows kept: min(B, N_u)
};
constexpr uint32_t kModeThreshold = 0, kModeAll = 1, kModeNone = 2;

// Workspace: per-unit top-digit histograms [n_units][kHistBins] (zero at rest: the score kernel
// adds into them, the threshold kernel reads and clears them), then scratch written before it
// is read in every call: unit states, per-chunk output offsets and per-chunk counts of ties
// before the chunk. The histograms come first so that tri_score's workspace is a prefix.
struct WsLayout {
  int chunk_rows, chunk_shift, chunks;
  size_t hist, state, chunk_off, chunk_eq, total;
};

inline size_t hist_bytes(int n_units) { return (size_t)n_units * kHistBins * 4; }

inline WsLayout ws_layout(int n_units, int64_t max_rows) {
  WsLayout L{};
  int64_t cr = kChunkMin;
  while (cr * kMaxChunks < max_rows) cr *= 2;
  L.chunk_rows = (int)cr;
  L.chunk_shift = 0;
  while ((int64_t(1) << L.chunk_shift) < cr) ++L.chunk_shift;
  const int64_t ch = (max_rows + cr - 1) / cr;
  L.chunks = ch < 1 ? 1 : (int)ch;
  const size_t U = (size_t)n_units;
  size_t off = 0;
  L.hist = off;      off = align256(off + hist_bytes(n_units));
  L.state = off;     off = align256(off + U * sizeof(UnitState));
  L.chunk_off = off; off = align256(off + U * L.chunks * 4);
  L.chunk_eq = off;  off = align256(off + U * L.chunks * 4);
  L.total = off;
  return L;
}

struct ScoreArgs {
  const void* keys;
  int dtype, layout, d;
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

hipError_t launch_score(const ScoreArgs& a, const BandConst& bc, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);

}  // namespace tri
