// Internal declarations shared by the C entry points (tri_api.cpp) and the kernel launchers
// (tri_kernels.hip). Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tri {

constexpr int kMaxBands = 128;     // d <= 256 on the device path
constexpr int kHistBins = 4096;    // top radix digit: bits 31..20 of the order key
constexpr int kHistShift = 20;

// Per-band rotation constants of tri_score. The phase of band f at distance delta is
// frac(delta * omega_f / 2pi) revolutions, evaluated as
//     ((delta * step[f]) mod 2^23) / 2^23  +  delta * resid[f]
// with step[f] = round(frac(omega_f / 2pi) * 2^23) and resid[f] the binary32 remainder.
struct BandConst {
  uint32_t step[kMaxBands];
  float resid[kMaxBands];
};

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

struct SelectArgs {
  const float* scores;
  const int64_t* row_off;
  int n_units;
  int64_t total_rows, max_rows;
  int B;
  int32_t* kept_idx;
  int32_t* kept_cnt;
  uint32_t* hist;   // [n_units][kHistBins] or nullptr
  bool hist_ready;  // hist holds the score kernel's histogram
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
