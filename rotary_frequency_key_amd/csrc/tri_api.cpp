// C entry points of libtri: host-side argument checks, the offline fold (fp64), the per-band
// rotation constants, and the kernel launches. Every check runs before the first HIP call.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "tri.h"
#include "tri_internal.h"

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes > 0 ? bytes : 0)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

size_t hist_bytes(int n_units) { return static_cast<size_t>(n_units) * tri::kHistBins * sizeof(uint32_t); }

// omega_f = theta^(-2f/d): "The future-offset average in TriAttention can be precomputed",
// section "The score TriAttention computes".
double omega(int f, int d, double theta) { return std::pow(theta, -2.0 * f / d); }

// Per-band fixed-point rotation constants: r = omega_f / 2pi revolutions per position,
// step = round(frac(r) 2^23) mod 2^23, resid = frac(r) - round(frac(r) 2^23) / 2^23.
// With delta < 2^24: frac(delta r) = frac((delta step mod 2^23) / 2^23 + delta resid).
void band_constants(int d, double theta, tri::BandConst* bc) {
  std::memset(bc, 0, sizeof(*bc));
  for (int f = 0; f < d / 2; ++f) {
    const double r = omega(f, d, theta) / kTwoPi;
    const double fr = r - std::floor(r);
    const double scaled = fr * 8388608.0;  // exact: power-of-two scaling
    const double q = std::nearbyint(scaled);
    bc->step[f] = static_cast<uint32_t>(static_cast<int64_t>(q) & 0x7FFFFF);
    bc->resid[f] = static_cast<float>((scaled - q) / 8388608.0);
  }
}

bool finite_positive(double x) { return std::isfinite(x) && x > 0.0; }

}  // namespace

extern "C" {

const char* tri_status_string(int status) {
  switch (status) {
    case TRI_OK: return "ok";
    case TRI_ERR_ARG: return "invalid argument";
    case TRI_ERR_UNSUPPORTED: return "unsupported configuration";
    case TRI_ERR_ALIAS: return "output overlaps an input or another output";
    case TRI_ERR_WORKSPACE: return "workspace missing or too small";
    case TRI_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int tri_fold_weights(int d, double theta, const int64_t* offsets, int n_offsets,
                     const float* centers, int n_units, double* W_out, float* mu_out) {
  if (d < 2 || d > 512 || (d % 2) != 0) return TRI_ERR_ARG;
  if (!finite_positive(theta)) return TRI_ERR_ARG;
  if (offsets == nullptr || n_offsets < 1 || W_out == nullptr) return TRI_ERR_ARG;
  if (centers != nullptr && n_units < 0) return TRI_ERR_ARG;
  const int F = d / 2;
  // W_f = (1/|D|) sum_delta e^{i omega_f delta}: section "The averaging step".
  for (int f = 0; f < F; ++f) {
    const double w = omega(f, d, theta);
    double re = 0.0, im = 0.0;
    for (int j = 0; j < n_offsets; ++j) {
      const double ang = w * static_cast<double>(offsets[j]);
      re += std::cos(ang);
      im += std::sin(ang);
    }
    W_out[2 * f] = re / n_offsets;
    W_out[2 * f + 1] = im / n_offsets;
  }
  // mu'_f = E[q_f] W_f, rounded once to binary32.
  if (centers != nullptr && mu_out != nullptr) {
    for (int u = 0; u < n_units; ++u) {
      for (int f = 0; f < F; ++f) {
        const double qr = centers[(static_cast<size_t>(u) * F + f) * 2];
        const double qi = centers[(static_cast<size_t>(u) * F + f) * 2 + 1];
        const double wr = W_out[2 * f], wi = W_out[2 * f + 1];
        mu_out[(static_cast<size_t>(u) * F + f) * 2] = static_cast<float>(qr * wr - qi * wi);
        mu_out[(static_cast<size_t>(u) * F + f) * 2 + 1] = static_cast<float>(qr * wi + qi * wr);
      }
    }
  }
  return TRI_OK;
}

int tri_score(const void* keys, int dtype, int layout, int d, double theta,
              const int64_t* row_off, int n_units, int64_t total_rows, int64_t max_rows,
              const int32_t* pos, const int32_t* t_now, const float* mu, float* scores,
              void* ws, size_t* ws_bytes, void* stream) {
  if (n_units < 1) return TRI_ERR_ARG;
  const size_t need = hist_bytes(n_units);
  if (ws == nullptr && ws_bytes != nullptr) {  // size query
    *ws_bytes = need;
    return TRI_OK;
  }
  if (total_rows < 0 || max_rows < 0 || max_rows >= (int64_t(1) << 31)) return TRI_ERR_ARG;
  if (dtype != TRI_DT_F32 && dtype != TRI_DT_BF16) return TRI_ERR_ARG;
  if (layout != TRI_BANDS_INTERLEAVED && layout != TRI_BANDS_HALF_SPLIT) return TRI_ERR_ARG;
  if (!finite_positive(theta)) return TRI_ERR_ARG;
  if (d < 2 || (d % 2) != 0) return TRI_ERR_ARG;
  if (d != 64 && d != 128 && d != 256) return TRI_ERR_UNSUPPORTED;
  if (row_off == nullptr || !aligned(row_off, 8)) return TRI_ERR_ARG;
  if (t_now == nullptr || mu == nullptr || !aligned(t_now, 4) || !aligned(mu, 16)) return TRI_ERR_ARG;
  if (total_rows > 0) {
    if (keys == nullptr || pos == nullptr || scores == nullptr) return TRI_ERR_ARG;
    if (!aligned(keys, 16) || !aligned(pos, 4) || !aligned(scores, 4)) return TRI_ERR_ARG;
  }
  uint32_t* hist = nullptr;
  if (ws_bytes != nullptr) {
    if (*ws_bytes < need) return TRI_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return TRI_ERR_ARG;
    hist = static_cast<uint32_t*>(ws);
  }
  const int elem = dtype == TRI_DT_BF16 ? 2 : 4;
  const Range out = span(scores, total_rows * 4);
  if (overlap(out, span(keys, total_rows * d * elem)) || overlap(out, span(pos, total_rows * 4)) ||
      overlap(out, span(mu, int64_t(n_units) * d * 4)) || overlap(out, span(t_now, int64_t(n_units) * 4)) ||
      overlap(out, span(row_off, int64_t(n_units + 1) * 8)))
    return TRI_ERR_ALIAS;
  if (hist) {
    const Range h = span(hist, static_cast<int64_t>(need));
    if (overlap(h, out) || overlap(h, span(keys, total_rows * d * elem)) || overlap(h, span(pos, total_rows * 4)) ||
        overlap(h, span(mu, int64_t(n_units) * d * 4)) || overlap(h, span(t_now, int64_t(n_units) * 4)) ||
        overlap(h, span(row_off, int64_t(n_units + 1) * 8)))
      return TRI_ERR_ALIAS;
  }

  tri::BandConst bc;
  band_constants(d, theta, &bc);
  tri::ScoreArgs a{keys, dtype, layout, d, row_off, n_units, total_rows, max_rows,
                   pos, t_now, mu, scores, hist};
  if (tri::launch_score(a, bc, static_cast<hipStream_t>(stream)) != hipSuccess) return TRI_ERR_HIP;
  return TRI_OK;
}

int tri_select_topb(const float* scores, const int64_t* row_off, int n_units,
                    int64_t total_rows, int64_t max_rows, int B, int32_t* kept_idx,
                    int32_t* kept_cnt, void* ws, size_t* ws_bytes, unsigned flags,
                    void* stream) {
  if (n_units < 1 || (flags & ~TRI_SELECT_HIST_FROM_SCORE) != 0) return TRI_ERR_ARG;
  const bool from_score = (flags & TRI_SELECT_HIST_FROM_SCORE) != 0;
  const size_t need = from_score ? hist_bytes(n_units) : 0;
  if (ws == nullptr && ws_bytes != nullptr) {  // size query
    *ws_bytes = need;
    return TRI_OK;
  }
  if (total_rows < 0 || max_rows < 0 || max_rows >= (int64_t(1) << 31) || B < 0) return TRI_ERR_ARG;
  if (row_off == nullptr || !aligned(row_off, 8)) return TRI_ERR_ARG;
  if (kept_cnt == nullptr || !aligned(kept_cnt, 4)) return TRI_ERR_ARG;
  if (B > 0 && (kept_idx == nullptr || !aligned(kept_idx, 4))) return TRI_ERR_ARG;
  if (total_rows > 0 && (scores == nullptr || !aligned(scores, 4))) return TRI_ERR_ARG;
  uint32_t* hist = nullptr;
  if (from_score) {
    if (ws == nullptr || ws_bytes == nullptr || *ws_bytes < need) return TRI_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return TRI_ERR_ARG;
    hist = static_cast<uint32_t*>(ws);
  }
  const Range ki = span(kept_idx, int64_t(n_units) * B * 4);
  const Range kc = span(kept_cnt, int64_t(n_units) * 4);
  const Range in_s = span(scores, total_rows * 4);
  const Range in_r = span(row_off, int64_t(n_units + 1) * 8);
  if (overlap(ki, kc) || overlap(ki, in_s) || overlap(ki, in_r) || overlap(kc, in_s) || overlap(kc, in_r))
    return TRI_ERR_ALIAS;
  if (hist) {
    const Range h = span(hist, static_cast<int64_t>(need));
    if (overlap(h, ki) || overlap(h, kc) || overlap(h, in_s) || overlap(h, in_r)) return TRI_ERR_ALIAS;
  }
  tri::SelectArgs a{scores, row_off, n_units, total_rows, max_rows, B, kept_idx, kept_cnt, hist, from_score};
  if (tri::launch_select(a, static_cast<hipStream_t>(stream)) != hipSuccess) return TRI_ERR_HIP;
  return TRI_OK;
}

int tri_compact_kv(const void* K, const void* V, const int32_t* pos, int dtype, int d,
                   const int64_t* row_off, int n_units, int64_t total_rows,
                   const int32_t* kept_idx, const int32_t* kept_cnt, int B, void* K_out,
                   void* V_out, int32_t* pos_out, void* stream) {
  if (n_units < 1 || total_rows < 0 || B < 0) return TRI_ERR_ARG;
  if (dtype != TRI_DT_F32 && dtype != TRI_DT_BF16) return TRI_ERR_ARG;
  if (d < 2 || (d % 2) != 0) return TRI_ERR_ARG;
  const int elem = dtype == TRI_DT_BF16 ? 2 : 4;
  const int row_bytes = d * elem;
  if (row_bytes != 128 && row_bytes != 256 && row_bytes != 512 && row_bytes != 1024) return TRI_ERR_UNSUPPORTED;
  if (row_off == nullptr || !aligned(row_off, 8)) return TRI_ERR_ARG;
  if (kept_cnt == nullptr || !aligned(kept_cnt, 4)) return TRI_ERR_ARG;
  if (B > 0 && pos_out != nullptr && pos == nullptr) return TRI_ERR_ARG;
  if (B > 0) {
    if (kept_idx == nullptr || K_out == nullptr || V_out == nullptr) return TRI_ERR_ARG;
    if (!aligned(kept_idx, 4) || !aligned(K_out, 16) || !aligned(V_out, 16)) return TRI_ERR_ARG;
    if (pos_out != nullptr && !aligned(pos_out, 4)) return TRI_ERR_ARG;
  }
  if (total_rows > 0) {
    if (K == nullptr || V == nullptr || !aligned(K, 16) || !aligned(V, 16)) return TRI_ERR_ARG;
    if (pos != nullptr && !aligned(pos, 4)) return TRI_ERR_ARG;
  }
  const int64_t out_rows = int64_t(n_units) * B;
  const Range ko = span(K_out, out_rows * row_bytes), vo = span(V_out, out_rows * row_bytes);
  const Range po = span(pos_out, out_rows * 4);
  const Range ins[] = {span(K, total_rows * row_bytes), span(V, total_rows * row_bytes),
                       span(pos, total_rows * 4), span(row_off, int64_t(n_units + 1) * 8),
                       span(kept_idx, out_rows * 4), span(kept_cnt, int64_t(n_units) * 4)};
  for (const Range& r : ins)
    if (overlap(ko, r) || overlap(vo, r) || overlap(po, r)) return TRI_ERR_ALIAS;
  if (overlap(ko, vo) || overlap(ko, po) || overlap(vo, po)) return TRI_ERR_ALIAS;
  tri::CompactArgs a{K, V, pos, row_bytes, row_off, n_units, total_rows, kept_idx, kept_cnt, B,
                     K_out, V_out, pos_out};
  if (tri::launch_compact(a, static_cast<hipStream_t>(stream)) != hipSuccess) return TRI_ERR_HIP;
  return TRI_OK;
}

}  // extern "C"
