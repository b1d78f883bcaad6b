// C entry points of libtri: host-side argument checks, the offline fold (fp64), the per-band
// rotation constants, and the kernel launches. Every check of a call runs before its first HIP
// call; a failed check enqueues nothing.
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

bool finite_positive(double x) { return std::isfinite(x) && x > 0.0; }

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

// ---- argument checks (no HIP calls) ------------------------------------------------------------

int check_score(const void* keys, int dtype, int layout, int d, double theta, const int64_t* row_off,
                int n_units, int64_t total_rows, int64_t max_rows, const int32_t* pos, const int32_t* t_now,
                const float* mu, const float* scores, const void* hist, size_t hist_bytes) {
  if (n_units < 1 || total_rows < 0 || max_rows < 0 || max_rows >= (int64_t(1) << 31)) return TRI_ERR_ARG;
  if (dtype != TRI_DT_F32 && dtype != TRI_DT_BF16) return TRI_ERR_ARG;
  const int bands = layout & ~TRI_KEYS_ROTATED;
  const bool rotated = (layout & TRI_KEYS_ROTATED) != 0;
  if (bands != TRI_BANDS_INTERLEAVED && bands != TRI_BANDS_HALF_SPLIT) return TRI_ERR_ARG;
  if (!finite_positive(theta)) return TRI_ERR_ARG;
  if (d < 2 || (d % 2) != 0) return TRI_ERR_ARG;
  if (d != 64 && d != 128 && d != 256) return TRI_ERR_UNSUPPORTED;
  if (row_off == nullptr || !aligned(row_off, 8)) return TRI_ERR_ARG;
  if (t_now == nullptr || mu == nullptr || !aligned(t_now, 4) || !aligned(mu, 16)) return TRI_ERR_ARG;
  if (total_rows > 0) {
    if (keys == nullptr || scores == nullptr || (!rotated && pos == nullptr)) return TRI_ERR_ARG;
    if (!aligned(keys, 16) || !aligned(pos, 4) || !aligned(scores, 4)) return TRI_ERR_ARG;
  }
  if (hist != nullptr && !aligned(hist, 256)) return TRI_ERR_ARG;
  const int elem = dtype == TRI_DT_BF16 ? 2 : 4;
  const Range ins[] = {span(keys, total_rows * d * elem), span(pos, total_rows * 4),
                       span(mu, int64_t(n_units) * d * 4), span(t_now, int64_t(n_units) * 4),
                       span(row_off, int64_t(n_units + 1) * 8)};
  const Range out = span(scores, total_rows * 4);
  const Range h = span(hist, hist ? static_cast<int64_t>(hist_bytes) : 0);
  for (const Range& r : ins)
    if (overlap(out, r) || overlap(h, r)) return TRI_ERR_ALIAS;
  if (overlap(out, h)) return TRI_ERR_ALIAS;
  return TRI_OK;
}

int check_select(const float* scores, const int64_t* row_off, int n_units, int64_t total_rows,
                 int64_t max_rows, int B, const int32_t* kept_idx, const int32_t* kept_cnt, const void* ws,
                 size_t ws_total) {
  if (n_units < 1 || total_rows < 0 || max_rows < 0 || max_rows >= (int64_t(1) << 31) || B < 0)
    return TRI_ERR_ARG;
  if (max_rows > tri::kMaxSelectRows) return TRI_ERR_UNSUPPORTED;
  if (row_off == nullptr || !aligned(row_off, 8)) return TRI_ERR_ARG;
  if (kept_cnt == nullptr || !aligned(kept_cnt, 4)) return TRI_ERR_ARG;
  if (B > 0 && (kept_idx == nullptr || !aligned(kept_idx, 4))) return TRI_ERR_ARG;
  if (total_rows > 0 && (scores == nullptr || !aligned(scores, 4))) return TRI_ERR_ARG;
  if (!aligned(ws, 256)) return TRI_ERR_ARG;
  const Range ki = span(kept_idx, int64_t(n_units) * B * 4);
  const Range kc = span(kept_cnt, int64_t(n_units) * 4);
  const Range in_s = span(scores, total_rows * 4);
  const Range in_r = span(row_off, int64_t(n_units + 1) * 8);
  const Range w = span(ws, static_cast<int64_t>(ws_total));
  if (overlap(ki, kc) || overlap(ki, in_s) || overlap(ki, in_r) || overlap(kc, in_s) || overlap(kc, in_r) ||
      overlap(w, ki) || overlap(w, kc) || overlap(w, in_s) || overlap(w, in_r))
    return TRI_ERR_ALIAS;
  return TRI_OK;
}

// Compaction outputs: K_out/V_out [n_units][B] rows, pos_out [n_units][B] or null. `others` are
// further ranges the outputs may not overlap.
int check_compact(const void* K, const void* V, const int32_t* pos, int dtype, int d, int n_units,
                  int64_t total_rows, int B, const void* K_out, const void* V_out, const int32_t* pos_out,
                  const Range* others, int n_others, int* row_bytes_out) {
  if (dtype != TRI_DT_F32 && dtype != TRI_DT_BF16) return TRI_ERR_ARG;
  if (d < 2 || (d % 2) != 0) return TRI_ERR_ARG;
  const int row_bytes = d * (dtype == TRI_DT_BF16 ? 2 : 4);
  if (row_bytes != 128 && row_bytes != 256 && row_bytes != 512 && row_bytes != 1024) return TRI_ERR_UNSUPPORTED;
  if (B > 0) {
    if (K_out == nullptr || V_out == nullptr || !aligned(K_out, 16) || !aligned(V_out, 16)) return TRI_ERR_ARG;
    if (pos_out != nullptr && ((total_rows > 0 && pos == nullptr) || !aligned(pos_out, 4))) return TRI_ERR_ARG;
  }
  if (total_rows > 0) {
    if (K == nullptr || V == nullptr || !aligned(K, 16) || !aligned(V, 16)) return TRI_ERR_ARG;
    if (pos != nullptr && !aligned(pos, 4)) return TRI_ERR_ARG;
  }
  const int64_t out_rows = int64_t(n_units) * B;
  const Range ko = span(K_out, out_rows * row_bytes), vo = span(V_out, out_rows * row_bytes);
  const Range po = span(pos_out, out_rows * 4);
  const Range ins[] = {span(K, total_rows * row_bytes), span(V, total_rows * row_bytes), span(pos, total_rows * 4)};
  for (const Range& r : ins)
    if (overlap(ko, r) || overlap(vo, r) || overlap(po, r)) return TRI_ERR_ALIAS;
  for (int i = 0; i < n_others; ++i)
    if (overlap(ko, others[i]) || overlap(vo, others[i]) || overlap(po, others[i])) return TRI_ERR_ALIAS;
  if (overlap(ko, vo) || overlap(ko, po) || overlap(vo, po)) return TRI_ERR_ALIAS;
  *row_bytes_out = row_bytes;
  return TRI_OK;
}

// The offset set of the max-over-offsets score: 1 .. kMaxOffsets distances in [0, 2^24).
int parse_offsets(const int64_t* offsets, int n_offsets, tri::OffsetSet* os) {
  if (offsets == nullptr || n_offsets < 1) return TRI_ERR_ARG;
  if (n_offsets > tri::kMaxOffsets) return TRI_ERR_UNSUPPORTED;
  *os = tri::OffsetSet{};
  os->n = n_offsets;
  for (int i = 0; i < n_offsets; ++i) {
    if (offsets[i] < 0 || offsets[i] >= (int64_t(1) << 24)) return TRI_ERR_ARG;
    os->delta[i] = static_cast<uint32_t>(offsets[i]);
  }
  return TRI_OK;
}

hipError_t launch_score_call(const void* keys, int dtype, int layout, int d, double theta, const int64_t* row_off,
                             int n_units, int64_t total_rows, int64_t max_rows, const int32_t* pos,
                             const int32_t* t_now, const float* mu, float* scores, void* hist, hipStream_t s) {
  tri::BandConst bc;
  band_constants(d, theta, &bc);
  tri::ScoreArgs a{keys, dtype, layout & ~TRI_KEYS_ROTATED, d, (layout & TRI_KEYS_ROTATED) != 0, row_off,
                   n_units, total_rows, max_rows, pos, t_now, mu, scores, static_cast<uint32_t*>(hist)};
  return tri::launch_score(a, bc, s);
}

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
  const size_t need = tri::hist_bytes(n_units);
  if (ws == nullptr && ws_bytes != nullptr) {  // size query
    *ws_bytes = need;
    return TRI_OK;
  }
  void* hist = nullptr;
  if (ws_bytes != nullptr) {
    if (*ws_bytes < need) return TRI_ERR_WORKSPACE;
    hist = ws;
  }
  const int st = check_score(keys, dtype, layout, d, theta, row_off, n_units, total_rows, max_rows, pos, t_now,
                             mu, scores, hist, need);
  if (st != TRI_OK) return st;
  if (launch_score_call(keys, dtype, layout, d, theta, row_off, n_units, total_rows, max_rows, pos, t_now, mu,
                        scores, hist, static_cast<hipStream_t>(stream)) != hipSuccess)
    return TRI_ERR_HIP;
  return TRI_OK;
}

int tri_score_max(const void* keys, int dtype, int layout, int d, double theta, const int64_t* offsets,
                  int n_offsets, const int64_t* row_off, int n_units, int64_t total_rows, int64_t max_rows,
                  const int32_t* pos, const int32_t* t_now, const float* centers, float* scores, void* ws,
                  size_t* ws_bytes, void* stream) {
  if (n_units < 1) return TRI_ERR_ARG;
  const size_t need = tri::hist_bytes(n_units);
  if (ws == nullptr && ws_bytes != nullptr) {  // size query
    *ws_bytes = need;
    return TRI_OK;
  }
  tri::OffsetSet os;
  const int so = parse_offsets(offsets, n_offsets, &os);
  if (so != TRI_OK) return so;
  void* hist = nullptr;
  if (ws_bytes != nullptr) {
    if (*ws_bytes < need) return TRI_ERR_WORKSPACE;
    hist = ws;
  }
  const int st = check_score(keys, dtype, layout, d, theta, row_off, n_units, total_rows, max_rows, pos, t_now,
                             centers, scores, hist, need);
  if (st != TRI_OK) return st;
  tri::BandConst bc;
  band_constants(d, theta, &bc);
  tri::ScoreArgs a{keys, dtype, layout & ~TRI_KEYS_ROTATED, d, (layout & TRI_KEYS_ROTATED) != 0, row_off, n_units,
                   total_rows, max_rows, pos, t_now, centers, scores, static_cast<uint32_t*>(hist)};
  if (tri::launch_score_max(a, bc, os, static_cast<hipStream_t>(stream)) != hipSuccess) return TRI_ERR_HIP;
  return TRI_OK;
}

int tri_select_topb(const float* scores, const int64_t* row_off, int n_units,
                    int64_t total_rows, int64_t max_rows, int B, int32_t* kept_idx,
                    int32_t* kept_cnt, void* ws, size_t* ws_bytes, unsigned flags,
                    void* stream) {
  if (n_units < 1 || (flags & ~TRI_SELECT_HIST_FROM_SCORE) != 0) return TRI_ERR_ARG;
  if (max_rows < 0 || max_rows >= (int64_t(1) << 31)) return TRI_ERR_ARG;
  const tri::WsLayout lay = tri::ws_layout(n_units, max_rows);
  const size_t total = lay.total;
  if (ws == nullptr && ws_bytes != nullptr) {  // size query
    *ws_bytes = total;
    return TRI_OK;
  }
  const int st = check_select(scores, row_off, n_units, total_rows, max_rows, B, kept_idx, kept_cnt, ws, total);
  if (st != TRI_OK) return st;
  if (ws == nullptr || ws_bytes == nullptr || *ws_bytes < total) return TRI_ERR_WORKSPACE;
  tri::SelectArgs a{};
  a.scores = scores; a.row_off = row_off; a.n_units = n_units; a.total_rows = total_rows;
  a.max_rows = max_rows; a.B = B; a.kept_idx = kept_idx; a.kept_cnt = kept_cnt;
  a.ws = ws;
  a.lay = lay;
  a.hist_ready = (flags & TRI_SELECT_HIST_FROM_SCORE) != 0;
  if (tri::launch_select(a, static_cast<hipStream_t>(stream)) != hipSuccess) return TRI_ERR_HIP;
  return TRI_OK;
}

int tri_compact_kv(const void* K, const void* V, const int32_t* pos, int dtype, int d,
                   const int64_t* row_off, int n_units, int64_t total_rows,
                   const int32_t* kept_idx, const int32_t* kept_cnt, int B, void* K_out,
                   void* V_out, int32_t* pos_out, void* stream) {
  if (n_units < 1 || total_rows < 0 || B < 0) return TRI_ERR_ARG;
  if (row_off == nullptr || !aligned(row_off, 8)) return TRI_ERR_ARG;
  if (kept_cnt == nullptr || !aligned(kept_cnt, 4)) return TRI_ERR_ARG;
  if (B > 0 && (kept_idx == nullptr || !aligned(kept_idx, 4))) return TRI_ERR_ARG;
  const int64_t out_rows = int64_t(n_units) * B;
  const Range others[] = {span(row_off, int64_t(n_units + 1) * 8), span(kept_idx, out_rows * 4),
                          span(kept_cnt, int64_t(n_units) * 4)};
  int row_bytes = 0;
  const int st = check_compact(K, V, pos, dtype, d, n_units, total_rows, B, K_out, V_out, pos_out, others, 3,
                               &row_bytes);
  if (st != TRI_OK) return st;
  tri::CompactArgs a{K, V, pos, row_bytes, row_off, n_units, total_rows, kept_idx, kept_cnt, B,
                     K_out, V_out, pos_out};
  if (tri::launch_compact(a, static_cast<hipStream_t>(stream)) != hipSuccess) return TRI_ERR_HIP;
  return TRI_OK;
}

int tri_prune_pass(const void* K, const void* V, int dtype, int layout, int d, double theta,
                   const int64_t* row_off, int n_units, int64_t total_rows, int64_t max_rows,
                   const int32_t* pos, const int32_t* t_now, const float* mu, int B, float* scores,
                   int32_t* kept_idx, int32_t* kept_cnt, void* K_out, void* V_out, int32_t* pos_out,
                   void* ws, size_t* ws_bytes, void* stream) {
  if (n_units < 1 || max_rows < 0 || max_rows >= (int64_t(1) << 31)) return TRI_ERR_ARG;
  if (ws == nullptr && ws_bytes != nullptr) {  // size query
    *ws_bytes = tri::ws_layout(n_units, max_rows).total;
    return TRI_OK;
  }
  return tri::prune_pass_run(K, V, dtype, layout, d, theta, row_off, n_units, total_rows, max_rows, pos, t_now, mu,
                             B, scores, kept_idx, kept_cnt, K_out, V_out, pos_out, ws,
                             ws_bytes != nullptr ? *ws_bytes : 0, false, static_cast<hipStream_t>(stream));
}

int tri_prune_pass_max(const void* K, const void* V, int dtype, int layout, int d, double theta,
                       const int64_t* offsets, int n_offsets, const int64_t* row_off, int n_units,
                       int64_t total_rows, int64_t max_rows, const int32_t* pos, const int32_t* t_now,
                       const float* centers, int B, float* scores, int32_t* kept_idx, int32_t* kept_cnt,
                       void* K_out, void* V_out, int32_t* pos_out, void* ws, size_t* ws_bytes, void* stream) {
  if (n_units < 1 || max_rows < 0 || max_rows >= (int64_t(1) << 31)) return TRI_ERR_ARG;
  if (ws == nullptr && ws_bytes != nullptr) {  // size query: the workspace of tri_prune_pass
    *ws_bytes = tri::ws_layout(n_units, max_rows).total;
    return TRI_OK;
  }
  tri::OffsetSet os;
  const int so = parse_offsets(offsets, n_offsets, &os);
  if (so != TRI_OK) return so;
  return tri::prune_pass_run(K, V, dtype, layout, d, theta, row_off, n_units, total_rows, max_rows, pos, t_now,
                             centers, B, scores, kept_idx, kept_cnt, K_out, V_out, pos_out, ws,
                             ws_bytes != nullptr ? *ws_bytes : 0, false, static_cast<hipStream_t>(stream), &os);
}

}  // extern "C"

namespace tri {

int prune_pass_run(const void* K, const void* V, int dtype, int layout, int d, double theta, const int64_t* row_off,
                   int n_units, int64_t total_rows, int64_t max_rows, const int32_t* pos, const int32_t* t_now,
                   const float* mu, int B, float* scores, int32_t* kept_idx, int32_t* kept_cnt, void* K_out,
                   void* V_out, int32_t* pos_out, void* ws, size_t ws_cap, bool clear_hist, hipStream_t s,
                   const OffsetSet* os) {
  if (n_units < 1 || max_rows < 0 || max_rows >= (int64_t(1) << 31)) return TRI_ERR_ARG;
  const WsLayout lay = ws_layout(n_units, max_rows);
  const size_t total = lay.total;
  int st = check_score(K, dtype, layout, d, theta, row_off, n_units, total_rows, max_rows, pos, t_now, mu, scores,
                       ws, total);
  if (st != TRI_OK) return st;
  st = check_select(scores, row_off, n_units, total_rows, max_rows, B, kept_idx, kept_cnt, ws, total);
  if (st != TRI_OK) return st;
  const int64_t out_rows = int64_t(n_units) * B;
  const Range others[] = {span(row_off, int64_t(n_units + 1) * 8), span(t_now, int64_t(n_units) * 4),
                          span(mu, int64_t(n_units) * d * 4), span(scores, total_rows * 4),
                          span(kept_idx, out_rows * 4), span(kept_cnt, int64_t(n_units) * 4),
                          span(ws, static_cast<int64_t>(total))};
  int row_bytes = 0;
  st = check_compact(K, V, pos, dtype, d, n_units, total_rows, B, K_out, V_out, pos_out, others, 7, &row_bytes);
  if (st != TRI_OK) return st;
  // scores vs kept_idx / kept_cnt: the one pair of outputs the checks above do not compare
  if (overlap(span(scores, total_rows * 4), span(kept_idx, out_rows * 4)) ||
      overlap(span(scores, total_rows * 4), span(kept_cnt, int64_t(n_units) * 4)))
    return TRI_ERR_ALIAS;
  if (ws == nullptr || ws_cap < total) return TRI_ERR_WORKSPACE;

  if (clear_hist && launch_clear(ws, hist_bytes(n_units), s) != hipSuccess) return TRI_ERR_HIP;
  if (os != nullptr) {  // the maximum over the offsets, from the raw centers, histogram into ws
    BandConst bc;
    band_constants(d, theta, &bc);
    const ScoreArgs sa{K, dtype, layout & ~TRI_KEYS_ROTATED, d, (layout & TRI_KEYS_ROTATED) != 0, row_off,
                       n_units, total_rows, max_rows, pos, t_now, mu, scores, static_cast<uint32_t*>(ws)};
    if (launch_score_max(sa, bc, *os, s) != hipSuccess) return TRI_ERR_HIP;
  } else if (launch_score_call(K, dtype, layout, d, theta, row_off, n_units, total_rows, max_rows, pos, t_now, mu,
                               scores, ws, s) != hipSuccess) {
    return TRI_ERR_HIP;
  }
  SelectArgs a{};
  a.scores = scores; a.row_off = row_off; a.n_units = n_units; a.total_rows = total_rows;
  a.max_rows = max_rows; a.B = B; a.kept_idx = kept_idx; a.kept_cnt = kept_cnt;
  a.ws = ws;
  a.lay = lay;
  a.hist_ready = true;
  if (B > 0) {
    a.K = K; a.V = V; a.pos = pos; a.row_bytes = row_bytes;
    a.K_out = K_out; a.V_out = V_out; a.pos_out = pos_out;
  }
  if (launch_select(a, s) != hipSuccess) return TRI_ERR_HIP;
  return TRI_OK;
}

}  // namespace tri

extern "C" {

int tri_prune_inplace(void* K, void* V, int32_t* pos, int dtype, int layout, int d, double theta,
                      const int64_t* row_off, int n_units, int64_t total_rows, int64_t max_rows,
                      const int32_t* t_now, const float* mu, int B, float* scores, int32_t* kept_cnt,
                      void* ws, size_t* ws_bytes, void* stream) {
  if (n_units < 1 || B < 0 || max_rows < 0 || max_rows >= (int64_t(1) << 31)) return TRI_ERR_ARG;
  const tri::InplaceLayout lay = tri::inplace_layout(n_units, max_rows, B);
  if (ws == nullptr && ws_bytes != nullptr) {  // size query
    *ws_bytes = lay.total;
    return TRI_OK;
  }
  int st = check_score(K, dtype, layout, d, theta, row_off, n_units, total_rows, max_rows, pos, t_now, mu, scores,
                       ws, lay.total);
  if (st != TRI_OK) return st;
  if (max_rows > tri::kMaxSelectRows) return TRI_ERR_UNSUPPORTED;
  if (kept_cnt == nullptr || !aligned(kept_cnt, 4)) return TRI_ERR_ARG;
  if (!aligned(ws, 256)) return TRI_ERR_ARG;
  const int row_bytes = d * (dtype == TRI_DT_BF16 ? 2 : 4);
  if (total_rows > 0 && (V == nullptr || !aligned(V, 16))) return TRI_ERR_ARG;
  // K, V and pos are read and written; none of the buffers may overlap another
  const Range bufs[] = {span(K, total_rows * row_bytes), span(V, total_rows * row_bytes),
                        span(pos, total_rows * 4),        span(scores, total_rows * 4),
                        span(kept_cnt, int64_t(n_units) * 4), span(ws, static_cast<int64_t>(lay.total)),
                        span(row_off, int64_t(n_units + 1) * 8), span(t_now, int64_t(n_units) * 4),
                        span(mu, int64_t(n_units) * d * 4)};
  const int nb = static_cast<int>(sizeof(bufs) / sizeof(bufs[0]));
  for (int i = 0; i < nb; ++i)
    for (int j = i + 1; j < nb; ++j)
      if (overlap(bufs[i], bufs[j])) return TRI_ERR_ALIAS;
  if (ws == nullptr || ws_bytes == nullptr || *ws_bytes < lay.total) return TRI_ERR_WORKSPACE;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_score_call(K, dtype, layout, d, theta, row_off, n_units, total_rows, max_rows, pos, t_now, mu, scores,
                        ws, s) != hipSuccess)
    return TRI_ERR_HIP;
  tri::SelectArgs a{};
  a.scores = scores; a.row_off = row_off; a.n_units = n_units; a.total_rows = total_rows;
  a.max_rows = max_rows; a.B = B; a.kept_idx = nullptr; a.kept_cnt = kept_cnt;
  a.ws = ws;
  a.lay = lay.sel;
  a.hist_ready = true;
  char* w = static_cast<char*>(ws);
  tri::MoveArgs mv{K, V, pos, row_bytes, reinterpret_cast<uint32_t*>(w + lay.hole),
                   reinterpret_cast<uint32_t*>(w + lay.mover), lay.hcap};
  if (tri::launch_select_inplace(a, mv, s) != hipSuccess) return TRI_ERR_HIP;
  return TRI_OK;
}

}  // extern "C"

#ifdef TRI_STAMPS
#include "stamps.h"
#include "tri_stamps.h"

extern "C" {

int tri_stamps_layout(int* wgs, int* points, int* kernels) {
  if (wgs) *wgs = tri::stamps::kWgs;
  if (points) *points = tri::stamps::kPoints;
  if (kernels) *kernels = tri::stamps::kKernels;
  return TRI_OK;
}

int tri_stamps_attach(void* buf) {
  if (tri::attach_g_stamps_score(buf) != hipSuccess) return TRI_ERR_HIP;
  if (tri::attach_g_stamps_select(buf) != hipSuccess) return TRI_ERR_HIP;
  return TRI_OK;
}

}  // extern "C"
#endif
