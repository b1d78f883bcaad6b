// Standalone compaction of libtri for gfx950: dense copy of the kept rows of every unit.
//
//   K_out[u][j] = K[row_off[u] + kept_idx[u][j]],  V_out and pos_out likewise,  j < kept_cnt[u]
//
// "The future-offset average in TriAttention can be precomputed", introduction (the cache is
// pruned to the kept entries). One thread per 16-byte piece of a row: a workgroup of 256
// threads copies 256 / CPR rows of K and of V with one load and one store each per thread.
#include "tri_device.h"

namespace tri {
namespace {

constexpr int kNT = 256;

template <int CPR>  // 16-byte pieces per row
__global__ __launch_bounds__(kNT) void compact_kernel(CompactArgs a, int blocks_per_unit) {
  constexpr int ROWS = kNT / CPR;
  const int u = blockIdx.x / blocks_per_unit;
  const int b = blockIdx.x - u * blocks_per_unit;
  const dev::UnitRows ur = dev::unit_rows(a.row_off, u, a.total_rows, a.total_rows);
  const int j = b * ROWS + (int)threadIdx.x / CPR;
  const int part = (int)threadIdx.x % CPR;
  // the count and the index are read together (slot j < B is always in range)
  const int32_t src = a.kept_idx[(int64_t)u * a.B + (j < a.B ? j : a.B - 1)];
  int cnt = a.kept_cnt[u];
  cnt = cnt < 0 ? 0 : (cnt > a.B ? a.B : cnt);
  if (j >= cnt) return;
  if (src < 0 || src >= ur.n) return;
  const int64_t srow = ur.beg + src;
  const int64_t drow = (int64_t)u * a.B + j;
  // every load before the stores: a load issued after a store waits for that store too
  const bool with_pos = part == 0 && a.pos_out != nullptr;
  const uint4 kv = static_cast<const uint4*>(a.K)[srow * CPR + part];
  const uint4 vv = static_cast<const uint4*>(a.V)[srow * CPR + part];
  const int32_t pv = with_pos ? a.pos[srow] : 0;
  static_cast<uint4*>(a.K_out)[drow * CPR + part] = kv;
  static_cast<uint4*>(a.V_out)[drow * CPR + part] = vv;
  if (with_pos) a.pos_out[drow] = pv;
}

template <int CPR>
hipError_t launch_t(const CompactArgs& a, hipStream_t s) {
  constexpr int ROWS = kNT / CPR;
  const int64_t bpu = (a.B + ROWS - 1) / ROWS;
  const int64_t grid = bpu * a.n_units;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(compact_kernel<CPR>, dim3((unsigned)grid), dim3(kNT), 0, s, a, (int)bpu);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  switch (a.row_bytes / 16) {
    case 8: return launch_t<8>(a, s);
    case 16: return launch_t<16>(a, s);
    case 32: return launch_t<32>(a, s);
    case 64: return launch_t<64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tri
