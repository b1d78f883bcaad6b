// tri_prune_pass_noalloc: the pruning pass with its workspace in a static device array instead of
// a caller's buffer, for callers that cannot allocate device memory.
//
// The array lives in the library's code object, one copy per GPU, from the first launch of the
// library on that GPU until the process ends. Its address on a GPU is taken once, with that GPU
// current, through hipGetSymbolAddress, and kept per device; host code uses only that address
// (the array's own name is a host-side stand-in, not a device address). Each call zero-fills the
// histograms it uses, so it does not depend on what an earlier call left behind; calls that
// overlap on one GPU share the array and race.
#include <mutex>

#include "tri.h"
#include "tri_internal.h"

namespace tri {
namespace {

static_assert(TRI_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[TRI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once taken

__global__ __launch_bounds__(256) void clear_kernel(uint4* p, size_t n16) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The scratch address on the stream's device, which must be the current device.
int scratch_address(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TRI_ERR_HIP;
  if (s != nullptr) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(s, &sd) != hipSuccess) return TRI_ERR_HIP;
    if (sd != dev) return TRI_ERR_ARG;
  }
  if (dev < 0 || dev >= kMaxDevices) return TRI_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TRI_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TRI_OK;
}

}  // namespace

hipError_t launch_clear(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t grid = (n16 + 255) / 256;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)grid), dim3(256), 0, s, static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace tri

int tri_prune_pass_noalloc(const void* K, const void* V, int dtype, int layout, int d, double theta,
                           const int64_t* row_off, int n_units, int64_t total_rows, int64_t max_rows,
                           const int32_t* pos, const int32_t* t_now, const float* mu, int B, float* scores,
                           int32_t* kept_idx, int32_t* kept_cnt, void* K_out, void* V_out, int32_t* pos_out,
                           void* stream) {
  if (n_units < 1 || max_rows < 0 || max_rows >= (int64_t(1) << 31)) return TRI_ERR_ARG;
  if (tri::ws_layout(n_units, max_rows).total > (size_t)TRI_NOALLOC_SCRATCH_BYTES) return TRI_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const int st = tri::scratch_address(s, &ws);
  if (st != TRI_OK) return st;
  return tri::prune_pass_run(K, V, dtype, layout, d, theta, row_off, n_units, total_rows, max_rows, pos, t_now, mu,
                             B, scores, kept_idx, kept_cnt, K_out, V_out, pos_out, ws,
                             (size_t)TRI_NOALLOC_SCRATCH_BYTES, true, s);
}
