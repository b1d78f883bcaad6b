// Per-workgroup timestamps of the pass's kernels, for measurement only.
//
// Compiled in only when the library is built with -DTRI_STAMPS (a separate library,
// libtri_stamps.so); in the normal build every TRI_STAMP is empty. Thread 0 of a workgroup writes
// the 100 MHz memory clock (one time base for every CU) at named points into a device buffer the
// caller attaches with tri_stamps_attach: entry [kernel][blockIdx.x][point], as uint64, zero where
// no stamp was written. Each source file that stamps holds its own pointer to the buffer, so no
// device symbol crosses files. Every launch overwrites its kernel's entries: after a stream of
// passes the buffer holds the last pass.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tri {
namespace stamps {

constexpr int kWgs = 4096;   // workgroups stamped per kernel (blockIdx.x below this)
constexpr int kPoints = 8;   // points per workgroup
enum Kernel { kScore = 0, kCand = 1, kFinish = 2, kKernels = 3 };
// points of finish_kernel
enum FinishPoint { kFinStart = 0, kFinLoads = 1, kFinResolved = 2, kFinListed = 3, kFinPlaced = 4, kFinEnd = 5 };

}  // namespace stamps
}  // namespace tri

#ifdef TRI_STAMPS
// The buffer pointer of this source file, and the host call that sets it.
#define TRI_STAMPS_BUFFER(name)                                             \
  __device__ uint64_t* name = nullptr;                                      \
  hipError_t attach_##name(void* p) {                                       \
    return hipMemcpyToSymbol(HIP_SYMBOL(name), &p, sizeof(p), 0, hipMemcpyHostToDevice); \
  }
#define TRI_STAMP(buf, kernel, point)                                                                        \
  do {                                                                                                       \
    uint64_t* tri_stamp_b_ = (buf);                                                                         \
    if (threadIdx.x == 0 && tri_stamp_b_ != nullptr && blockIdx.x < (unsigned)::tri::stamps::kWgs)           \
      tri_stamp_b_[((size_t)(kernel) * ::tri::stamps::kWgs + blockIdx.x) * ::tri::stamps::kPoints + (point)] = \
          __builtin_amdgcn_s_memrealtime();                                                                  \
  } while (0)
#else
#define TRI_STAMPS_BUFFER(name)
#define TRI_STAMP(buf, kernel, point) ((void)0)
#endif
