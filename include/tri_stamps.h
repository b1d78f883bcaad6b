/* tri_stamps.h - per-workgroup timestamps of the pass's kernels, for measuring where a pass's
 * time goes. These two calls exist only in libtri_stamps.so, the library built with
 * -DTRI_STAMPS (python -m rotary_frequency_key_amd.build --stamps); libtri.so does not export
 * them, and its kernels carry no stamps.
 *
 * In that build, thread 0 of each workgroup of the score kernel, the candidate kernel and the
 * finish kernel (the arrangement of a one-layer pass, tri_prune_pass) writes the 100 MHz memory
 * clock, one time base for every CU, into an attached device buffer at named points:
 *     buf[(kernel * wgs + blockIdx.x) * points + point]    (uint64)
 * with kernel 0 the score kernel (points 0 start, 1 end), 1 the candidate kernel (0 start,
 * 1 end), 2 the finish kernel (0 start, 1 first loads used, 2 threshold and per-granule counts
 * resolved, 3 granules listed, 4 kept rows placed, 5 end). Workgroups with blockIdx.x >= wgs,
 * and points a workgroup does not reach (it returns early), are not written. Every launch
 * overwrites its kernel's entries, so after a stream of passes the buffer holds the last one.
 * A stamp costs one memory-clock read and one store by one thread: differences of about a
 * microsecond and more are meaningful.
 */
#ifndef TRI_STAMPS_H
#define TRI_STAMPS_H

#ifdef __cplusplus
extern "C" {
#endif

/* The buffer's shape: workgroups per kernel, points per workgroup, kernels. Always TRI_OK. */
int tri_stamps_layout(int* wgs, int* points, int* kernels);

/* Attach a device buffer of kernels * wgs * points uint64 (caller-owned, zeroed by the caller;
 * NULL detaches). Synchronous with respect to the host; call it outside graph capture, between
 * passes. Returns TRI_OK, or TRI_ERR_HIP when the runtime fails to set the device pointer. */
int tri_stamps_attach(void* buf);

#ifdef __cplusplus
}
#endif

#endif /* TRI_STAMPS_H */
