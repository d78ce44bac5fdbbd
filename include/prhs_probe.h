/*
 * prhs_probe.h -- measurement aid shipped beside the PrHS decode library.
 *
 * Not part of the method: a plain streaming-read kernel that gives the HBM
 * read ceiling the decode kernels are compared against (all of their HBM
 * traffic is reads of K and V rows). It reads every byte of a device buffer
 * once with 16-byte non-temporal loads over a grid-stride loop and folds the
 * words into a value that is written to `sink` only if it equals a fixed
 * sentinel, so the loads stay live without adding write traffic.
 */
#ifndef PRHS_PROBE_H
#define PRHS_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of device memory at `buf` once, on `stream`.
 *   buf   device pointer, 16-byte aligned, caller-owned, read only
 *   bytes > 0 and a multiple of 16
 *   sink  device pointer to one uint32 (written only on the sentinel value)
 * Returns PRHS_OK (0), PRHS_E_NULL for a NULL pointer, PRHS_E_ALIGN for a
 * misaligned buf, PRHS_E_DIMS for a bad size, PRHS_E_HIP if the launch fails;
 * validation happens before any launch. */
int prhs_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PRHS_PROBE_H */
