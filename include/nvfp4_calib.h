/*
 * nvfp4_calib.h - C ABI of libnvfp4_calib.so, the bandwidth calibration
 * kernels used by the benchmark (not part of the NVFP4 path itself).
 *
 * Both functions take DEVICE pointers, allocate nothing, never synchronize
 * and enqueue one kernel on `stream` (NULL = default stream). `blocks` is the
 * number of 256-thread workgroups (grid-stride loops cover any size).
 * Return: 0 success, 1 invalid argument (negative size, size not a multiple
 * of 16, blocks < 1, pointer not 16-byte aligned; checked before any HIP
 * call), 4 launch failure (hipGetLastError()).
 */
#ifndef NVFP4_CALIB_H
#define NVFP4_CALIB_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Copy `bytes` from src to dst (reads and writes `bytes`). */
int nvfp4_calib_copy(const void *src, void *dst, int64_t bytes, int32_t blocks,
                     hipStream_t stream);

/* Read `bytes` from src; write one 16-byte checksum per workgroup to out
 * (out holds `blocks` x 16 bytes). */
int nvfp4_calib_read(const void *src, void *out, int64_t bytes, int32_t blocks,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_CALIB_H */
