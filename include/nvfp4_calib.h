/*
 * nvfp4_calib.h - C ABI of libnvfp4_calib.so, the bandwidth calibration
 * kernels used by the benchmark (not part of the NVFP4 path itself).
 *
 * The functions take DEVICE pointers, allocate nothing, never synchronize
 * and enqueue one kernel on `stream` (NULL = default stream). `blocks` is the
 * number of 256-thread workgroups (grid-stride loops cover any size).
 * Return: 0 success, 1 invalid argument (negative size, size not a multiple
 * of 16 (of 4096 for the mix), blocks < 1, LDS bytes outside [0, 65536],
 * pointer not 16-byte aligned; checked before any HIP call), 4 launch
 * failure (hipGetLastError()).
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

/* The fused quantize kernel's traffic mix without its compute: for every
 * 4096-byte tile of src (`bytes`, a multiple of 4096) write 576 bytes of dst
 * (dst holds bytes / 4096 * 576 bytes), one tile per wave. `lds_bytes` of
 * unused dynamic LDS per 256-thread workgroup cap the workgroups per CU. */
int nvfp4_calib_mix(const void *src, void *dst, int64_t bytes, int32_t lds_bytes,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_CALIB_H */
