/*
 * retention_calib.h -- measurement helpers exported by libretention.so.
 *
 * These are not steps of the retention method: they are the two plain
 * kernels against which the method's kernels are measured on the machine at
 * hand (a streaming copy for the HBM ceiling, a loop of fp16 MFMAs for the
 * matrix-core ceiling).  Conventions as in retention.h: device buffers belong
 * to the caller, work is enqueued on `stream`, arguments are validated before
 * any HIP call and a ret_status is returned (retention_last_error() gives the
 * message).
 */
#ifndef RETENTION_CALIB_H
#define RETENTION_CALIB_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ret_calib_copy -- dst[i] = src[i] for n16 16-byte words: every byte of src
 * is read once and every byte of dst written once, with 16-byte non-temporal
 * loads and stores, eight in flight per thread.  src and dst are device
 * pointers, 16-byte aligned, non-overlapping; n16 >= 1.
 */
int ret_calib_copy(const void* src, void* dst, size_t n16, hipStream_t stream);

/*
 * ret_calib_mfma -- `blocks` workgroups of four waves; each wave runs `iters`
 * rounds of four independent v_mfma_f32_32x32x16_f16 on register operands
 * (2 * 32 * 32 * 16 = 32768 flop each), then writes one float per lane to
 * out (device, blocks * 256 floats) so that no product is dead.  Flops
 * executed: blocks * 4 * iters * 4 * 32768.  blocks >= 1, iters >= 1.
 */
int ret_calib_mfma(float* out, int blocks, int iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* RETENTION_CALIB_H */
