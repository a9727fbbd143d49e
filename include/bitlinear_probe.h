/*
 * bitlinear_probe.h -- attainable-peak probes for the BitLinear benchmark.
 *
 * A separate library (libbitlinear_probe.so), not part of the BitLinear ABI in
 * bitlinear.h: plain kernels that measure what the GPU delivers to simple
 * code, reported by the benchmark beside the published MI355X peaks (8 TB/s
 * HBM3E, 5 POPS dense INT8, 2.5 PFLOP/s dense bf16) that the roofline
 * fractions use.
 *
 * Pointers are device pointers owned by the caller; `stream` is a hipStream_t
 * passed as void*; calls only enqueue work.  Arguments are checked on the host
 * before anything is launched.
 */
#ifndef BITLINEAR_PROBE_H
#define BITLINEAR_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITLINEAR_PROBE_OK         0
#define BITLINEAR_PROBE_ERR_NULL  -1 /* a required pointer is NULL          */
#define BITLINEAR_PROBE_ERR_SHAPE -2 /* a size is out of the accepted range */
#define BITLINEAR_PROBE_ERR_ALIGN -4 /* a pointer is not aligned            */
#define BITLINEAR_PROBE_ERR_HIP   -6 /* the kernel launch failed            */

/*
 * `blocks` 256-thread workgroups each stream one contiguous slice of
 * `bytes` / `blocks` bytes from src with 16-byte streaming loads (eight per
 * lane in flight, one KiB per wave per load).  dst != NULL: the slices are
 * copied to dst (`bytes` written); else each thread folds what it read into
 * one word of out (blocks * 256 uint32).
 * Requires bytes a multiple of 32768 * blocks, bytes / blocks < 2^31,
 * 1 <= blocks <= 2^20; src and dst 16-byte aligned, out 4-byte aligned.
 */
int bitlinear_probe_stream(const void* src, void* dst, int64_t bytes, int blocks, uint32_t* out,
                           void* stream);

/*
 * `blocks` 256-thread workgroups (two per CU), each wave issuing 8 * iters
 * v_mfma_i32_32x32x32_i8 (65536 operations each) on eight independent
 * register accumulators, no memory traffic; each thread writes one word of
 * out (blocks * 256 int32).  Operations per call:
 * blocks * 4 * 8 * iters * 65536.  Requires iters >= 1, 1 <= blocks <= 2^20.
 */
int bitlinear_probe_mfma_i8(int iters, int blocks, int32_t* out, void* stream);

/*
 * The same with v_mfma_f32_32x32x16_bf16 (32768 floating-point operations
 * each) on eight independent float32 accumulators, against the 2.5 PFLOP/s
 * dense bf16 peak; operands are small integers, so `out` (blocks * 256 float)
 * is exact and the same on every call.  Operations per call:
 * blocks * 4 * 8 * iters * 32768.  Requires 1 <= iters <= 2^20,
 * 1 <= blocks <= 2^20.
 */
int bitlinear_probe_mfma_bf16(int iters, int blocks, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_PROBE_H */
