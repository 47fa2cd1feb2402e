/*
 * moe_peaks.h -- C ABI of two measurement kernels for MI355X (gfx950): the
 * sustainable rates that the layer's kernels are rated against beside the
 * datasheet peaks.
 *
 * "Optimizing on-device inference for Apple Silicon" (Perplexity 2026),
 * section "Limits of further optimization", rates the MoE GEMM and the
 * sparse GEMV against the fastest sustainable weight-read rate for their
 * access pattern and the prefill matmul against the matrix units' limit.
 * These two kernels measure the corresponding rates on this chip:
 *   - a plain streaming read of a device buffer (16-byte loads, every byte
 *     read once, nothing written but one word per workgroup), whose rate for
 *     a buffer far larger than the last-level cache is the sustainable HBM
 *     read rate;
 *   - a loop of independent bf16 matrix-core products (32x32x16, fp32
 *     accumulation) on register operands on every SIMD of every compute
 *     unit, whose rate is the sustainable dense bf16 MFMA rate.
 *
 * Conventions as in moe_layer.h: device pointers owned by the caller, work
 * enqueued on `stream`, no allocation, no synchronisation; arguments are
 * checked first and a failed check returns 1 (2 for a failed launch) with
 * nothing enqueued.
 */
#ifndef MOE_PEAKS_H
#define MOE_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

/* Reads bytes of buf (16-byte aligned, bytes % 16 == 0, bytes > 0) once;
 * writes one 32-bit word per workgroup to sink[0 .. moe_peak_stream_blocks())
 * (the XOR of what the workgroup read, so the reads cannot be dropped). */
int moe_peak_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Workgroups the stream read launches (the length sink must have). */
int moe_peak_stream_blocks(void);

/* Runs iters (>= 1) iterations of 8 independent 32x32x16 bf16 MFMAs on each
 * of 8 waves per compute unit (two per SIMD) of `cus` workgroups (one per
 * compute unit: pass the device's compute-unit count); writes one float per
 * wave to sink[0 .. cus*8).  FLOPs = cus * 8 * iters * 8 * 32*32*16*2. */
int moe_peak_mfma_loop(int cus, int iters, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PEAKS_H */
