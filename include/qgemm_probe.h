/* qgemm_probe.h -- measured-peak probes (libqgemm_probe.so).
 *
 * Diagnostic kernels for the benchmark's peak mode, kept out of libqgemm.so:
 * they compute nothing of the GEMM. The benchmark page (MNN GemmSpeed,
 * section "Sample data") explains small-M results by a bandwidth floor and
 * large-M results by cache behaviour and scheduling; these probes measure
 * those floors on the chip at hand, so the GEMM kernels' roofline fractions
 * (against published peaks) can be read against what plain kernels reach.
 *
 * Conventions: every pointer is a device pointer, `stream` is a hipStream_t
 * (NULL: the default stream). Return 0 on success, 1 for a NULL pointer or a
 * non-positive count, 2 or 3 for an argument out of range (nothing launched),
 * 7 when the launch failed. Calls are asynchronous on `stream`; the caller
 * owns every buffer and keeps it alive until the stream has passed the call.
 */
#ifndef QGEMM_PROBE_H
#define QGEMM_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16) of src once with 16-byte loads (grid
 * workgroups of 256 threads, eight loads in flight per thread) and writes one
 * word per thread to sink (grid * 256 words). */
int qgemm_probe_read(const void *src, size_t bytes, unsigned *sink, int grid, void *stream);

/* Copies `bytes` (a multiple of 16) from src to dst (non-overlapping) with
 * 16-byte loads and stores. */
int qgemm_probe_copy(const void *src, void *dst, size_t bytes, int grid, void *stream);

/* grid workgroups of `waves` waves (1..16), each wave running `iters` turns
 * of four independent 32x32x16 fp16 MFMAs, with valu_per_mfma (0, 4, 8 or
 * 16; else 3) fp32 fused multiply-adds rounded to fp16 issued by the same
 * wave after each MFMA. clk receives, per workgroup b, four words at 4b:
 * shader clock at start and end, 100 MHz reference clock at start and end
 * (wave 0). sink: grid * 64 * waves floats. */
int qgemm_probe_mfma(int iters, int valu_per_mfma, int waves, int grid, unsigned long long *clk,
                     float *sink, void *stream);

/* grid workgroups of `waves` waves (1..8) read, iters x 8 times per thread,
 * 16-byte pieces of the first 2^wbits bytes of buf (2^wbits <= bytes, wbits
 * 12..30), per wave load instruction: pattern 0 one contiguous KiB, pattern 1
 * eight rows of 128 bytes, pattern 2 sixteen rows of 64 bytes, rows `stride`
 * bytes apart (a multiple of 16). clk receives the shader clock at start and
 * end per workgroup (two words at 2b); sink: grid * 64 * waves words. */
int qgemm_probe_l2(const void *buf, size_t bytes, int wbits, int pattern, int stride, int iters,
                   int waves, int grid, unsigned long long *clk, unsigned *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_PROBE_H */
