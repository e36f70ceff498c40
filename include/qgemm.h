/*
 * qgemm.h -- C ABI of libqgemm, the weight-quantized GEMM for AMD MI355X
 * (gfx950 / CDNA4).
 *
 * The one operation (MNN GemmSpeed benchmark page, section "Why Conv1x1 is
 * used to measure GEMM"): an LLM linear layer C = A[M,K] x B[K,N], where the
 * weight B is held in one of the page's formats:
 *
 *   QGEMM_F32       float weights (page mode 0, "float-gemm"); fp32 A, B, C.
 *   QGEMM_INT4_B64  Int4-Block64 (mode 1, "int4b64-gemm"): 4-bit codes, one
 *                   [offset, scale] pair per 64 K-elements per output
 *                   channel, w = offset + scale * q.
 *   QGEMM_INT8_B0   Int8-Block0 (mode 2, "int8b0-gemm"): 8-bit codes, one
 *                   pair per output channel (blockSize = K).
 *   QGEMM_W4A8      Int4-Block0 W4A8 (mode 3, section "Test cases and
 *                   registration"): 4-bit per-channel codes unpacked to
 *                   int8; each row of A is quantised on the fly to int8; the
 *                   product is s8 x s8 -> s32, exact, then rescaled to fp32.
 *   QGEMM_F16       fp16 weights: the float mode at FP16 precision, as the
 *                   page ran it (section "Sample data"); fp16 A and B, fp32
 *                   accumulation, fp32 C.
 *   QGEMM_INT4_B0   Int4-Block0 without A8: W4A8's per-channel 4-bit weights
 *                   with fp16 activations (no activation quantisation);
 *                   K % 64 == 0.
 *   QGEMM_INT4_BLOCK(b)  Int4 with one pair per b K-elements (the page's
 *                   blockSize parameter, section "Why Conv1x1 is used to
 *                   measure GEMM"), b a multiple of 16 that divides K, and
 *                   K % 64 == 0; fp16 activations.
 *                   QGEMM_INT4_BLOCK(64) behaves as QGEMM_INT4_B64 and
 *                   QGEMM_INT4_BLOCK(K) as QGEMM_INT4_B0.
 *   QGEMM_INT8_BLOCK(b)  Int8 (codes 0..255) with one pair per b K-elements,
 *                   b a multiple of 16 that divides K, and K % 64 == 0;
 *                   fp16 activations. Canonical codes are u8
 *                   [N][K] as for QGEMM_INT8_B0, pairs [N][K/b][2].
 *
 * Format ids 0-3 equal the page's mode numbers. For every format but F32, A
 * is fp16; C is fp32 (or fp16 through qgemm_run_ex).
 *
 * Canonical (user-facing) weight layouts, on the host:
 *   - F32:      B float [K][N] row-major (the page's weight shape {ic, oc}).
 *   - F16:      B fp16 [K][N] row-major, as F32.
 *   - INT8_B0:  q uint8 [N][K]; pairs float [N][1][2] = {offset, scale}.
 *   - INT4_B64: q uint8 [N][K/2], byte j of a row = q[2j] | q[2j+1] << 4
 *               (two codes per byte along K, low nibble first);
 *               pairs float [N][K/64][2] = {offset, scale} (the page: oc x
 *               blockNum groups of [offset, scale]).
 *   - W4A8, INT4_B0: q as INT4_B64 with one block over all of K; pairs
 *               float [N][1][2].
 *   - INT4_BLOCK(b): q as INT4_B64; pairs float [N][K/b][2].
 * Codes are unsigned: q in [0, 2^bits - 1].
 *
 * Packed (device) layouts are opaque and owned by this library: they are
 * produced by qgemm_pack_weights on the host, copied to device memory by the
 * caller, and consumed by qgemm_run. They are padded (channels to a multiple
 * of 4 or 32, K to the kernels' step) with zero codes and zero pairs.
 *
 * Conventions shared by every function:
 *   - Return a qgemm_status; nothing aborts, throws, prints or exits.
 *   - Every argument is checked before anything is enqueued on the GPU; a
 *     rejected call has no effect.
 *   - Shapes are ints; M, N >= 0, K >= 0. M == 0 or N == 0 is a valid empty
 *     product: OK, nothing is read or written, pointers are not inspected.
 *   - Device pointers must be 16-byte aligned (torch allocations are).
 *   - The caller owns every buffer. qgemm_run keeps no pointer after it
 *     returns, but the GPU reads and writes the buffers asynchronously until
 *     the stream reaches that point: keep them alive until then.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream. Faults during execution surface at the caller's next
 *     synchronisation with the stream (ordinary HIP semantics).
 *   - Functions are thread-safe: the only global state is the dispatch
 *     threshold (an atomic) and the per-process HIP module state.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QGEMM_ABI_VERSION 1

typedef enum qgemm_format {
    QGEMM_F32 = 0,
    QGEMM_INT4_B64 = 1,
    QGEMM_INT8_B0 = 2,
    QGEMM_W4A8 = 3,
    QGEMM_F16 = 4,
    QGEMM_INT4_B0 = 5,
    QGEMM_INT4_BLOCK_BASE = 0x10000,  /* + b: see QGEMM_INT4_BLOCK */
    QGEMM_INT8_BLOCK_BASE = 0x2000000 /* + b: see QGEMM_INT8_BLOCK */
} qgemm_format;

/* Format id of Int4 weights with one pair per b K-elements. */
#define QGEMM_INT4_BLOCK(b) ((qgemm_format)(QGEMM_INT4_BLOCK_BASE + (b)))
/* Format id of Int8 weights (codes 0..255, fp16 activations) with one pair
 * per b K-elements: the blockSize parameter of the GemmSpeed page ("Why
 * Conv1x1 is used to measure GEMM") applied to 8-bit codes. b is a multiple
 * of 16 that divides K, and K % 64 == 0 (else ERR_FORMAT / ERR_SHAPE). */
#define QGEMM_INT8_BLOCK(b) ((qgemm_format)(QGEMM_INT8_BLOCK_BASE + (b)))

typedef enum qgemm_status {
    QGEMM_OK = 0,
    QGEMM_ERR_NULL = 1,     /* a required pointer is NULL                     */
    QGEMM_ERR_SHAPE = 2,    /* a shape is negative, too large, or violates the
                               format's block rule (INT4_B64: K % 64 == 0;
                               INT4/W4A8: K even; quantised formats: K > 0)   */
    QGEMM_ERR_FORMAT = 3,   /* unknown format, or an operation the format does
                               not have (e.g. quantising to F32)              */
    QGEMM_ERR_ALIGN = 4,    /* a device pointer is not 16-byte aligned        */
    QGEMM_ERR_NOMEM = 5,    /* the library could not allocate its scratch     */
    QGEMM_ERR_DEVICE = 6,   /* no usable HIP device                           */
    QGEMM_ERR_LAUNCH = 7,   /* the HIP runtime rejected a kernel launch       */
    QGEMM_ERR_SIZE = 8,     /* a caller buffer is smaller than required       */
    QGEMM_ERR_VALUE = 9     /* non-finite input to the quantiser              */
} qgemm_status;

/* Human-readable name of a status; never NULL. */
const char *qgemm_status_string(int status);

/* QGEMM_ABI_VERSION of the built library. */
int qgemm_abi_version(void);

/*
 * Sizes of the canonical buffers of a format: q_bytes for the codes (or the
 * fp32 B for F32) and pair_floats for the [offset, scale] pairs (0 for F32).
 * Errors: ERR_NULL, ERR_FORMAT, ERR_SHAPE.
 */
qgemm_status qgemm_canonical_size(int K, int N, qgemm_format f,
                                  size_t *q_bytes, size_t *pair_floats);

/*
 * Host-side quantiser (the offline export step the page attributes to
 * mnnconvert; MNN GemmSpeed page, section "Why Conv1x1 is used to measure
 * GEMM": asymmetric quantisation with [offset, scale] pairs).
 * W: host float [N][K] (one row per output channel). For each (channel,
 * block): offset = minimum, scale = (maximum - minimum) / (2^bits - 1)
 * computed in double and stored as float, q = rint((w - offset) / scale) in
 * double from the stored pair, clamped to [0, 2^bits - 1]; a constant block
 * gets scale 0 and q 0. Writes the canonical q (q_bytes) and pairs
 * (pair_floats floats), both host memory owned by the caller.
 * Errors: ERR_NULL, ERR_FORMAT (F32 or unknown), ERR_SHAPE, ERR_SIZE,
 * ERR_VALUE (a NaN or infinite weight; nothing useful is written then).
 */
qgemm_status qgemm_quantize_weights(int K, int N, qgemm_format f,
                                    const float *W, void *q, size_t q_bytes,
                                    float *pairs, size_t pair_floats);

/*
 * Device-side quantiser: the same export step on the GPU (MNN GemmSpeed page,
 * section "Why Conv1x1 is used to measure GEMM"), for weights that already
 * live in device memory. Every step is the host quantiser's, in the same IEEE
 * double operations, so codes and pairs equal qgemm_quantize_weights' bit for
 * bit; of equal extremes (+0 and -0) the first in k order is kept, as a
 * sequential scan keeps it.
 *   W      device float [N][K], read-only.
 *   q      device, canonical codes (qgemm_canonical_size's q_bytes).
 *   pairs  device, canonical pairs [N][nblk][2] (pair_floats floats).
 * Enqueued on `stream`; returns without waiting. The device cannot report a
 * NaN or infinite weight before it runs, so instead of ERR_VALUE the block
 * (the channel, for the per-channel formats) that holds one gets NaN offset
 * and scale and zero codes.
 * Errors: ERR_FORMAT (F32, F16, unknown, and INT4_BLOCK(b) / INT8_BLOCK(b)
 * with b other than 16, 32 or a multiple of 64: blocks that straddle the
 * quantiser's 64-element steps; quantise those with qgemm_quantize_weights),
 * ERR_SHAPE, ERR_NULL, ERR_ALIGN (a pointer not 16-byte aligned), ERR_DEVICE,
 * ERR_LAUNCH. N == 0 is a no-op.
 */
qgemm_status qgemm_quantize_weights_device(int K, int N, qgemm_format f, const float *W,
                                           void *q, float *pairs, void *stream);

/*
 * Device-side quantise-and-pack: as qgemm_quantize_weights_device, but the
 * codes and pairs go straight into the packed layouts qgemm_run reads (Bq
 * and scales of qgemm_packed_size's w_bytes / s_bytes, every byte written,
 * padding as zeros), byte-identical to qgemm_pack_weights of the canonical
 * result. Same arguments, errors and non-finite handling.
 */
qgemm_status qgemm_quantize_pack_device(int K, int N, qgemm_format f, const float *W,
                                        void *Bq, void *scales, void *stream);

/*
 * Sizes in bytes of the packed weight buffer (w_bytes) and the packed pair
 * buffer (s_bytes, 0 for F32) of a K x N weight.
 * Errors: ERR_NULL, ERR_FORMAT, ERR_SHAPE.
 */
qgemm_status qgemm_packed_size(int K, int N, qgemm_format f,
                               size_t *w_bytes, size_t *s_bytes);

/*
 * Host-side packer: canonical layout -> the library's device layout. Pure
 * byte/nibble permutation plus zero padding; no value changes (the
 * LLM-on-PowerVR page, section 2, re-lays weights out offline into the
 * order its kernel fetches them in; this packer does the same for gfx950).
 * w_canonical / pairs_canonical: host, read-only, canonical layouts above
 * (pairs_canonical ignored and may be NULL for F32). w_packed / s_packed:
 * host, caller-allocated, at least qgemm_packed_size() bytes; the caller
 * then copies them to device memory.
 * Errors: ERR_NULL, ERR_FORMAT, ERR_SHAPE, ERR_SIZE.
 */
qgemm_status qgemm_pack_weights(int K, int N, qgemm_format f,
                                const void *w_canonical,
                                const float *pairs_canonical,
                                void *w_packed, size_t w_bytes,
                                void *s_packed, size_t s_bytes);

/*
 * Inverse of qgemm_pack_weights (host): recovers the canonical buffers from
 * packed ones. Lets a caller check or re-export packed weights.
 * Errors: ERR_NULL, ERR_FORMAT, ERR_SHAPE, ERR_SIZE.
 */
qgemm_status qgemm_unpack_weights(int K, int N, qgemm_format f,
                                  const void *w_packed, size_t w_bytes,
                                  const void *s_packed, size_t s_bytes,
                                  void *w_canonical, float *pairs_canonical);

/*
 * Device scratch qgemm_run_ws may need for this shape; a function of
 * (M, K, N, f) alone. It holds, in order: for W4A8 the quantised
 * activations (int8 [M][K rounded up to 128]), the row scales (float [M])
 * and the row sums of the quantised activations (int32 [M]); then, when the
 * shape leaves too few output tiles (or, for the Int4 and W4A8 GEMVs, too
 * few 32-channel tiles) to fill the GPU and the kernel therefore splits K into S
 * slices, S partial products ([S][M][N], float; int32 for W4A8) that a
 * second kernel adds in the fixed order 0..S-1 (so results are
 * deterministic). The size covers whichever kernel the shape may take. 0
 * for shapes that need neither.
 * Errors: ERR_NULL, ERR_FORMAT, ERR_SHAPE.
 */
qgemm_status qgemm_workspace_size(int M, int K, int N, qgemm_format f,
                                  size_t *bytes);

/*
 * C = A x B on the GPU, enqueued on `stream`; returns without waiting.
 *   A       device, [M][K] row-major: float for F32, fp16 otherwise.
 *   Bq      device, packed weights from qgemm_pack_weights (for F32 the
 *           packed B is the float [K][N] matrix itself, read no further
 *           than its K*N elements).
 *   scales  device, packed pairs; must be NULL for F32.
 *   C       device, float [M][N] row-major, fully overwritten (no alpha or
 *           beta; K == 0 for F32 writes zeros).
 * Dispatch: every quantised format and F16 with M at most the GEMV threshold
 * (default 8), within the format's own crossover (see qgemm_set_gemv_max_m)
 * and K within the GEMV's limit (16384; 8192 for F16) take a streaming GEMV
 * (the page: M = 8 is the narrow, near-decode case, bounded by GEMV
 * bandwidth); other shapes take
 * the tiled MFMA kernels (fp16 MFMA; int8 MFMA for W4A8). W4A8 first runs
 * the activation quantiser. F32 runs the fp32 tiled kernel. Any scratch the shape
 * needs (qgemm_workspace_size) is allocated stream-ordered on `stream`
 * (hipMallocAsync / hipFreeAsync).
 * The buffers' sizes are not visible to the library: the caller guarantees
 * A holds M*K, C M*N elements and Bq / scales qgemm_packed_size() bytes.
 * Errors: ERR_NULL, ERR_FORMAT, ERR_SHAPE, ERR_ALIGN, ERR_DEVICE,
 * ERR_NOMEM, ERR_LAUNCH.
 */
qgemm_status qgemm_run(int M, int K, int N, qgemm_format f, const void *A,
                       const void *Bq, const void *scales, float *C,
                       void *stream);

/*
 * As qgemm_run, with caller-provided device scratch `workspace` (16-byte
 * aligned) of ws_bytes >= qgemm_workspace_size() bytes (may be NULL when
 * that size is 0, or when the call touches none of it: a GEMV of a format
 * other than W4A8 that does not split K). The
 * library allocates nothing. Calls that share a workspace must be ordered
 * (same stream, or synchronised).
 * Errors: as qgemm_run, plus ERR_SIZE for a short workspace.
 */
qgemm_status qgemm_run_ws(int M, int K, int N, qgemm_format f, const void *A,
                          const void *Bq, const void *scales, float *C,
                          void *workspace, size_t ws_bytes, void *stream);

/*
 * Fused epilogue (SimdPaddleOCR pull request, the GEMM change that keeps
 * accumulators in fp32 until bias, residual and activation are applied):
 *
 *   C[m][n] = act(P[m][n] + bias[n] + residual[m][n])
 *
 * with P = A x B the fp32-accumulated product, every step in fp32 in the
 * order written, and C stored once as fp32 or rounded once to fp16 (round
 * to nearest even). Fields:
 *   bias        device, float [N], or NULL (no bias).
 *   residual    device, [M][N] row-major in C's type (float or fp16), or
 *               NULL. It may be the same buffer as C (an in-place residual
 *               update): each element is read before it is written, by the
 *               same thread.
 *   activation  QGEMM_ACT_NONE, _RELU (max(x, 0)), _SILU (x / (1 + e^-x)) or
 *               _GELU (x * Phi(x), Phi the standard normal CDF, via erf).
 *   out_type    QGEMM_OUT_F32: C is float [M][N]; QGEMM_OUT_F16: C is fp16
 *               [M][N].
 * bias and residual must be 16-byte aligned.
 */
typedef enum qgemm_activation {
    QGEMM_ACT_NONE = 0,
    QGEMM_ACT_RELU = 1,
    QGEMM_ACT_SILU = 2,
    QGEMM_ACT_GELU = 3
} qgemm_activation;

typedef enum qgemm_out_type {
    QGEMM_OUT_F32 = 0,
    QGEMM_OUT_F16 = 1
} qgemm_out_type;

typedef struct qgemm_epilogue {
    const float *bias;
    const void *residual;
    int activation;
    int out_type;
} qgemm_epilogue;

/*
 * qgemm_run with a fused epilogue (`epi` may be NULL: none, fp32 C) and an
 * optional caller workspace: with workspace == NULL and ws_bytes == 0 any
 * scratch the shape needs is allocated stream-ordered as in qgemm_run;
 * otherwise it is used as in qgemm_run_ws. C is float or fp16 per
 * epi->out_type. Split-K shapes apply the epilogue once, after their slices
 * are added.
 * Errors: as qgemm_run_ws; ERR_FORMAT for an unknown activation or output
 * type; ERR_ALIGN for misaligned bias or residual.
 */
qgemm_status qgemm_run_ex(int M, int K, int N, qgemm_format f, const void *A,
                          const void *Bq, const void *scales, void *C,
                          const qgemm_epilogue *epi, void *workspace,
                          size_t ws_bytes, void *stream);

/*
 * qgemm_run_ex (fused epilogue, NULL for none) for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation. It calls no hipMalloc, hipFree or other
 * allocating routine. Whatever scratch the shape needs (W4A8 activation
 * codes, split-K partial tiles; qgemm_workspace_size reports it) lives in
 * one fixed array of QGEMM_NOALLOC_SCRATCH_BYTES in each GPU's memory,
 * reserved when the library's code is loaded on that GPU and held until the
 * process ends. Its address is looked up once per device, on the first call
 * on that device.
 *
 * Every call on one GPU shares that array and leaves its contents behind
 * (no call relies on them): calls that may overlap on one GPU (different
 * streams, or different host threads without ordering) race on it and
 * must be serialised by the caller. Calls on different GPUs do not
 * interact.
 *
 * Errors: as qgemm_run_ex, plus QGEMM_ERR_SIZE, checked before anything is
 * enqueued, when the shape needs more scratch than
 * QGEMM_NOALLOC_SCRATCH_BYTES (use qgemm_run_ex with a workspace then).
 */
#define QGEMM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
qgemm_status qgemm_run_noalloc(int M, int K, int N, qgemm_format f, const void *A,
                               const void *Bq, const void *scales, void *C,
                               const qgemm_epilogue *epi, void *stream);

/*
 * W4A8 with its intermediate results exposed, for bit-exact checks of the
 * integer path: the quantised activations qa (int8 [M][K]), the row scales
 * sa (float [M]), the row sums S of qa (int32 [M]) and the exact integer
 * product D (int32 [M][N], D[m][n] = sum_k qa[m][k] * q[n][k]); C as
 * qgemm_run. All device buffers, caller-owned; workspace as qgemm_run_ws.
 * Errors: as qgemm_run_ws.
 */
qgemm_status qgemm_w4a8_debug(int M, int K, int N, const void *A,
                              const void *Bq, const void *scales, float *C,
                              int8_t *qa, float *sa, int32_t *S, int32_t *D,
                              void *workspace, size_t ws_bytes, void *stream);

/*
 * Sets the largest M that may take a GEMV kernel (below it each format keeps
 * its own crossover: Int8 up to 4 rows, the Int4 formats up to 4 rows or up
 * to 8 while M * K * N <= 2^29 (K <= 4096) or 3 * 2^26 (larger K), fp16 and
 * W4A8 up to 8 rows)
 * (0..8; default 8, or the QGEMM_GEMV_MAX_M environment variable read at
 * first use) and returns the previous value; a value outside 0..8 is
 * ignored and only the current value returned. Affects only which kernel
 * runs, never the result beyond rounding.
 */
int qgemm_set_gemv_max_m(int max_m);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
