/*
 * oracle.c -- plain, slow, CPU reference for the weight-quantized GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library. The product path never
 * calls it, and it shares no code, header, table or helper with the HIP
 * library: it is written from the pages' definitions alone.
 *
 * What it computes (the plain definition, so the oracle *is* the definition):
 *   C[m][n] = sum_k A[m][k] * B[k][n]          (MNN GemmSpeed benchmark page,
 *   section "Why Conv1x1 is used to measure GEMM": the LLM linear layer is
 *   C = A[M,K] x B[K,N]; the weight has shape {ic, oc} = {K, N}).
 * For the quantised formats B[k][n] is the dequantised weight
 *   w = offset + scale * q                     (same section: asymmetric
 *   quantisation, Int8-Block0 = 8 bit with one block over all of K,
 *   Int4-Block64 = 4 bit with one [offset, scale] group per 64 K-elements,
 *   pairs stored as oc x blockNum groups of [offset, scale]).
 * W4A8 (section "Test cases and registration", mode 3): per-channel int4
 * weights unpacked to int8, activations dynamically quantised to int8, an
 * s8 x s8 -> s32 product, then rescaled.
 *
 * Arithmetic: every product and sum in IEEE double, k strictly increasing,
 * no fused multiply-add (built with -ffp-contract=off, never -ffast-math).
 * The W4A8 activation quantisation is done in IEEE single precision because
 * that is the precision of the step it mirrors (row scale kept as fp32).
 * Loops are parallel only over independent outputs (OpenMP).
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - q is unsigned, q in [0, 2^bits - 1], w = offset + scale*q;
 *   - pair order is [offset, scale];
 *   - canonical code storage: Int8 q as bytes [N][K]; Int4 q as bytes
 *     [N][K/2] with byte j = q[2j] | q[2j+1] << 4 (low nibble first, along K);
 *   - quantiser: offset = block minimum, scale = (max - min) / (2^bits - 1)
 *     computed in double and stored as float; q = rint((w - offset)/scale)
 *     in double from the stored float pair, clamped; a constant block gets
 *     scale = 0 and q = 0;
 *   - W4A8 activations: per row amax = max |a|, sa = amax / 127 (fp32),
 *     qa = clamp(rint(a / sa), -127, 127) with fp32 correctly rounded
 *     division and round-half-to-even; an all-zero row gives sa = 0, qa = 0;
 *     the int4 code is zero-extended to int8 (q in [0, 15]).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD 1

/* IEEE binary16 -> double, from the format's definition: sign bit, 5-bit
 * exponent with bias 15, 10-bit fraction; exponent 0 encodes subnormals
 * (fraction * 2^-24), exponent 31 encodes inf / NaN. */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 31;
    int frac = h & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

/* One code of a canonical weight buffer. bits = 8: byte [n][k];
 * bits = 4: nibble (k & 1) of byte [n][k/2], low nibble first. */
static int code_at(const uint8_t *q, int K, int bits, int n, int k)
{
    if (bits == 8)
        return q[(size_t)n * K + k];
    uint8_t byte = q[(size_t)n * (K / 2) + k / 2];
    return (k & 1) ? (byte >> 4) : (byte & 15);
}

/*
 * Quantise float weights W [N][K] into canonical codes and [offset, scale]
 * pairs (pairs [N][K/block][2]). bits is 4 or 8, block divides K; for bits = 4
 * K must be even. q must hold N*K bytes (bits 8) or N*K/2 bytes (bits 4).
 */
int orc_quantize(int N, int K, int bits, int block, const float *W,
                 uint8_t *q, float *pairs)
{
    if (N <= 0 || K <= 0 || block <= 0 || K % block != 0)
        return ORC_BAD;
    if (bits != 4 && bits != 8)
        return ORC_BAD;
    if (bits == 4 && K % 2 != 0)
        return ORC_BAD;
    const int nblk = K / block;
    const int qmax = (1 << bits) - 1;
    if (bits == 4)
        memset(q, 0, (size_t)N * (K / 2));
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        for (int b = 0; b < nblk; ++b) {
            const float *wb = W + (size_t)n * K + (size_t)b * block;
            double lo = wb[0], hi = wb[0];
            for (int i = 1; i < block; ++i) {
                if (wb[i] < lo) lo = wb[i];
                if (wb[i] > hi) hi = wb[i];
            }
            float offset = (float)lo;
            float scale = (float)((hi - lo) / (double)qmax);
            pairs[((size_t)n * nblk + b) * 2 + 0] = offset;
            pairs[((size_t)n * nblk + b) * 2 + 1] = scale;
            for (int i = 0; i < block; ++i) {
                int code = 0;
                if (scale != 0.0f) {
                    double t = ((double)wb[i] - (double)offset) / (double)scale;
                    double r = rint(t);
                    if (r < 0.0) r = 0.0;
                    if (r > (double)qmax) r = (double)qmax;
                    code = (int)r;
                }
                int k = b * block + i;
                if (bits == 8)
                    q[(size_t)n * K + k] = (uint8_t)code;
                else
                    q[(size_t)n * (K / 2) + k / 2] |= (uint8_t)(code << (4 * (k & 1)));
            }
        }
    }
    return ORC_OK;
}

/* Dequantised weight of channel n at k: offset + scale * q, in double. */
static double dequant(const uint8_t *q, const float *pairs, int K, int bits,
                      int block, int n, int k)
{
    const int nblk = K / block;
    const int b = k / block;
    double offset = pairs[((size_t)n * nblk + b) * 2 + 0];
    double scale = pairs[((size_t)n * nblk + b) * 2 + 1];
    return offset + scale * (double)code_at(q, K, bits, n, k);
}

/* fp32 GEMM: A fp32 [M][K], B fp32 [K][N] -> C double [M][N]. */
int orc_gemm_f32(int M, int K, int N, const float *A, const float *B, double *C)
{
    if (M < 0 || K < 0 || N < 0)
        return ORC_BAD;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += (double)A[(size_t)m * K + k] * (double)B[(size_t)k * N + n];
            C[(size_t)m * N + n] = acc;
        }
    return ORC_OK;
}

/*
 * Dequantise-then-multiply for a block-quantised weight: A fp16 bits [M][K],
 * canonical codes q, pairs [N][K/block][2] -> C double [M][N].
 * bits = 8, block = K is Int8-Block0; bits = 4, block = 64 is Int4-Block64.
 */
int orc_gemm_blockq(int M, int K, int N, int bits, int block,
                    const uint16_t *A, const uint8_t *q, const float *pairs,
                    double *C)
{
    if (M < 0 || K <= 0 || N < 0 || block <= 0 || K % block != 0)
        return ORC_BAD;
    if (bits != 4 && bits != 8)
        return ORC_BAD;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += orc_half_to_double(A[(size_t)m * K + k]) *
                       dequant(q, pairs, K, bits, block, n, k);
            C[(size_t)m * N + n] = acc;
        }
    return ORC_OK;
}

/*
 * W4A8 step 1, dynamic per-row activation quantisation, in IEEE fp32:
 * A fp16 bits [M][K] -> qa int8 [M][K], sa float [M], S int32 [M] (row sums
 * of qa).
 */
int orc_w4a8_actquant(int M, int K, const uint16_t *A, int8_t *qa, float *sa,
                      int32_t *S)
{
    if (M < 0 || K <= 0)
        return ORC_BAD;
    #pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m) {
        const uint16_t *row = A + (size_t)m * K;
        float amax = 0.0f;
        for (int k = 0; k < K; ++k) {
            float a = (float)orc_half_to_double(row[k]);   /* exact */
            float mag = a < 0.0f ? -a : a;
            if (mag > amax) amax = mag;
        }
        int32_t sum = 0;
        if (amax == 0.0f) {
            sa[m] = 0.0f;
            for (int k = 0; k < K; ++k)
                qa[(size_t)m * K + k] = 0;
        } else {
            float s = amax / 127.0f;            /* one fp32 rounding */
            sa[m] = s;
            for (int k = 0; k < K; ++k) {
                float a = (float)orc_half_to_double(row[k]);
                float t = a / s;                 /* one fp32 rounding */
                float r = rintf(t);              /* ties to even */
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                qa[(size_t)m * K + k] = (int8_t)r;
                sum += (int32_t)r;
            }
        }
        S[m] = sum;
    }
    return ORC_OK;
}

/*
 * W4A8 step 2, the exact integer product D[m][n] = sum_k qa[m][k] * q[n][k]
 * with q the zero-extended int4 code of the canonical nibble buffer
 * [N][K/2]. Accumulated in int64.
 */
int orc_w4a8_dot(int M, int K, int N, const int8_t *qa, const uint8_t *q,
                 int64_t *D)
{
    if (M < 0 || K <= 0 || N < 0 || K % 2 != 0)
        return ORC_BAD;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int k = 0; k < K; ++k)
                acc += (int64_t)qa[(size_t)m * K + k] * (int64_t)code_at(q, K, 4, n, k);
            D[(size_t)m * N + n] = acc;
        }
    return ORC_OK;
}

/*
 * W4A8 step 3, the rescale: C = sa_m * (scale_n * D + offset_n * S_m) in
 * double, with pairs [N][1][2] (blockSize = K, one pair per channel). This is
 * sum_k (sa_m*qa) * (offset_n + scale_n*q) regrouped.
 */
int orc_w4a8_rescale(int M, int N, const int64_t *D, const float *sa,
                     const int32_t *S, const float *pairs, double *C)
{
    if (M < 0 || N < 0)
        return ORC_BAD;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double offset = pairs[(size_t)n * 2 + 0];
            double scale = pairs[(size_t)n * 2 + 1];
            C[(size_t)m * N + n] = (double)sa[m] *
                (scale * (double)D[(size_t)m * N + n] + offset * (double)S[m]);
        }
    return ORC_OK;
}

/*
 * W4A8 the long way round, as a self-check of the regrouping: dequantise
 * both operands and multiply, sum_k (sa_m*qa[m][k]) * (offset_n + scale_n*q).
 */
int orc_w4a8_dequant_product(int M, int K, int N, const int8_t *qa,
                             const float *sa, const uint8_t *q,
                             const float *pairs, double *C)
{
    if (M < 0 || K <= 0 || N < 0 || K % 2 != 0)
        return ORC_BAD;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                double a = (double)sa[m] * (double)qa[(size_t)m * K + k];
                acc += a * dequant(q, pairs, K, 4, K, n, k);
            }
            C[(size_t)m * N + n] = acc;
        }
    return ORC_OK;
}

/*
 * The fused epilogue of the SimdPaddleOCR pull request (the GEMM keeps its
 * accumulators wide until bias, residual and activation are applied), as
 * the plain definition in double, in the order the pull request names them:
 *   out[m][n] = act(P[m][n] + bias[n] + residual[m][n])
 * act 0: identity; 1: ReLU, max(x, 0); 2: SiLU, x * sigma(x) with
 * sigma(x) = 1 / (1 + e^-x); 3: GELU, x * Phi(x) with Phi the standard
 * normal distribution function, Phi(x) = (1 + erf(x / sqrt(2))) / 2.
 * bias (float [N]) may be NULL; the residual is float [M][N] (res_f32) or
 * fp16 bits [M][N] (res_f16), or neither.
 */
static double act_apply(double x, int act)
{
    switch (act) {
    case 1: return x > 0.0 ? x : 0.0;
    case 2: return x / (1.0 + exp(-x));
    case 3: return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
    default: return x;
    }
}

int orc_epilogue(int M, int N, const double *P, const float *bias, const float *res_f32,
                 const uint16_t *res_f16, int act, double *out)
{
    if (M < 0 || N < 0 || act < 0 || act > 3 || (res_f32 && res_f16))
        return ORC_BAD;
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            const size_t i = (size_t)m * N + n;
            double v = P[i];
            if (bias) v += (double)bias[n];
            if (res_f32) v += (double)res_f32[i];
            if (res_f16) v += orc_half_to_double(res_f16[i]);
            out[i] = act_apply(v, act);
        }
    return ORC_OK;
}

/*
 * The value of x rounded to IEEE binary16 (round to nearest, ties to even;
 * magnitudes that round past the largest finite value 65504 become
 * infinite; the subnormal step is 2^-24), returned as a double. Written
 * from the format's definition: 11 significant bits down to 2^-14, a fixed
 * quantum of 2^-24 below it.
 */
double orc_round_half(double x)
{
    if (isnan(x) || isinf(x) || x == 0.0)
        return x;
    const double ax = fabs(x);
    int e;
    frexp(ax, &e);                        /* ax = f * 2^e, f in [0.5, 1) */
    const int exp2 = e - 1;               /* ax in [2^exp2, 2^(exp2+1)) */
    const double quantum = exp2 < -14 ? ldexp(1.0, -24) : ldexp(1.0, exp2 - 10);
    const double r = nearbyint(ax / quantum) * quantum;   /* exact scaling; ties to even */
    const double y = r > 65504.0 ? INFINITY : r;
    return x < 0 ? -y : y;
}
