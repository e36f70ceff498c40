// gemm_f16dq.hip -- prefill GEMM (M above the GEMV threshold) with
// Int4-Block64 / Int8-Block0 weights on the fp16 matrix cores.
//
// What is computed (MNN GemmSpeed benchmark page, section "Why Conv1x1 is
// used to measure GEMM"): C = A x deq(B), deq(B)[k][n] = offset + scale * q.
// The dequantised weight is formed in fp32 (one fused multiply-add from the
// fp32 pair) and rounded once to fp16; A is fp16 already, so the fp16 tiles
// are exact copies of A and the nearest fp16 of each weight. Accumulation is
// fp32 in the MFMA accumulators and C is stored as fp32 (the SimdPaddleOCR
// pull request keeps fp16 shared-memory tiles exact and never narrows the
// accumulators; the pages' tile kernels were written for other GPUs and are
// not followed otherwise).
//
// Tiling: 128 x 64 output tile per 256-thread workgroup, K step 64 (one
// Int4 block, so one pair per channel per step). A and the dequantised B are
// staged in LDS as fp16 rows with K contiguous (B transposed); four waves
// split the tile 2 x 2 and each computes 64 x 32 with
// v_mfma_f32_32x32x16_f16.
#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

namespace {
constexpr int BM = 128, BN = 64, BK = 64;
constexpr int LDS_STRIDE = BK + 8;   // halves; 144-byte rows spread the banks
}

// Dequantise 16 Int4 codes (two 32-bit words, k ascending, low nibble
// first) to 16 fp16 weights w = offset + scale * q, returned as 8 packed
// pairs in k order.
__device__ __forceinline__ void dequant16_int4(u2_t nib, float offset, float scale,
                                               unsigned (&out)[8]) {
    // x = 1024 + q exactly in fp16, so w = x * scale + (offset - 1024 scale).
    const float bias = fmaf(-1024.0f, scale, offset);
#pragma unroll
    for (int wi = 0; wi < 2; ++wi) {
        const unsigned word = nib[wi];
        const h2_t x0 = as_h2((word & 0x000F000Fu) | 0x64006400u);          // q0, q4
        const h2_t x1 = as_h2(((word >> 4) & 0x000F000Fu) | 0x64006400u);   // q1, q5
        const h2_t x2 = as_h2(((word >> 8) & 0x000F000Fu) | 0x64006400u);   // q2, q6
        const h2_t x3 = as_h2(((word >> 12) & 0x000F000Fu) | 0x64006400u);  // q3, q7
        out[wi * 4 + 0] = pack_h2(fmaf((float)x0.x, scale, bias), fmaf((float)x1.x, scale, bias));
        out[wi * 4 + 1] = pack_h2(fmaf((float)x2.x, scale, bias), fmaf((float)x3.x, scale, bias));
        out[wi * 4 + 2] = pack_h2(fmaf((float)x0.y, scale, bias), fmaf((float)x1.y, scale, bias));
        out[wi * 4 + 3] = pack_h2(fmaf((float)x2.y, scale, bias), fmaf((float)x3.y, scale, bias));
    }
}

// Dequantise 16 Int8 codes (four words, k ascending) the same way.
__device__ __forceinline__ void dequant16_int8(u4_t codes, float offset, float scale,
                                               unsigned (&out)[8]) {
    const float bias = fmaf(-1024.0f, scale, offset);
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
        const unsigned word = codes[wi];
        const h2_t x0 = as_h2(__builtin_amdgcn_perm(0x64646464u, word, 0x04010400u));  // q0, q1
        const h2_t x1 = as_h2(__builtin_amdgcn_perm(0x64646464u, word, 0x04030402u));  // q2, q3
        out[wi * 2 + 0] = pack_h2(fmaf((float)x0.x, scale, bias), fmaf((float)x0.y, scale, bias));
        out[wi * 2 + 1] = pack_h2(fmaf((float)x1.x, scale, bias), fmaf((float)x1.y, scale, bias));
    }
}

template <int FMT>
__global__ __launch_bounds__(256) void gemm_f16dq_kernel(
    int M, int K, int N, int Kp, const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ Sp, float *__restrict__ C) {
    __shared__ __align__(16) _Float16 As[BM * LDS_STRIDE];
    __shared__ __align__(16) _Float16 Bs[BN * LDS_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const bool a_vec = (K & 7) == 0;
    const int Np = (N + 3) & ~3;
    const int nblk = Kp >> 6;

    f16_t acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;

    // B loader role: channel n = tid / 4 of the tile, K quarter tid % 4.
    const int bn = tid >> 2, bq = tid & 3;
    const int gn = n0 + bn;

    for (int kt = 0; kt < nblk; ++kt) {
        const int k0 = kt * BK;
        // ---- A tile: 128 rows x 64 halves ----
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = it * 256 + tid;
            const int r = idx >> 3, c8 = (idx & 7) * 8;
            const int gm = m0 + r, gk = k0 + c8;
            u4_t v = {0u, 0u, 0u, 0u};
            if (gm < M) {
                const _Float16 *src = A + (size_t)gm * K + gk;
                if (a_vec) {
                    if (gk < K) v = *reinterpret_cast<const u4_t *>(src);
                } else {
                    h8_t t;
#pragma unroll
                    for (int e = 0; e < 8; ++e) t[e] = (gk + e < K) ? src[e] : (_Float16)0.0f;
                    v = __builtin_bit_cast(u4_t, t);
                }
            }
            *reinterpret_cast<u4_t *>(As + r * LDS_STRIDE + c8) = v;
        }
        // ---- B tile: 64 channels x 64 k, dequantised to fp16 ----
        {
            unsigned w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
            if (gn < Np) {
                if (FMT == QGEMM_INT4_B64) {
                    const int g = gn >> 2, c = gn & 3;
                    const int j = 2 * c + (bq >> 1);
                    const u2_t nib = *reinterpret_cast<const u2_t *>(
                        Wp + (((size_t)g * 8 + j) * nblk + kt) * 16 + (bq & 1) * 8);
                    const f2_t pr = *reinterpret_cast<const f2_t *>(
                        Sp + (((size_t)g * 2 + (c >> 1)) * nblk + kt) * 4 + (c & 1) * 2);
                    dequant16_int4(nib, pr.x, pr.y, w);
                } else {
                    const u4_t codes = *reinterpret_cast<const u4_t *>(
                        Wp + (size_t)gn * Kp + k0 + bq * 16);
                    const f2_t pr = *reinterpret_cast<const f2_t *>(Sp + (size_t)gn * 2);
                    dequant16_int8(codes, pr.x, pr.y, w);
                }
            }
            u4_t *dst = reinterpret_cast<u4_t *>(Bs + bn * LDS_STRIDE + bq * 16);
            dst[0] = u4_t{w[0], w[1], w[2], w[3]};
            dst[1] = u4_t{w[4], w[5], w[6], w[7]};
        }
        __syncthreads();

        // ---- 4 MFMA steps of K = 16 ----
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int kk = s * 16 + (lane >> 5) * 8;
            const h8_t b = *reinterpret_cast<const h8_t *>(
                Bs + (wn * 32 + (lane & 31)) * LDS_STRIDE + kk);
#pragma unroll
            for (int fm = 0; fm < 2; ++fm) {
                const h8_t a = *reinterpret_cast<const h8_t *>(
                    As + (wm * 64 + fm * 32 + (lane & 31)) * LDS_STRIDE + kk);
                acc[fm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[fm], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- epilogue: 32x32 accumulator layout, row 8(j/4) + 4(lane/32) + j%4 ----
    const int col = n0 + wn * 32 + (lane & 31);
    if (col < N) {
#pragma unroll
        for (int fm = 0; fm < 2; ++fm) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int row = m0 + wm * 64 + fm * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
                if (row < M) C[(size_t)row * N + col] = acc[fm][j];
            }
        }
    }
}

template <int FMT>
static hipError_t launch_f16dq(int M, int K, int N, int Kp, const void *A, const void *Wp,
                               const void *Sp, float *C, hipStream_t s) {
    dim3 grid(div_up(N, BN), div_up(M, BM));
    hipLaunchKernelGGL((gemm_f16dq_kernel<FMT>), grid, dim3(256), 0, s, M, K, N, Kp,
                       static_cast<const _Float16 *>(A), static_cast<const uint8_t *>(Wp),
                       static_cast<const float *>(Sp), C);
    return hipGetLastError();
}

hipError_t launch_gemm_int4b64(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, float *C, hipStream_t s) {
    return launch_f16dq<QGEMM_INT4_B64>(M, K, N, K, A, Wp, Sp, C, s);
}

hipError_t launch_gemm_int8b0(int M, int K, int N, const void *A, const void *Wp,
                              const void *Sp, float *C, hipStream_t s) {
    return launch_f16dq<QGEMM_INT8_B0>(M, K, N, (int)round_up(K, 64), A, Wp, Sp, C, s);
}

}  // namespace qg
