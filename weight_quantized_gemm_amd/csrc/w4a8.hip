// w4a8.hip -- the W4A8 prefill path: per-row dynamic int8 quantisation of the
// fp16 activations, then an exact s8 x s8 -> s32 product on the int8 matrix
// cores with an fp32 rescale epilogue.
//
// MNN GemmSpeed benchmark page, section "Test cases and registration", mode 3
// (Int4-Block0 W4A8): per-channel 4-bit weights are unpacked to int8, the
// activations are dynamically quantised to int8 and an S8 x S8 -> S32 GEMM
// runs. The page fixes no formula; the reading implemented here:
//   sa[m] = max_k |A[m][k]| / 127 (fp32, correctly rounded division),
//   qa[m][k] = clamp(rint(A[m][k] / sa[m]), -127, 127) (ties to even),
//   a zero row gives sa = 0 and qa = 0, S[m] = sum_k qa[m][k];
//   D[m][n] = sum_k qa[m][k] * q[n][k] with q the zero-extended code in [0, 15];
//   C[m][n] = sa[m] * (scale[n] * D[m][n] + offset[n] * S[m]),
// which is sum_k (sa qa) (offset + scale q) regrouped so the inner loop is
// pure integer arithmetic.
#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

// ---------------------------------------------------------------------------
// Activation quantisation: one 256-thread workgroup per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void w4a8_actquant_kernel(int M, int K, int Kp,
                                                            const _Float16 *__restrict__ A,
                                                            int8_t *__restrict__ qa,
                                                            float *__restrict__ sa,
                                                            int32_t *__restrict__ S) {
    __shared__ float red_f[4];
    __shared__ int red_i[4];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const _Float16 *row = A + (size_t)m * K;
    int8_t *qrow = qa + (size_t)m * Kp;
    const bool vec = (K & 7) == 0;

    float amax = 0.0f;
    if (vec) {
        for (int k = tid * 8; k < K; k += 2048) {
            const h8_t v = *reinterpret_cast<const h8_t *>(row + k);
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[e]));
        }
    } else {
        for (int k = tid; k < K; k += 256) amax = fmaxf(amax, fabsf((float)row[k]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((tid & 63) == 0) red_f[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));

    const float s = amax / 127.0f;   // IEEE division, one rounding
    int sum = 0;
    if (vec) {
        for (int k = tid * 8; k < Kp; k += 2048) {
            unsigned lo = 0u, hi = 0u;
            if (k < K && amax != 0.0f) {
                const h8_t v = *reinterpret_cast<const h8_t *>(row + k);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float r = rintf((float)v[e] / s);
                    r = fminf(fmaxf(r, -127.0f), 127.0f);
                    const int qi = (int)r;
                    sum += qi;
                    const unsigned byte = (unsigned)(qi & 0xff);
                    if (e < 4) lo |= byte << (8 * e);
                    else hi |= byte << (8 * (e - 4));
                }
            }
            *reinterpret_cast<u2_t *>(qrow + k) = u2_t{lo, hi};
        }
    } else {
        for (int k = tid; k < Kp; k += 256) {
            int qi = 0;
            if (k < K && amax != 0.0f) {
                float r = rintf((float)row[k] / s);
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                qi = (int)r;
            }
            sum += qi;
            qrow[k] = (int8_t)qi;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if ((tid & 63) == 0) red_i[tid >> 6] = sum;
    __syncthreads();
    if (tid == 0) {
        sa[m] = amax != 0.0f ? s : 0.0f;
        S[m] = red_i[0] + red_i[1] + red_i[2] + red_i[3];
    }
}

hipError_t launch_w4a8_actquant(int M, int K, int Kp, const void *A, int8_t *qa, float *sa,
                                int32_t *S, hipStream_t s) {
    hipLaunchKernelGGL(w4a8_actquant_kernel, dim3(M), dim3(256), 0, s, M, K, Kp,
                       static_cast<const _Float16 *>(A), qa, sa, S);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// int8 GEMM: 128 x 128 tile per 256-thread workgroup, K step 64 bytes; four
// waves split the tile 2 x 2, each 64 x 64 with v_mfma_i32_32x32x32_i8.
// ---------------------------------------------------------------------------
namespace {
constexpr int TM = 128, TN = 128, TK = 64;
constexpr int ROW = TK + 16;   // bytes per LDS row; 80-byte rows spread the banks
}

template <bool DEBUG_D>
__global__ __launch_bounds__(256) void w4a8_gemm_kernel(
    int M, int N, int Kp, const int8_t *__restrict__ qa, const float *__restrict__ sa,
    const int32_t *__restrict__ S, const uint8_t *__restrict__ Wp, const f2_t *__restrict__ Sp,
    float *__restrict__ C, int32_t *__restrict__ D) {
    __shared__ __align__(16) int8_t As[TM * ROW];
    __shared__ __align__(16) int8_t Bs[TN * ROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * TM;
    const int n0 = blockIdx.x * TN;
    const int nkc = Kp >> 6;
    const int Np = (N + 31) & ~31;

    i16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[a][b][j] = 0;

    // B loader role: channel tid / 2 of the tile, half tid % 2 of its 32-byte record.
    const int bn = tid >> 1, bh = tid & 1;
    const int gn = n0 + bn;

    for (int kc = 0; kc < nkc; ++kc) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int idx = it * 256 + tid;
            const int r = idx >> 2, c16 = (idx & 3) * 16;
            const int gm = m0 + r;
            u4_t v = {0u, 0u, 0u, 0u};
            if (gm < M)
                v = *reinterpret_cast<const u4_t *>(qa + (size_t)gm * Kp + (size_t)kc * 64 + c16);
            *reinterpret_cast<u4_t *>(As + r * ROW + c16) = v;
        }
        {
            u4_t v = {0u, 0u, 0u, 0u};
            if (gn < Np) {
                const int g = gn >> 5, c = gn & 31;
                v = *reinterpret_cast<const u4_t *>(
                    Wp + (((size_t)g * nkc + kc) * 32 + c) * 32 + bh * 16);
            }
            // each word -> codes of k0..k0+3 and k0+4..k0+7 as int8 (natural order)
            u4_t lo, hi;
#pragma unroll
            for (int wi = 0; wi < 4; ++wi) {
                lo[wi] = v[wi] & 0x0F0F0F0Fu;
                hi[wi] = (v[wi] >> 4) & 0x0F0F0F0Fu;
            }
            u4_t *dst = reinterpret_cast<u4_t *>(Bs + bn * ROW + bh * 32);
            dst[0] = u4_t{lo[0], hi[0], lo[1], hi[1]};
            dst[1] = u4_t{lo[2], hi[2], lo[3], hi[3]};
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int kk = s * 32 + (lane >> 5) * 16;
            i4_t a[2], b[2];
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                a[f] = *reinterpret_cast<const i4_t *>(As + (wm * 64 + f * 32 + (lane & 31)) * ROW + kk);
                b[f] = *reinterpret_cast<const i4_t *>(Bs + (wn * 64 + f * 32 + (lane & 31)) * ROW + kk);
            }
#pragma unroll
            for (int fm = 0; fm < 2; ++fm)
#pragma unroll
                for (int fn = 0; fn < 2; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
        }
        __syncthreads();
    }

#pragma unroll
    for (int fn = 0; fn < 2; ++fn) {
        const int col = n0 + wn * 64 + fn * 32 + (lane & 31);
        if (col >= N) continue;
        const f2_t pr = Sp[col];
#pragma unroll
        for (int fm = 0; fm < 2; ++fm) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int row = m0 + wm * 64 + fm * 32 + (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
                if (row >= M) continue;
                const int d = acc[fm][fn][j];
                if (DEBUG_D) D[(size_t)row * N + col] = d;
                C[(size_t)row * N + col] = sa[row] * fmaf(pr.y, (float)d, pr.x * (float)S[row]);
            }
        }
    }
}

hipError_t launch_w4a8_gemm(int M, int K, int N, const int8_t *qa, const float *sa,
                            const int32_t *S, const void *Wp, const void *Sp, float *C,
                            int32_t *D_debug, hipStream_t s) {
    const int Kp = (int)round_up(K, 64);
    dim3 grid(div_up(N, TN), div_up(M, TM));
    if (D_debug)
        hipLaunchKernelGGL(w4a8_gemm_kernel<true>, grid, dim3(256), 0, s, M, N, Kp, qa, sa, S,
                           static_cast<const uint8_t *>(Wp), static_cast<const f2_t *>(Sp), C,
                           D_debug);
    else
        hipLaunchKernelGGL(w4a8_gemm_kernel<false>, grid, dim3(256), 0, s, M, N, Kp, qa, sa, S,
                           static_cast<const uint8_t *>(Wp), static_cast<const f2_t *>(Sp), C,
                           D_debug);
    return hipGetLastError();
}

}  // namespace qg
