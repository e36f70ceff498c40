// gemm_f32.hip -- the float-weight GEMM (MNN GemmSpeed benchmark page, mode 0
// "float-gemm": C = A[M,K] x B[K,N] with B laid out {ic, oc} = {K, N}).
//
// The float workloads are tiny and launch-bound, so this is a plain
// LDS-tiled fp32 FMA kernel that handles any M, K, N (ragged tails are
// masked, K == 0 writes zeros). Each output is one fp32 FMA chain over k in
// increasing order.
#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

namespace {
constexpr int FT = 64;   // output tile edge
constexpr int FK = 16;   // K step
}

__global__ __launch_bounds__(256) void gemm_f32_kernel(int M, int K, int N,
                                                       const float *__restrict__ A,
                                                       const float *__restrict__ B,
                                                       float *__restrict__ C) {
    __shared__ float As[FK][FT + 4];   // A tile transposed: As[k][m]
    __shared__ float Bs[FK][FT + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * FT, n0 = blockIdx.x * FT;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int k0 = 0; k0 < K; k0 += FK) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = it * 256 + tid;
            const int r = idx >> 4, c = idx & 15;          // A: 64 rows x 16 k
            const int gm = m0 + r, gk = k0 + c;
            As[c][r] = (gm < M && gk < K) ? A[(size_t)gm * K + gk] : 0.f;
            const int br = idx >> 6, bc = idx & 63;        // B: 16 k x 64 cols
            const int bk = k0 + br, bn = n0 + bc;
            Bs[br][bc] = (bk < K && bn < N) ? B[(size_t)bk * N + bn] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < FK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int gm = m0 + ty * 4 + i;
        if (gm >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gn = n0 + tx * 4 + j;
            if (gn < N) C[(size_t)gm * N + gn] = acc[i][j];
        }
    }
}

hipError_t launch_gemm_f32(int M, int K, int N, const float *A, const float *B, float *C,
                           hipStream_t s) {
    dim3 grid(div_up(N, FT), div_up(M, FT));
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, M, K, N, A, B, C);
    return hipGetLastError();
}

}  // namespace qg
