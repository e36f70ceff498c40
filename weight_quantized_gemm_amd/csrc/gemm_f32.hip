// gemm_f32.hip -- the float-weight GEMM (MNN GemmSpeed benchmark page, mode 0
// "float-gemm": C = A[M,K] x B[K,N] with B laid out {ic, oc} = {K, N}).
//
// The float workloads are tiny and bound by launch and memory latency, so
// this is a plain LDS-tiled fp32 FMA kernel (16 x 64 or 64 x 64 tiles, K in
// chunks of 64 loaded two chunks ahead) that handles any M, K, N: ragged tails are
// masked and K == 0 writes zeros. Each output is one fp32 FMA chain over k
// in increasing order.
#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

namespace {
constexpr int FT = 64;   // output tile width (columns)
constexpr int FK = 64;   // K chunk staged in LDS
constexpr int FVB = FT * FK / 256;   // values of B each thread loads per chunk

// One K chunk of the tile (16 TM rows x FT columns), held in registers
// between its global loads and its LDS stores: A rows m0 + idx / FK,
// k = k0 + idx % FK and B rows k0 + idx / FT, columns n0 + idx % FT,
// idx = i * 256 + tid (coalesced runs).
template <int TM>
struct Chunk {
    static constexpr int FVA = 16 * TM * FK / 256;
    float a[FVA], b[FVB];
};

template <int TM>
__device__ __forceinline__ void load_chunk(Chunk<TM> &c, int k0, int m0, int n0, int M, int K,
                                           int N, const float *__restrict__ A,
                                           const float *__restrict__ B, int tid) {
#pragma unroll
    for (int i = 0; i < Chunk<TM>::FVA; ++i) {
        const int idx = i * 256 + tid;
        const int gm = m0 + idx / FK, gk = k0 + idx % FK;
        c.a[i] = (gm < M && gk < K) ? A[(size_t)gm * K + gk] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < FVB; ++i) {
        const int idx = i * 256 + tid;
        const int bk = k0 + idx / FT, bn = n0 + idx % FT;
        c.b[i] = (bk < K && bn < N) ? B[(size_t)bk * N + bn] : 0.f;
    }
}
}

// Tile of 16 TM rows x 64 columns; thread (tx, ty) of the 16 x 16 grid owns
// rows ty * TM .. + TM - 1 and columns tx * 4 .. + 3. TM = 1 keeps small-M
// products spread over more CUs without idle rows.
template <int TM>
__global__ __launch_bounds__(256) void gemm_f32_kernel(int M, int K, int N,
                                                       const float *__restrict__ A,
                                                       const float *__restrict__ B,
                                                       float *__restrict__ C) {
    constexpr int BM = 16 * TM;
    __shared__ float As[FK][BM + 4];   // A chunk transposed: As[k][m]
    __shared__ float Bs[FK][FT + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * FT;
    float acc[TM][4];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    // Chunks c and c + 1 are in flight while chunk c - 1 is multiplied: the
    // two-deep ring keeps the latency of a global load off the critical path
    // for all but the first chunk.
    auto stage = [&](const Chunk<TM> &c) {
#pragma unroll
        for (int i = 0; i < Chunk<TM>::FVA; ++i) {
            const int idx = i * 256 + tid;
            As[idx % FK][idx / FK] = c.a[i];
        }
#pragma unroll
        for (int i = 0; i < FVB; ++i) {
            const int idx = i * 256 + tid;
            Bs[idx / FT][idx % FT] = c.b[i];
        }
    };
    auto multiply = [&]() {
#pragma unroll 8
        for (int kk = 0; kk < FK; ++kk) {
            float a[TM], b[4];
#pragma unroll
            for (int i = 0; i < TM; ++i) a[i] = As[kk][ty * TM + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
    };

    const int nch = (K + FK - 1) / FK;
    Chunk<TM> r0, r1;
    if (nch > 0) load_chunk<TM>(r0, 0, m0, n0, M, K, N, A, B, tid);
    if (nch > 1) load_chunk<TM>(r1, FK, m0, n0, M, K, N, A, B, tid);
    for (int c = 0; c < nch; c += 2) {
        stage(r0);
        __syncthreads();
        if (c + 2 < nch) load_chunk<TM>(r0, (c + 2) * FK, m0, n0, M, K, N, A, B, tid);
        multiply();
        __syncthreads();
        if (c + 1 >= nch) break;
        stage(r1);
        __syncthreads();
        if (c + 3 < nch) load_chunk<TM>(r1, (c + 3) * FK, m0, n0, M, K, N, A, B, tid);
        multiply();
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int gm = m0 + ty * TM + i;
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
    if (M <= 16) {
        hipLaunchKernelGGL(gemm_f32_kernel<1>, dim3(div_up(N, FT), div_up(M, 16)), dim3(256), 0,
                           s, M, K, N, A, B, C);
    } else {
        hipLaunchKernelGGL(gemm_f32_kernel<4>, dim3(div_up(N, FT), div_up(M, 64)), dim3(256), 0,
                           s, M, K, N, A, B, C);
    }
    return hipGetLastError();
}

}  // namespace qg
