// gemm_f32.hip -- the float-weight GEMM (MNN GemmSpeed benchmark page, mode 0
// "float-gemm": C = A[M,K] x B[K,N] with B laid out {ic, oc} = {K, N}).
//
// An LDS-tiled fp32 FMA kernel (16 x 64 or 64 x 64 tiles, K in chunks of 64
// loaded two chunks ahead) that handles any M, K, N. Every global load is
// unconditional, from indices clamped into the arrays; values past K are
// replaced by zero on both operands (so they add exactly zero) and rows or
// columns past M or N are computed and never stored. With no skippable load
// the two-chunk prefetch really stays in flight. Each output of a K-slice is
// one fp32 FMA chain over k in increasing order.
//
// Split-K: shapes with few output tiles split the chunks into contiguous
// slices over a third grid dimension; slice z writes partial tile z of a
// [nsplit][M][N] scratch array, which a second kernel adds in slice order.
// K == 0 writes zeros.
#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

namespace {
constexpr int FT = kF32TileN;    // output tile width (columns)
constexpr int FK = kF32ChunkK;   // K chunk staged in LDS
static_assert(kF32TileMSmall == 16 && kF32TileM == 64, "tile rows are 16 TM with TM = 1 or 4");
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
        const float v = A[(size_t)min(gm, M - 1) * K + min(gk, K - 1)];
        c.a[i] = gk < K ? v : 0.f;
    }
#pragma unroll
    for (int i = 0; i < FVB; ++i) {
        const int idx = i * 256 + tid;
        const int bk = k0 + idx / FT, bn = n0 + idx % FT;
        const float v = B[(size_t)min(bk, K - 1) * N + min(bn, N - 1)];
        c.b[i] = bk < K ? v : 0.f;
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
    // values at k >= kend (past K or past this slice) are stored as zero
    auto stage = [&](const Chunk<TM> &c, int k0, int kend) {
#pragma unroll
        for (int i = 0; i < Chunk<TM>::FVA; ++i) {
            const int idx = i * 256 + tid;
            As[idx % FK][idx / FK] = k0 + idx % FK < kend ? c.a[i] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < FVB; ++i) {
            const int idx = i * 256 + tid;
            Bs[idx / FT][idx % FT] = k0 + idx / FT < kend ? c.b[i] : 0.f;
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

    // this slice's chunks [c0, c1) (all of K without a split), padded to an
    // even count: a padded chunk lies past K and adds exactly zero
    const int nch = (K + FK - 1) / FK;
    const int c0 = (int)((long long)blockIdx.z * nch / gridDim.z);
    const int c1 = (int)((long long)(blockIdx.z + 1) * nch / gridDim.z);
    const int npad = (c1 - c0 + 1) & ~1;
    Chunk<TM> r0, r1;
    if (npad > 0) {            // K == 0 (or an empty slice) reads nothing
        load_chunk<TM>(r0, c0 * FK, m0, n0, M, K, N, A, B, tid);
        load_chunk<TM>(r1, (c0 + 1) * FK, m0, n0, M, K, N, A, B, tid);
    }
    for (int c = 0; c < npad; c += 2) {
        // a chunk of this slice past c1 is masked like one past K
        const int kend = min(K, c1 * FK);
        stage(r0, (c0 + c) * FK, kend);
        __syncthreads();
        load_chunk<TM>(r0, min(c0 + c + 2, nch) * FK, m0, n0, M, K, N, A, B, tid);
        multiply();
        __syncthreads();
        stage(r1, (c0 + c + 1) * FK, kend);
        __syncthreads();
        load_chunk<TM>(r1, min(c0 + c + 3, nch) * FK, m0, n0, M, K, N, A, B, tid);
        multiply();
        __syncthreads();
    }
    float *const out = C + (size_t)blockIdx.z * M * N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int gm = m0 + ty * TM + i;
        if (gm >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gn = n0 + tx * 4 + j;
            if (gn < N) out[(size_t)gm * N + gn] = acc[i][j];
        }
    }
}

hipError_t launch_gemm_f32(int M, int K, int N, const float *A, const float *B, float *C,
                           int nsplit, float *part, hipStream_t s) {
    float *out = nsplit > 1 ? part : C;
    if (M <= kF32TileMSmall) {
        hipLaunchKernelGGL(gemm_f32_kernel<1>, dim3(div_up(N, FT), div_up(M, 16), nsplit),
                           dim3(256), 0, s, M, K, N, A, B, out);
    } else {
        hipLaunchKernelGGL(gemm_f32_kernel<4>, dim3(div_up(N, FT), div_up(M, 64), nsplit),
                           dim3(256), 0, s, M, K, N, A, B, out);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nsplit <= 1) return e;
    return launch_splitk_reduce_f32(part, nsplit, M, N, C, s);
}

}  // namespace qg
