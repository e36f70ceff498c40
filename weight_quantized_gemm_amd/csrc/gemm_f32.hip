// gemm_f32.hip -- the float-weight GEMM (MNN GemmSpeed benchmark page, mode 0
// "float-gemm": C = A[M,K] x B[K,N] with B laid out {ic, oc} = {K, N}).
//
// An LDS-tiled kernel on the fp32 matrix cores (16 x 64 or 64 x 64 tiles, K
// in chunks of 64 loaded two chunks ahead) that handles any M, K, N. Each
// 256-thread group's four waves own a quadrant (64 x 64 tile: 32 x 32, with
// v_mfma_f32_32x32x2_f32) or a 16-column strip (16 x 64 tile: 16 x 16, with
// v_mfma_f32_16x16x4_f32) and read their operands straight from the
// transposed A and row-major B chunks in LDS (consecutive lanes, consecutive
// words: no bank conflicts). Every global load is
// unconditional, from indices clamped into the arrays; values past K are
// replaced by zero on both operands (so they add exactly zero) and rows or
// columns past M or N are computed and never stored. With no skippable load
// the two-chunk prefetch really stays in flight.
//
// Work along K is spread two ways when a shape has few output tiles:
//  - inside a workgroup, KG groups of 256 threads each take a contiguous
//    share of the tile's chunks with their own LDS tiles; their partial
//    tiles are added in LDS in group order (no second launch);
//  - across workgroups, a third grid dimension splits the chunks into
//    contiguous slices; slice z writes partial tile z of a [nsplit][M][N]
//    scratch array, which a second kernel adds in slice order.
// Each output of a group's share is accumulated in fp32 by the matrix cores
// over k in increasing order of MFMA steps (2 or 4 products per step), so
// repeated runs give identical bits. K == 0 writes zeros.
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
// VEC (K and N multiples of 4): the same chunk in 16-byte pieces, A piece
// idx = i * 256 + tid being row m0 + idx / 16, k = k0 + 4 (idx % 16) .. + 3
// and B piece idx row k0 + idx / 16, columns n0 + 4 (idx % 16) .. + 3; a piece
// lies wholly inside or wholly past K and N.
template <int TM, bool VEC>
struct Chunk {
    static constexpr int FVA = 16 * TM * FK / 256;
    float a[FVA], b[FVB];
};

template <int TM, bool VEC>
__device__ __forceinline__ void load_chunk(Chunk<TM, VEC> &c, int k0, int m0, int n0, int M, int K,
                                           int N, const float *__restrict__ A,
                                           const float *__restrict__ B, int tid) {
    if constexpr (VEC) {
#pragma unroll
        for (int i = 0; i < Chunk<TM, VEC>::FVA / 4; ++i) {
            const int idx = i * 256 + tid;
            const int gm = m0 + idx / 16, gk = k0 + 4 * (idx % 16);
            const f4_t v = *reinterpret_cast<const f4_t *>(A + (size_t)min(gm, M - 1) * K + min(gk, K - 4));
#pragma unroll
            for (int j = 0; j < 4; ++j) c.a[4 * i + j] = v[j];
        }
#pragma unroll
        for (int i = 0; i < FVB / 4; ++i) {
            const int idx = i * 256 + tid;
            const int bk = k0 + idx / 16, bn = n0 + 4 * (idx % 16);
            const f4_t v = *reinterpret_cast<const f4_t *>(B + (size_t)min(bk, K - 1) * N + min(bn, N - 4));
#pragma unroll
            for (int j = 0; j < 4; ++j) c.b[4 * i + j] = v[j];
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < Chunk<TM, VEC>::FVA; ++i) {
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

// Tile of 16 TM rows x 64 columns; in each 256-thread group, thread
// (tx, ty) of the 16 x 16 grid owns rows ty * TM .. + TM - 1 and columns
// tx * 4 .. + 3. TM = 1 keeps small-M products spread over more CUs without
// idle rows.
template <int TM>
struct F32Tiles {
    float As[FK][16 * TM + 1];   // A chunk transposed: As[k][m] (odd row stride: the transposing stores of consecutive k hit distinct banks)
    float Bs[FK][FT + 4];
};

template <int TM, int KG, bool VEC>
__global__ __launch_bounds__(256 * KG) void gemm_f32_kernel(int M, int K, int N,
                                                            const float *__restrict__ A,
                                                            const float *__restrict__ B,
                                                            void *__restrict__ C,
                                                            Epilogue epi) {
    constexpr int BM = 16 * TM;
    constexpr size_t TILE_BYTES = KG * sizeof(F32Tiles<TM>);
    constexpr size_t RED_BYTES = (KG > 1 ? KG : 0) * (size_t)BM * (FT + 4) * sizeof(float);
    __shared__ __align__(16) unsigned char smem[TILE_BYTES > RED_BYTES ? TILE_BYTES : RED_BYTES];
    const int gi = uniform(threadIdx.x >> 8);
    const int tid = threadIdx.x & 255;
    F32Tiles<TM> &T = reinterpret_cast<F32Tiles<TM> *>(smem)[gi];
    const int tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * FT;
    const int lane = tid & 63, wv = tid >> 6;
    // matrix-core accumulators: 64 x 64 tile -> wave quadrant (wv >> 1, wv & 1)
    // of 32 x 32; 16 x 64 tile -> wave strip wv of 16 x 16
    f16_t mc32 = {};
    f4_t mc16 = {};

    // values at k >= kend (past K or past this group's share) are stored as zero
    auto stage = [&](const Chunk<TM, VEC> &c, int k0, int kend) {
        if constexpr (VEC) {
#pragma unroll
            for (int i = 0; i < Chunk<TM, VEC>::FVA / 4; ++i) {
                const int idx = i * 256 + tid;
                const int m = idx / 16, k = 4 * (idx % 16);
                const bool in = k0 + k < kend;
#pragma unroll
                for (int j = 0; j < 4; ++j) T.As[k + j][m] = in ? c.a[4 * i + j] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < FVB / 4; ++i) {
                const int idx = i * 256 + tid;
                const int k = idx / 16, n = 4 * (idx % 16);
                const bool in = k0 + k < kend;
                *reinterpret_cast<f4_t *>(&T.Bs[k][n]) =
                    in ? f4_t{c.b[4 * i], c.b[4 * i + 1], c.b[4 * i + 2], c.b[4 * i + 3]}
                       : f4_t{0.f, 0.f, 0.f, 0.f};
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < Chunk<TM, VEC>::FVA; ++i) {
            const int idx = i * 256 + tid;
            T.As[idx % FK][idx / FK] = k0 + idx % FK < kend ? c.a[i] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < FVB; ++i) {
            const int idx = i * 256 + tid;
            T.Bs[idx / FT][idx % FT] = k0 + idx / FT < kend ? c.b[i] : 0.f;
        }
    };
    // lane l of a 32x32x2 step holds A[row l % 32][k + l / 32] and
    // B[k + l / 32][col l % 32]; of a 16x16x4 step A[row l % 16][k + l / 16]
    // and B[k + l / 16][col l % 16]
    auto multiply = [&]() {
        if constexpr (TM == 4) {
            const int r = lane & 31, h = lane >> 5;
            const int ma = 32 * (wv >> 1) + r, nb = 32 * (wv & 1) + r;
#pragma unroll 8
            for (int kk = 0; kk < FK; kk += 2)
                mc32 = __builtin_amdgcn_mfma_f32_32x32x2f32(T.As[kk + h][ma], T.Bs[kk + h][nb], mc32, 0, 0, 0);
        } else {
            const int r = lane & 15, q = lane >> 4;
            const int nb = 16 * wv + r;
#pragma unroll 8
            for (int kk = 0; kk < FK; kk += 4)
                mc16 = __builtin_amdgcn_mfma_f32_16x16x4f32(T.As[kk + q][r], T.Bs[kk + q][nb], mc16, 0, 0, 0);
        }
    };

    // chunks of this slice [s0, s1) (all of K without a split), then this
    // group's share [c0, c1); every group runs the same padded, even number
    // of iterations (a chunk past its share is neither staged nor
    // multiplied: a uniform branch that contains no load)
    const int nch = (K + FK - 1) / FK;
    const int s0 = slice_begin(blockIdx.z, nch, gridDim.z);
    const int s1 = slice_begin(blockIdx.z + 1, nch, gridDim.z);
    const int c0 = s0 + gi * (s1 - s0) / KG, c1 = s0 + (gi + 1) * (s1 - s0) / KG;
    const int npad = ((s1 - s0 + KG - 1) / KG + 1) & ~1;
    const int kend = min(K, c1 * FK);
    Chunk<TM, VEC> r0, r1;
    if (npad > 0) {            // K == 0 (or an empty slice) reads nothing
        load_chunk<TM, VEC>(r0, c0 * FK, m0, n0, M, K, N, A, B, tid);
        load_chunk<TM, VEC>(r1, (c0 + 1) * FK, m0, n0, M, K, N, A, B, tid);
    }
    for (int c = 0; c < npad; c += 2) {
        const bool live0 = c0 + c < c1, live1 = c0 + c + 1 < c1;
        if (live0) stage(r0, (c0 + c) * FK, kend);
        __syncthreads();
        load_chunk<TM, VEC>(r0, min(c0 + c + 2, nch) * FK, m0, n0, M, K, N, A, B, tid);
        if (live0) multiply();
        __syncthreads();
        if (live1) stage(r1, (c0 + c + 1) * FK, kend);
        __syncthreads();
        load_chunk<TM, VEC>(r1, min(c0 + c + 3, nch) * FK, m0, n0, M, K, N, A, B, tid);
        if (live1) multiply();
        __syncthreads();
    }

    // the matrix-core layout to thread (tx, ty)'s rows ty * TM .. and
    // columns tx * 4 .. (through this group's part of LDS, over its tiles;
    // the loop's last barrier has passed)
    float acc[TM][4];
    {
        float *cv = reinterpret_cast<float *>(smem) + (size_t)gi * BM * (FT + 4);
        if constexpr (TM == 4) {
            const int r = lane & 31, h = lane >> 5;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                cv[(32 * (wv >> 1) + 8 * (i >> 2) + 4 * h + (i & 3)) * (FT + 4) + 32 * (wv & 1) + r] = mc32[i];
        } else {
            const int r = lane & 15, q = lane >> 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) cv[(4 * q + i) * (FT + 4) + 16 * wv + r] = mc16[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = cv[(ty * TM + i) * (FT + 4) + tx * 4 + j];
        __syncthreads();
    }

    // the groups' partial tiles meet in LDS (reusing the tiles' space) and
    // are added in group order
    if (KG > 1) {
        float *red = reinterpret_cast<float *>(smem);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                red[((size_t)gi * BM + ty * TM + i) * (FT + 4) + tx * 4 + j] = acc[i][j];
        __syncthreads();
        if (gi != 0) return;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v = red[(size_t)(ty * TM + i) * (FT + 4) + tx * 4 + j];
#pragma unroll
                for (int g = 1; g < KG; ++g) v += red[((size_t)g * BM + ty * TM + i) * (FT + 4) + tx * 4 + j];
                acc[i][j] = v;
            }
    }
    // partial tiles (split-K) and plain fp32 C take the raw store
    const bool raw = gridDim.z > 1 || epi.plain;
    float *const out = static_cast<float *>(C) + (size_t)blockIdx.z * M * N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int gm = m0 + ty * TM + i;
        if (gm >= M) continue;
        const int gn0 = n0 + tx * 4;
        if (!raw && (N & 3) == 0 && gn0 + 4 <= N) {
            epi_put4(epi, C, gm, gn0, N, f4_t{acc[i][0], acc[i][1], acc[i][2], acc[i][3]});
            continue;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gn = gn0 + j;
            if (gn >= N) continue;
            if (raw) out[(size_t)gm * N + gn] = acc[i][j];
            else epi_put(epi, C, gm, gn, N, acc[i][j]);
        }
    }
}

hipError_t launch_gemm_f32(int M, int K, int N, const float *A, const float *B, void *C,
                           const Epilogue &epi, int nsplit, float *part, hipStream_t s) {
    void *out = nsplit > 1 ? static_cast<void *>(part) : C;
    const bool small = M <= kF32TileMSmall;
    const dim3 grid(div_up(N, FT), div_up(M, small ? kF32TileMSmall : kF32TileM), nsplit);
    // 16-byte pieces when every row of A and B starts 16-byte aligned
    const bool vec = (K & 3) == 0 && (N & 3) == 0 && K > 0 &&
                     ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) == 0;
    auto go = [&](auto kernel, int threads) {
        hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, s, M, K, N, A, B, out, epi);
    };
    const bool kg = f32_kgroups(M, N) > 1;
    if (kg && small) vec ? go(gemm_f32_kernel<1, kF32KGroups, true>, 256 * kF32KGroups)
                         : go(gemm_f32_kernel<1, kF32KGroups, false>, 256 * kF32KGroups);
    else if (kg) vec ? go(gemm_f32_kernel<4, kF32KGroups, true>, 256 * kF32KGroups)
                     : go(gemm_f32_kernel<4, kF32KGroups, false>, 256 * kF32KGroups);
    else if (small) vec ? go(gemm_f32_kernel<1, 1, true>, 256) : go(gemm_f32_kernel<1, 1, false>, 256);
    else vec ? go(gemm_f32_kernel<4, 1, true>, 256) : go(gemm_f32_kernel<4, 1, false>, 256);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nsplit <= 1) return e;
    return launch_splitk_reduce_f32(part, nsplit, M, N, C, epi, s);
}

}  // namespace qg
