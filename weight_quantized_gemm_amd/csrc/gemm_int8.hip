// gemm_int8.hip -- prefill GEMM (M above the GEMV threshold) with
// Int8-Block0 weights on the fp16 matrix cores.
//
// What is computed (MNN GemmSpeed benchmark page, section "Why Conv1x1 is
// used to measure GEMM"): C = A x deq(B), deq(B)[k][n] = offset[n] +
// scale[n] * q[n][k] (one pair per output channel, blockSize = K). The
// weight is formed in fp32 (one fused multiply-add) and rounded once to
// fp16; accumulation is fp32 in the MFMA accumulators and C is fp32.
//
// Decomposition: a 256-thread workgroup owns a 128 x 64 tile of C; its four
// waves split K (wave w takes the 64-wide K-blocks w, w+4, ...) and each
// accumulates the whole tile with v_mfma_f32_16x16x32_f16. Each K-block is
// consumed as two halves of 32; lane (r, g) = (lane % 16, lane / 16) owns
// K-elements k0 + 8 g .. +7 of a half for its A rows and B columns alike.
// Loads run ahead of the arithmetic through register rings; the four partial
// tiles are summed in LDS in a fixed order.
#include <type_traits>

#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

namespace {
constexpr int BM = 128, BN = 64, BK = 64;
constexpr int RF = BM / 16;   // 16-row accumulator tiles per wave
constexpr int CF = BN / 16;   // 16-column accumulator tiles per wave
constexpr int RED_STRIDE = BN + 4;   // floats per LDS row of the reduction
// Register rings, in half-block iterations (32 K-elements): A is loaded
// RA - 1 iterations ahead and codes RB iterations ahead (about four K-blocks,
// enough to cover an HBM miss). The main loop is unrolled UNROLL times so
// every ring slot is a fixed register.
constexpr int RA = 4, RB = 8, UNROLL = 8;
}

// 8 Int8 codes (two words, k ascending) -> 8 fp16 weights.
__device__ __forceinline__ h8_t dequant8_int8(u2_t codes, float scale, float bias) {
    h8_t o;
#pragma unroll
    for (int wi = 0; wi < 2; ++wi) {
        const unsigned word = codes[wi];
        const h2_t x0 = as_h2(__builtin_amdgcn_perm(0x64646464u, word, 0x04010400u));  // q0, q1
        const h2_t x1 = as_h2(__builtin_amdgcn_perm(0x64646464u, word, 0x04030402u));  // q2, q3
        o[wi * 4 + 0] = (_Float16)fmaf((float)x0.x, scale, bias);
        o[wi * 4 + 1] = (_Float16)fmaf((float)x0.y, scale, bias);
        o[wi * 4 + 2] = (_Float16)fmaf((float)x1.x, scale, bias);
        o[wi * 4 + 3] = (_Float16)fmaf((float)x1.y, scale, bias);
    }
    return o;
}

__global__ __launch_bounds__(256) void gemm_int8b0_kernel(
    int M, int K, int N, int Kp, int tiles_n, int xcd_order, const _Float16 *__restrict__ A,
    const uint8_t *__restrict__ Wp, const float *__restrict__ Sp, float *__restrict__ C) {
    __shared__ __align__(16) float red[4][BM * RED_STRIDE];   // 4 x 34 KiB

    // Tile of this workgroup. With xcd_order, the workgroups the hardware
    // deals to one XCD (ids equal mod 8) get a contiguous run of tiles.
    const int L = blockIdx.x;
    const int T = gridDim.x;
    const int t = xcd_order ? (L % 8) * (T / 8) + (L / 8) : L;
    const int m0 = (t / tiles_n) * BM;
    const int n0 = (t % tiles_n) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const bool a_vec = (K & 7) == 0;
    const int Np = (N + 3) & ~3;
    const int nblk = Kp / BK;
    const int nb_w = nblk > wave ? (nblk - wave + 3) / 4 : 0;   // K-blocks of this wave
    const int n_it = 2 * nb_w;                                   // half-block iterations

    // lane (r, g) holds K-elements k0 + 8 g .. k0 + 8 g + 7 of each half-block,
    // for A rows m0 + 16 rf + r and B columns n0 + 16 cf + r.
    auto load_a = [&](u4_t (&dst)[RF], int it) {
        const int k = (wave + 4 * (it >> 1)) * BK + 32 * (it & 1) + 8 * g;
#pragma unroll
        for (int rf = 0; rf < RF; ++rf) {
            const int gm = m0 + rf * 16 + r;
            u4_t v = {0u, 0u, 0u, 0u};
            if (gm < M) {
                const _Float16 *src = A + (size_t)gm * K + k;
                if (a_vec) {   // K % 8 == 0: each 8-element piece is all in or all out
                    if (k < K) v = *reinterpret_cast<const u4_t *>(src);
                } else {
                    h8_t t8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) t8[e] = (k + e < K) ? src[e] : (_Float16)0.0f;
                    v = __builtin_bit_cast(u4_t, t8);
                }
            }
            dst[rf] = v;
        }
    };
    auto load_b = [&](u2_t (&dst)[CF], int it) {
        const int kt = wave + 4 * (it >> 1), h = it & 1;
#pragma unroll
        for (int cf = 0; cf < CF; ++cf) {
            const int gn = n0 + cf * 16 + r;
            u2_t v = {0u, 0u};
            if (gn < Np)
                v = *reinterpret_cast<const u2_t *>(Wp + (size_t)gn * Kp + kt * BK + 32 * h + 8 * g);
            dst[cf] = v;
        }
    };
    auto load_p = [&](f2_t (&dst)[CF], int j) {   // pairs of the wave's j-th K-block
        const int kt = wave + 4 * j;
#pragma unroll
        for (int cf = 0; cf < CF; ++cf) {
            const int gn = n0 + cf * 16 + r;
            f2_t v = {0.f, 0.f};
            if (gn < Np) v = *reinterpret_cast<const f2_t *>(Sp + (size_t)gn * 2);
            dst[cf] = v;
        }
    };

    f4_t acc[RF][CF];
#pragma unroll
    for (int i = 0; i < RF; ++i)
#pragma unroll
        for (int j = 0; j < CF; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    u4_t ra[RA][RF];
    u2_t rb[RB][CF];
    f2_t rp[1][CF];
#pragma unroll
    for (int d = 0; d < RA - 1; ++d)
        if (d < n_it) load_a(ra[d], d);
#pragma unroll
    for (int d = 0; d < RB; ++d)
        if (d < n_it) load_b(rb[d], d);
    load_p(rp[0], 0);   // one pair per channel for all of K

    for (int base = 0; base < n_it; base += UNROLL) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int it = base + u;
            if (it < n_it) {
                if (it + RA - 1 < n_it) load_a(ra[(u + RA - 1) % RA], it + RA - 1);
                const int ps = 0;
                h8_t bw[CF];
#pragma unroll
                for (int cf = 0; cf < CF; ++cf) {
                    const float sc = rp[ps][cf].y;
                    const float bias = fmaf(-1024.0f, sc, rp[ps][cf].x);
                    bw[cf] = dequant8_int8(rb[u % RB][cf], sc, bias);
                }
                if (it + RB < n_it) load_b(rb[u % RB], it + RB);
#pragma unroll
                for (int rf = 0; rf < RF; ++rf) {
                    const h8_t a = __builtin_bit_cast(h8_t, ra[u % RA][rf]);
#pragma unroll
                    for (int cf = 0; cf < CF; ++cf)
                        acc[rf][cf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bw[cf], acc[rf][cf], 0, 0, 0);
                }
            }
        }
    }

    // Partial tiles to LDS: accumulator element i of lane l in tile (rf, cf)
    // is C[rf*16 + 4*(l/16) + i][cf*16 + l%16].
    float *mine = red[wave];
#pragma unroll
    for (int rf = 0; rf < RF; ++rf)
#pragma unroll
        for (int cf = 0; cf < CF; ++cf)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mine[(rf * 16 + 4 * g + i) * RED_STRIDE + cf * 16 + r] = acc[rf][cf][i];
    __syncthreads();

    // Sum the four partials (fixed order) and store: thread -> row tid/2,
    // 32 consecutive columns.
    const int row = tid >> 1;
    const int c0 = (tid & 1) * 32;
    const int gm = m0 + row;
    if (gm >= M) return;
    float *dst = C + (size_t)gm * N + n0 + c0;
    const bool vec_store = (N & 3) == 0 && n0 + c0 + 32 <= N;
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
        const int o = row * RED_STRIDE + c0 + j;
        const f4_t sum = *reinterpret_cast<const f4_t *>(&red[0][o]) +
                         *reinterpret_cast<const f4_t *>(&red[1][o]) +
                         *reinterpret_cast<const f4_t *>(&red[2][o]) +
                         *reinterpret_cast<const f4_t *>(&red[3][o]);
        if (vec_store) {
            *reinterpret_cast<f4_t *>(dst + j) = sum;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n0 + c0 + j + e < N) dst[j + e] = sum[e];
        }
    }
}

hipError_t launch_gemm_int8b0(int M, int K, int N, const void *A, const void *Wp,
                              const void *Sp, float *C, hipStream_t s) {
    const int Kp = (int)round_up(K, 64);
    const int tiles_n = div_up(N, BN);
    const int tiles = tiles_n * div_up(M, BM);
    const int xcd_order = (tiles % 8) == 0 ? 1 : 0;
    hipLaunchKernelGGL(gemm_int8b0_kernel, dim3(tiles), dim3(256), 0, s, M, K, N, Kp,
                       tiles_n, xcd_order, static_cast<const _Float16 *>(A),
                       static_cast<const uint8_t *>(Wp), static_cast<const float *>(Sp), C);
    return hipGetLastError();
}

}  // namespace qg
