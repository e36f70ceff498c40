// gemm_int8.hip -- prefill GEMM (M above the GEMV threshold) for weights
// stored as channel rows [Np][Kp] on the fp16 matrix cores: Int8-Block0
// codes, or fp16 weights (the float mode at FP16 precision, which the same
// kernel multiplies as they are, with no pair and no regrouping).
//
// What is computed (MNN GemmSpeed benchmark page, section "Why Conv1x1 is
// used to measure GEMM"): C = A x deq(B), deq(B)[k][n] = offset[n] +
// scale[n] * q[n][k], one [offset, scale] pair per output channel over all
// of K (blockSize = K). Because the pair does not change along K, the
// product regroups exactly as
//   C[m][n] = scale[n] * P[m][n] + (offset[n] - 1024 scale[n]) * rowsum(A)[m],
//   P[m][n] = sum_k A[m][k] * (1024 + q[n][k]),
// and the matrix cores only ever see the codes: 1024 + q (q in [0, 255]) is
// an exact fp16 integer made by one byte permute per two codes, every
// product A * (1024 + q) is exact in fp32, and the MFMAs accumulate in fp32.
// Scale, offset and the row sums (fp32, from v_dot2 on the A fragments
// already in registers) enter once, in the epilogue. There is no per-weight
// arithmetic besides the permute. The pages' dequantise-then-multiply gives
// the same value up to rounding: this form rounds fewer times (the weight is
// never narrowed to fp16).
//
// Decomposition: a 256-thread workgroup owns a 128 x 64 tile of C (over a
// contiguous slice of the K-blocks when the shape has too few tiles to fill
// the chip: split-K, slice blockIdx.y of gridDim.y, written as a partial tile
// that already carries its slice's share of the regrouped pair terms, for
// the fixed-order split-K reduce to add); its four
// waves split K (wave w takes the 64-wide K-blocks w, w+4, ...) and each
// accumulates the whole tile with v_mfma_f32_16x16x32_f16. Each K-block is
// consumed as two halves of 32; lane (r, g) = (lane % 16, lane / 16) owns
// K-elements k0 + 8 g .. +7 of a half for its A rows and B columns alike.
// Operands come straight from global memory through register rings (A
// three half-blocks ahead, codes four). Every load is unconditional, from
// an index clamped into the arrays (rows past M and channels past N are
// computed and never stored; A past K is replaced by zero, so the padded
// codes there add nothing); a wave's last iterations past its own count
// re-load its last half-block and skip only the arithmetic, in a uniform
// branch that contains no load. The four partial tiles and row sums are
// added in LDS in a fixed order.
#include <type_traits>

#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

namespace {
constexpr int BM = kRowsTileM, BN = kRowsTileN, BK = 64;
constexpr int RF = BM / 16;   // 16-row accumulator tiles per wave
constexpr int CF = BN / 16;   // 16-column accumulator tiles per wave
constexpr int RED_STRIDE = BN + 4;   // floats per LDS row of the reduction
// Register rings, in half-block iterations (32 K-elements): A is loaded
// RA - 1 iterations ahead (RA = 4, or 2 for element loads) and codes RB
// iterations ahead. The main loop is unrolled UNROLL times so every ring
// slot is a fixed register; a wave's trip count is padded to UNROLL with
// clamped re-loads, and since these loads touch 16 rows each (the texture
// path, not bandwidth, limits this kernel) a short unroll keeps that
// padding small.
constexpr int RA_FAST = 4, RB = 4, UNROLL = 4;
}

// 8 Int8 codes (two words, k ascending) -> the fp16 values 1024 + q, exact.
__device__ __forceinline__ h8_t codes_biased(u2_t codes) {
    u4_t o;
    o[0] = __builtin_amdgcn_perm(0x64646464u, codes[0], 0x04010400u);   // q0, q1
    o[1] = __builtin_amdgcn_perm(0x64646464u, codes[0], 0x04030402u);   // q2, q3
    o[2] = __builtin_amdgcn_perm(0x64646464u, codes[1], 0x04010400u);
    o[3] = __builtin_amdgcn_perm(0x64646464u, codes[1], 0x04030402u);
    return __builtin_bit_cast(h8_t, o);
}

// KMODE 0: K % 64 == 0 (no masking); 1: K % 8 == 0 (16-byte pieces, masked
// past K); 2: any K (element loads, masked past K). WF16: the rows hold fp16
// weights (2 bytes each) instead of Int8-Block0 codes.
template <int KMODE, bool WF16>
__global__ __launch_bounds__(256) void gemm_rows_kernel(
    int M, int K, int N, int Kp, int tiles_n, int xcd_order, const _Float16 *__restrict__ A,
    const uint8_t *__restrict__ Wp, const float *__restrict__ Sp, void *__restrict__ C,
    Epilogue epi) {
    // element loads (any K) keep a shallower A ring to stay in registers
    constexpr int RA = KMODE == 2 ? 2 : RA_FAST;
    __shared__ __align__(16) float red[4][BM * RED_STRIDE];   // 4 x 34 KiB
    __shared__ float rsum[4][BM];

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
    // this workgroup's K-blocks [KB0, KB0 + nblk) (all of them unless split)
    const int KB0 = (int)((long long)blockIdx.y * (Kp / BK) / gridDim.y);
    const int nblk = (int)((long long)(blockIdx.y + 1) * (Kp / BK) / gridDim.y) - KB0;
    const int nb_w = nblk > wave ? (nblk - wave + 3) / 4 : 0;   // K-blocks of this wave
    const int n_it = 2 * nb_w;                                   // half-block iterations
    const int n_pad = (n_it + UNROLL - 1) / UNROLL * UNROLL;     // every wave: same unrolled body
    const int it_last = max(n_it - 1, 0);

    // row and channel of each fragment, clamped into the arrays
    const _Float16 *a_row[RF];
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) a_row[rf] = A + (size_t)min(m0 + rf * 16 + r, M - 1) * K;
    constexpr int WB = WF16 ? 2 : 1;          // bytes per weight
    using BV = std::conditional_t<WF16, u4_t, u2_t>;   // one lane's 8 weights
    const uint8_t *b_row[CF];
#pragma unroll
    for (int cf = 0; cf < CF; ++cf) b_row[cf] = Wp + (size_t)min(n0 + cf * 16 + r, N - 1) * Kp * WB;

    // lane (r, g) holds K-elements k0 + 8 g .. k0 + 8 g + 7 of each half-block
    auto k_of = [&](int it) { return (KB0 + wave + 4 * (it >> 1)) * BK + 32 * (it & 1) + 8 * g; };
    auto load_a = [&](u4_t (&dst)[RF], int it) {
        const int k = k_of(it);
#pragma unroll
        for (int rf = 0; rf < RF; ++rf) {
            if (KMODE == 0) {
                dst[rf] = *reinterpret_cast<const u4_t *>(a_row[rf] + k);
            } else if (KMODE == 1) {
                const u4_t v = *reinterpret_cast<const u4_t *>(a_row[rf] + min(k, K - 8));
                const unsigned keep = k < K ? ~0u : 0u;
                dst[rf] = v & keep;
            } else {
                h8_t t8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const _Float16 v = a_row[rf][min(k + e, K - 1)];
                    t8[e] = k + e < K ? v : (_Float16)0.0f;
                }
                dst[rf] = __builtin_bit_cast(u4_t, t8);
            }
        }
    };
    auto load_b = [&](BV (&dst)[CF], int it) {
        const int k = k_of(it);
#pragma unroll
        for (int cf = 0; cf < CF; ++cf) dst[cf] = *reinterpret_cast<const BV *>(b_row[cf] + (size_t)k * WB);
    };

    f4_t acc[RF][CF];
#pragma unroll
    for (int i = 0; i < RF; ++i)
#pragma unroll
        for (int j = 0; j < CF; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};
    float rs[RF];              // row sums of this lane's K-elements
#pragma unroll
    for (int i = 0; i < RF; ++i) rs[i] = 0.f;
    const h2_t ones = {(_Float16)1.0f, (_Float16)1.0f};

    u4_t ra[RA][RF];
    BV rb[RB][CF];
    if (n_it > 0) {            // a wave with no K-block (K < 256) loads nothing
#pragma unroll
        for (int d = 0; d < RA - 1; ++d) load_a(ra[d], min(d, it_last));
#pragma unroll
        for (int d = 0; d < RB; ++d) load_b(rb[d], min(d, it_last));
        // one full wait: the loop header then merges an empty count with the
        // loop's own, and the compiler's in-order count stays exact
        __builtin_amdgcn_s_waitcnt(0);

        for (int base = 0; base < n_pad; base += UNROLL) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int it = base + u;
                load_a(ra[(u + RA - 1) % RA], min(it + RA - 1, it_last));
                h8_t bw[CF];
#pragma unroll
                for (int cf = 0; cf < CF; ++cf) {
                    if constexpr (WF16) bw[cf] = __builtin_bit_cast(h8_t, rb[u % RB][cf]);
                    else bw[cf] = codes_biased(rb[u % RB][cf]);
                }
                const u4_t (&av)[RF] = ra[u % RA];
                if (it < n_it) {
#pragma unroll
                    for (int rf = 0; rf < RF; ++rf) {
                        const h8_t a = __builtin_bit_cast(h8_t, av[rf]);
                        if constexpr (!WF16) {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                rs[rf] = dot2(h2_t{a[2 * e], a[2 * e + 1]}, ones, rs[rf]);
                        }
#pragma unroll
                        for (int cf = 0; cf < CF; ++cf)
                            acc[rf][cf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bw[cf], acc[rf][cf], 0, 0, 0);
                    }
                }
                load_b(rb[u % RB], min(it + RB, it_last));
            }
        }
    }

    // Partial tiles to LDS: accumulator element i of lane l in tile (rf, cf)
    // is P[rf*16 + 4*(l/16) + i][cf*16 + l%16]. Row sums: lanes r, r + 16,
    // r + 32, r + 48 hold disjoint K-elements of row rf*16 + r.
    float *mine = red[wave];
#pragma unroll
    for (int rf = 0; rf < RF; ++rf)
#pragma unroll
        for (int cf = 0; cf < CF; ++cf)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mine[(rf * 16 + 4 * g + i) * RED_STRIDE + cf * 16 + r] = acc[rf][cf][i];
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) {
        float v = rs[rf];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (g == 0) rsum[wave][rf * 16 + r] = v;
    }
    __syncthreads();

    // Sum the four partials (fixed order), apply the channel pairs and store:
    // thread -> row tid/2, 32 consecutive columns. A split-K slice stores its
    // raw partial tile (plain fp32) at slice blockIdx.y of C.
    const int row = tid >> 1;
    const int c0 = (tid & 1) * 32;
    const int gm = m0 + row;
    if (gm >= M) return;
    const bool raw = gridDim.y > 1 || epi.plain;
    const float rsm = ((rsum[0][row] + rsum[1][row]) + rsum[2][row]) + rsum[3][row];
    float *dst = static_cast<float *>(C) + (size_t)blockIdx.y * M * N + (size_t)gm * N + n0 + c0;
    const bool vec_store = (N & 3) == 0 && n0 + c0 + 32 <= N;
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
        const int o = row * RED_STRIDE + c0 + j;
        const f4_t p = *reinterpret_cast<const f4_t *>(&red[0][o]) +
                       *reinterpret_cast<const f4_t *>(&red[1][o]) +
                       *reinterpret_cast<const f4_t *>(&red[2][o]) +
                       *reinterpret_cast<const f4_t *>(&red[3][o]);
        f4_t out;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (WF16) {
                out[e] = p[e];
            } else {
                const f2_t pr = *reinterpret_cast<const f2_t *>(Sp + (size_t)min(n0 + c0 + j + e, N - 1) * 2);
                out[e] = fmaf(pr.y, p[e], fmaf(-1024.0f, pr.y, pr.x) * rsm);
            }
        }
        if (!raw && vec_store) {
            epi_put4(epi, C, gm, n0 + c0 + j, N, out);
        } else if (!raw) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n0 + c0 + j + e < N) epi_put(epi, C, gm, n0 + c0 + j + e, N, out[e]);
        } else if (vec_store) {
            *reinterpret_cast<f4_t *>(dst + j) = out;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n0 + c0 + j + e < N) dst[j + e] = out[e];
        }
    }
}

template <bool WF16>
static hipError_t launch_rows(int M, int K, int N, const void *A, const void *Wp, const void *Sp,
                              void *C, const Epilogue &epi, int nsplit, float *part,
                              hipStream_t s) {
    const int Kp = (int)round_up(K, 64);
    const int tiles_n = div_up(N, BN);
    const int tiles = tiles_n * div_up(M, BM);
    const int xcd_order = (tiles % 8) == 0 ? 1 : 0;
    void *out = nsplit > 1 ? static_cast<void *>(part) : C;
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(tiles, nsplit), dim3(256), 0, s, M, K, N, Kp, tiles_n,
                           xcd_order, static_cast<const _Float16 *>(A),
                           static_cast<const uint8_t *>(Wp), static_cast<const float *>(Sp), out,
                           epi);
    };
    if (K % 64 == 0) launch(gemm_rows_kernel<0, WF16>);
    else if (K % 8 == 0) launch(gemm_rows_kernel<1, WF16>);
    else launch(gemm_rows_kernel<2, WF16>);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || nsplit <= 1) return e;
    return launch_splitk_reduce_f32(part, nsplit, M, N, C, epi, s);
}

hipError_t launch_gemm_int8b0(int M, int K, int N, const void *A, const void *Wp,
                              const void *Sp, void *C, const Epilogue &epi, int nsplit,
                              float *part, hipStream_t s) {
    return launch_rows<false>(M, K, N, A, Wp, Sp, C, epi, nsplit, part, s);
}

hipError_t launch_gemm_f16(int M, int K, int N, const void *A, const void *Wp, void *C,
                           const Epilogue &epi, int nsplit, float *part, hipStream_t s) {
    return launch_rows<true>(M, K, N, A, Wp, nullptr, C, epi, nsplit, part, s);
}

}  // namespace qg
