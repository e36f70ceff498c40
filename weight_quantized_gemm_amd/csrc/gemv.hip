// gemv.hip -- streaming GEMV for the decode shape (M = 1, and small M up to
// the dispatch threshold) with Int4-Block64 and Int8-Block0 weights.
//
// What is computed (MNN GemmSpeed benchmark page, section "Why Conv1x1 is
// used to measure GEMM"): C[m][n] = sum_k A[m][k] * (offset + scale * q[n][k]),
// one [offset, scale] pair per (channel, block). Per block the sum is
// regrouped as offset * sum(a) + scale * sum(a * q), so the per-weight work
// is a code decode and a dot product; offset and scale are applied once per
// block. The page's observation that small M is bounded by the GEMV
// bandwidth floor (section "Sample data") makes this kernel an HBM stream:
// every weight byte is read exactly once, with 16-byte loads that are
// contiguous across the 64 lanes of a wave.
//
// Work split: lane b of a wave owns K-block b (64 K-elements) of every
// channel the wave processes, so a wave covers K = 4096 in one pass; a wave
// takes GPW groups of 4 channels (Int4) or CPW channels (Int8). The lane's 64
// activations are decoded once per block slot and reused for all channels.
// Codes become fp16 by a magic-number decode (one byte permute per pair of
// codes): a 4-bit code placed in mantissa bits 4..7 under exponent 2^10 reads
// as 1024 + 16 q; an 8-bit code in bits 0..7 reads as 1024 + q. The bias is removed per block with the
// block sum of the activations, so no per-weight subtract is needed.
// The partial sums of the 64 lanes are combined by a transposing butterfly
// (each exchange step halves the values a lane holds) before the store.
#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

template <int N>
struct Log2 { static constexpr int value = 1 + Log2<N / 2>::value; };
template <>
struct Log2<1> { static constexpr int value = 0; };

// Sums each of NV per-lane values over the 64 lanes. On return every lane
// holds the total of value `idx`; lanes whose low (6 - log2 NV) bits are zero
// are the ones to store it.
template <int NV>
__device__ __forceinline__ float wave_transpose_sum(float (&v)[NV], int lane, int &idx) {
    constexpr int L = Log2<NV>::value;
    static_assert((1 << L) == NV && L <= 6, "NV must be a power of two <= 64");
    idx = 0;
#pragma unroll
    for (int step = 0; step < L; ++step) {
        const int half = NV >> (step + 1);
        const int off = 32 >> step;
        const bool up = (lane & off) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float keep = up ? v[i + half] : v[i];
            const float send = up ? v[i] : v[i + half];
            v[i] = keep + __shfl_xor(send, off);
        }
        if (up) idx += half;
    }
    float s = v[0];
#pragma unroll
    for (int off = 32 >> L; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    return s;
}

// ---------------------------------------------------------------------------
// Int4-Block64
// ---------------------------------------------------------------------------
template <int MR, int GPW>
__global__ __launch_bounds__(256) void gemv_int4b64_kernel(
    int M, int K, int N, const _Float16 *__restrict__ A, const u4_t *__restrict__ Wp,
    const f4_t *__restrict__ Sp, float *__restrict__ C) {
    extern __shared__ __align__(16) _Float16 As[];   // [MR][K]
    const int tid = threadIdx.x;
    const int m0 = blockIdx.y * MR;
    const int pieces = K >> 3;
    for (int p = tid; p < MR * pieces; p += 256) {
        const int r = p / pieces, c = p - r * pieces;
        u4_t v = {0u, 0u, 0u, 0u};
        if (m0 + r < M)
            v = *reinterpret_cast<const u4_t *>(A + (size_t)(m0 + r) * K + (size_t)c * 8);
        *reinterpret_cast<u4_t *>(As + (size_t)r * K + (size_t)c * 8) = v;
    }
    __syncthreads();

    const int lane = tid & 63;
    const int nblk = K >> 6;
    const int G = (N + 3) >> 2;
    const int g0 = uniform((int)(blockIdx.x * 4 + (tid >> 6)) * GPW);
    if (g0 >= G) return;

    constexpr int NV = GPW * 4 * MR;
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.f;
    const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    // high byte of every fp16 half: exponent 2^10, so a code c in mantissa
    // bits 4..7 reads as 1024 + 16 c
    const unsigned magic = 0x64646464u;

    for (int b = lane; b < nblk; b += 64) {
        // Issue every weight and pair load of this block slot first.
        u4_t wq[GPW][8];
        f4_t pr[GPW][2];
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
            const int g = g0 + gi;
            if (g < G) {
#pragma unroll
                for (int j = 0; j < 8; ++j) wq[gi][j] = Wp[((size_t)g * 8 + j) * nblk + b];
                pr[gi][0] = Sp[((size_t)g * 2 + 0) * nblk + b];
                pr[gi][1] = Sp[((size_t)g * 2 + 1) * nblk + b];
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) wq[gi][j] = u4_t{0u, 0u, 0u, 0u};
                pr[gi][0] = pr[gi][1] = f4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
        // Activations of this block: pairs (a_i, a_{i+4}) of every 8-group,
        // matching the decode below, and the block sum.
        h2_t ap[MR][8][4];
        float s0[MR];
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const u4_t v = *reinterpret_cast<const u4_t *>(As + (size_t)r * K + b * 64 + w * 8);
                const h2_t p01 = as_h2(v.x), p23 = as_h2(v.y), p45 = as_h2(v.z), p67 = as_h2(v.w);
                ap[r][w][0] = h2_t{p01.x, p45.x};
                ap[r][w][1] = h2_t{p01.y, p45.y};
                ap[r][w][2] = h2_t{p23.x, p67.x};
                ap[r][w][3] = h2_t{p23.y, p67.y};
                s = dot2(p01, one, s);
                s = dot2(p23, one, s);
                s = dot2(p45, one, s);
                s = dot2(p67, one, s);
            }
            s0[r] = s;
        }
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float T[MR];
#pragma unroll
                for (int r = 0; r < MR; ++r) T[r] = 0.f;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u4_t ch = wq[gi][2 * c + h];
#pragma unroll
                    for (int wi = 0; wi < 4; ++wi) {
                        const unsigned word = ch[wi];
                        const int w = 4 * h + wi;
                        // even codes q0 q2 q4 q6 / odd codes q1 q3 q5 q7, each in
                        // the high nibble of a byte
                        const unsigned ev = (word << 4) & 0xF0F0F0F0u;
                        const unsigned od = word & 0xF0F0F0F0u;
                        const h2_t x04 = as_h2(__builtin_amdgcn_perm(magic, ev, 0x04020400u));
                        const h2_t x26 = as_h2(__builtin_amdgcn_perm(magic, ev, 0x04030401u));
                        const h2_t x15 = as_h2(__builtin_amdgcn_perm(magic, od, 0x04020400u));
                        const h2_t x37 = as_h2(__builtin_amdgcn_perm(magic, od, 0x04030401u));
#pragma unroll
                        for (int r = 0; r < MR; ++r) {
                            T[r] = dot2(x04, ap[r][w][0], T[r]);
                            T[r] = dot2(x15, ap[r][w][1], T[r]);
                            T[r] = dot2(x26, ap[r][w][2], T[r]);
                            T[r] = dot2(x37, ap[r][w][3], T[r]);
                        }
                    }
                }
                const f4_t rec = pr[gi][c >> 1];
                const float off = (c & 1) ? rec.z : rec.x;
                const float sc = (c & 1) ? rec.w : rec.y;
                // offset*s0 + scale*sum(a q), with T = 1024 s0 + 16 sum(a q)
                const float c1 = fmaf(-64.0f, sc, off);
                const float c2 = sc * 0.0625f;
#pragma unroll
                for (int r = 0; r < MR; ++r)
                    acc[(gi * 4 + c) * MR + r] += fmaf(c1, s0[r], c2 * T[r]);
            }
        }
    }

    int idx;
    const float total = wave_transpose_sum<NV>(acc, lane, idx);
    constexpr int LOW = 6 - Log2<NV>::value;
    if ((lane & ((1 << LOW) - 1)) == 0) {
        const int r = idx % MR;
        const int c = (idx / MR) & 3;
        const int gi = idx / (4 * MR);
        const int n = 4 * (g0 + gi) + c;
        const int m = m0 + r;
        if (n < N && m < M) C[(size_t)m * N + n] = total;
    }
}

// ---------------------------------------------------------------------------
// Int8-Block0
// ---------------------------------------------------------------------------
template <int MR, int CPW>
__global__ __launch_bounds__(256) void gemv_int8b0_kernel(
    int M, int K, int N, int Kp, const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    const f2_t *__restrict__ Sp, float *__restrict__ C) {
    extern __shared__ __align__(16) _Float16 As[];   // [MR][Kp], zero beyond K
    const int tid = threadIdx.x;
    const int m0 = blockIdx.y * MR;
    if ((K & 7) == 0) {
        const int pieces = Kp >> 3;
        for (int p = tid; p < MR * pieces; p += 256) {
            const int r = p / pieces, c = p - r * pieces;
            u4_t v = {0u, 0u, 0u, 0u};
            if (m0 + r < M && c * 8 < K)
                v = *reinterpret_cast<const u4_t *>(A + (size_t)(m0 + r) * K + (size_t)c * 8);
            *reinterpret_cast<u4_t *>(As + (size_t)r * Kp + (size_t)c * 8) = v;
        }
    } else {
        for (int e = tid; e < MR * Kp; e += 256) {
            const int r = e / Kp, k = e - r * Kp;
            As[e] = (m0 + r < M && k < K) ? A[(size_t)(m0 + r) * K + k] : (_Float16)0.0f;
        }
    }
    __syncthreads();

    const int lane = tid & 63;
    const int Np = (N + 3) & ~3;
    const int ch0 = uniform((int)(blockIdx.x * 4 + (tid >> 6)) * CPW);
    if (ch0 >= N) return;
    const int nchunk = Kp >> 4;   // 16-byte chunks per channel
    const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};

    float T[CPW][MR];
    float s0[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        s0[r] = 0.f;
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) T[cc][r] = 0.f;
    }
    for (int ci = lane; ci < nchunk; ci += 64) {
        u4_t wq[CPW];
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc)
            wq[cc] = (ch0 + cc < Np)
                         ? *reinterpret_cast<const u4_t *>(Wp + (size_t)(ch0 + cc) * Kp + (size_t)ci * 16)
                         : u4_t{0u, 0u, 0u, 0u};
        h2_t ap[MR][8];
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const u4_t v0 = *reinterpret_cast<const u4_t *>(As + (size_t)r * Kp + ci * 16);
            const u4_t v1 = *reinterpret_cast<const u4_t *>(As + (size_t)r * Kp + ci * 16 + 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ap[r][i] = as_h2(v0[i]);
                ap[r][4 + i] = as_h2(v1[i]);
                s0[r] = dot2(ap[r][i], one, s0[r]);
                s0[r] = dot2(ap[r][4 + i], one, s0[r]);
            }
        }
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
#pragma unroll
            for (int wi = 0; wi < 4; ++wi) {
                const unsigned word = wq[cc][wi];
                // bytes (q0, q1) and (q2, q3) under 0x64: halves 1024 + q
                const h2_t x0 = as_h2(__builtin_amdgcn_perm(0x64646464u, word, 0x04010400u));
                const h2_t x1 = as_h2(__builtin_amdgcn_perm(0x64646464u, word, 0x04030402u));
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    T[cc][r] = dot2(x0, ap[r][2 * wi], T[cc][r]);
                    T[cc][r] = dot2(x1, ap[r][2 * wi + 1], T[cc][r]);
                }
            }
        }
    }

    constexpr int NV = CPW * MR;
    float acc[NV];
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
        f2_t pr = {0.f, 0.f};
        if (ch0 + cc < Np) pr = Sp[ch0 + cc];
        // offset*s0 + scale*sum(a q), with T = 1024 s0 + sum(a q)
        const float c1 = fmaf(-1024.0f, pr.y, pr.x);
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[cc * MR + r] = fmaf(c1, s0[r], pr.y * T[cc][r]);
    }
    int idx;
    const float total = wave_transpose_sum<NV>(acc, lane, idx);
    constexpr int LOW = 6 - Log2<NV>::value;
    if ((lane & ((1 << LOW) - 1)) == 0) {
        const int r = idx % MR;
        const int cc = idx / MR;
        const int n = ch0 + cc;
        const int m = m0 + r;
        if (n < N && m < M) C[(size_t)m * N + n] = total;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static int rows_per_pass(int M, int K, int kp_bytes_per_row) {
    // Rows of A staged in LDS at once, bounded by 64 KiB of LDS.
    (void)K;
    int mr = M >= 4 ? 4 : (M >= 2 ? 2 : 1);
    while (mr > 1 && mr * kp_bytes_per_row > 65536) mr >>= 1;
    return mr;
}

template <int MR>
static hipError_t gemv_int4_mr(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, float *C, hipStream_t s) {
    constexpr int GPW = 2;
    const int G = (N + 3) / 4;
    const int waves = div_up(G, GPW);
    dim3 grid(div_up(waves, 4), div_up(M, MR));
    const size_t lds = (size_t)MR * K * sizeof(_Float16);
    hipLaunchKernelGGL((gemv_int4b64_kernel<MR, GPW>), grid, dim3(256), lds, s, M, K, N,
                       static_cast<const _Float16 *>(A), static_cast<const u4_t *>(Wp),
                       static_cast<const f4_t *>(Sp), C);
    return hipGetLastError();
}

hipError_t launch_gemv_int4b64(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, float *C, hipStream_t s) {
    switch (rows_per_pass(M, K, K * 2)) {
    case 4: return gemv_int4_mr<4>(M, K, N, A, Wp, Sp, C, s);
    case 2: return gemv_int4_mr<2>(M, K, N, A, Wp, Sp, C, s);
    default: return gemv_int4_mr<1>(M, K, N, A, Wp, Sp, C, s);
    }
}

template <int MR>
static hipError_t gemv_int8_mr(int M, int K, int N, int Kp, const void *A, const void *Wp,
                               const void *Sp, float *C, hipStream_t s) {
    constexpr int CPW = 4;
    const int waves = div_up(N, CPW);
    dim3 grid(div_up(waves, 4), div_up(M, MR));
    const size_t lds = (size_t)MR * Kp * sizeof(_Float16);
    hipLaunchKernelGGL((gemv_int8b0_kernel<MR, CPW>), grid, dim3(256), lds, s, M, K, N, Kp,
                       static_cast<const _Float16 *>(A), static_cast<const uint8_t *>(Wp),
                       static_cast<const f2_t *>(Sp), C);
    return hipGetLastError();
}

hipError_t launch_gemv_int8b0(int M, int K, int N, const void *A, const void *Wp,
                              const void *Sp, float *C, hipStream_t s) {
    const int Kp = (int)round_up(K, 64);
    switch (rows_per_pass(M, K, Kp * 2)) {
    case 4: return gemv_int8_mr<4>(M, K, N, Kp, A, Wp, Sp, C, s);
    case 2: return gemv_int8_mr<2>(M, K, N, Kp, A, Wp, Sp, C, s);
    default: return gemv_int8_mr<1>(M, K, N, Kp, A, Wp, Sp, C, s);
    }
}

}  // namespace qg
