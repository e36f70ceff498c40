// gemm_int8.hip -- prefill GEMM (M above the GEMV threshold) for weights
// stored as channel rows [Np][Kp] on the fp16 matrix cores: Int8-Block0
// codes, fp16 weights (the float mode at FP16 precision, which the same
// kernel multiplies as they are, with no pair and no regrouping), or Int8
// codes with a pair per block of K (dequantised per weight in registers, see
// gemm_rows_kernel's PM mode).
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
// the fixed-order split-K reduce to add). Its four waves split K (wave w
// takes the 64-wide K-blocks w, w+4, ...) and each accumulates the whole tile
// with v_mfma_f32_16x16x32_f16, so no wave shares an operand with another
// and the loop has no barrier:
//  - a wave's A block (128 rows x 64 K-elements) arrives with fully coalesced
//    loads (8 rows x 128 bytes per instruction; rows of 64 bytes, as the MFMA
//    lane layout would read them, take about 1.7x as long on this chip) two
//    blocks ahead through a register ring, and passes through the wave's own
//    two LDS tiles into the MFMA lane layout;
//  - B comes straight from the channel rows, one 16-byte load per lane and
//    block for the codes (two for fp16 weights), also two blocks ahead;
//  - lane (r, g) = (lane % 16, lane / 16) holds K-elements 16 g + 8 s .. +7
//    of a block in MFMA step s (s = 0, 1), for its A row and B column alike
//    (the K order inside an MFMA only has to agree between the operands).
// Every global load is unconditional, from an index clamped into the arrays
// (rows past M and channels past N are computed and never stored; A past K is
// replaced by zero, so the padded codes there add nothing); a wave's last
// iterations past its own count re-load its last block and skip only the
// arithmetic, in a uniform branch that contains no load. The four partial
// tiles and row sums are added in LDS in a fixed order.
#include <type_traits>

#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

namespace {
constexpr int BM = kRowsTileM, BN = kRowsTileN, BK = 64;
constexpr int RF = BM / 16;   // 16-row accumulator tiles per wave
constexpr int CF = BN / 16;   // 16-column accumulator tiles per wave
constexpr int RED_STRIDE = BN + 4;   // floats per LDS row of the reduction
constexpr int AS_STRIDE = BK + 8;    // halves per LDS row of an A tile (144 bytes)
constexpr int A_TILE = BM * AS_STRIDE;            // halves per A tile
constexpr int A_PIECES = BM * BK / 8 / 64;        // 16-byte A pieces per lane and block (16)
// A and B are loaded DEPTH blocks ahead through register rings; the loop is
// unrolled DEPTH times so every ring slot is a fixed register, and each wave
// has DEPTH LDS tiles for A. The any-K mode (KMODE 2) loads A element by
// element, eight registers per 16-byte piece, and keeps one block in flight
// (two would not fit the register file beside the accumulators).
constexpr int DEPTH = 2;
template <int KMODE>
constexpr int depth_of() { return KMODE == 2 ? 1 : DEPTH; }
constexpr size_t A_LDS = (size_t)4 * DEPTH * A_TILE * 2;
constexpr size_t RED_LDS = (size_t)4 * BM * RED_STRIDE * 4 + (size_t)4 * BM * 4;
constexpr size_t ROWS_LDS = A_LDS > RED_LDS ? A_LDS : RED_LDS;
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

// 8 fp16 values 1024 + q -> the weights offset + scale * q, each one fp32
// fused multiply-add x * scale + b (b = offset - 1024 scale, folded once per
// block) rounded once to fp16.
__device__ __forceinline__ h8_t dequant8_biased(h8_t x, float scale, float b) {
    h8_t w;
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = (_Float16)fmaf((float)x[e], scale, b);
    return w;
}

// KMODE: 0: K % 64 == 0 (16-byte loads, no mask); 1: K % 8 == 0 (16-byte
// loads, pieces past K masked); 2: any K (element loads, masked past K).
// WF16: the rows hold fp16 weights (2 bytes each) instead of Int8-Block0 codes.
// PM (blocked Int8, KMODE 0): the rows hold Int8 codes with a pair per
// 64-block (PM = 1), per 32-element half (PM = 2) or per 16-element quarter
// (PM = 4), channel-major; each
// lane dequantises its 16 codes of a block with their pair (one fused
// multiply-add per weight, rounded once to fp16) and the MFMAs take the
// weights, so the epilogue adds no pair term.
template <int KMODE, bool WF16, int PM = 0>
__global__ __launch_bounds__(256) void gemm_rows_kernel(
    int M, int K, int N, int Kp, int tiles_n, const _Float16 *__restrict__ A,
    const uint8_t *__restrict__ Wp, const float *__restrict__ Sp, void *__restrict__ C,
    Epilogue epi) {
    __shared__ __align__(16) unsigned char lds[ROWS_LDS];
    constexpr int DEPTH = depth_of<KMODE>();

    // Tile of this workgroup: plain row-major order (the hardware deals
    // workgroups to the eight XCDs round-robin). Giving each XCD a contiguous
    // run of tiles instead measured slower with fp16 weights (38.1 against
    // 35.5 us at 512 x 4096 x 4096, 196.6 against 188.8 us at 1024 x 4096 x
    // 11008, one box) and no different with Int8-Block0.
    const int t = blockIdx.x;
    const int m0 = (t / tiles_n) * BM;
    const int n0 = (t % tiles_n) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    // this workgroup's K-blocks [KB0, KB0 + nblk) (all of them unless split)
    const int KB0 = slice_begin(blockIdx.y, Kp / BK, gridDim.y);
    const int nblk = slice_begin(blockIdx.y + 1, Kp / BK, gridDim.y) - KB0;
    const int n_it = nblk > wave ? (nblk - wave + 3) / 4 : 0;    // K-blocks of this wave
    const int n_pad = (n_it + DEPTH - 1) / DEPTH * DEPTH;          // every wave: same unrolled body
    const int it_last = max(n_it - 1, 0);
    auto k_of = [&](int it) { return (KB0 + wave + 4 * it) * BK; };   // first K-element of a block

    // A loader role: piece i of a block is row 8 i + lane / 8, elements
    // 8 (lane % 8) .. +7 of the block's 64 (128 bytes per row)
    const int prow = lane >> 3, ppc = lane & 7;
    const _Float16 *a_row[A_PIECES];
#pragma unroll
    for (int i = 0; i < A_PIECES; ++i) a_row[i] = A + (size_t)min(m0 + 8 * i + prow, M - 1) * K;
    constexpr int WB = WF16 ? 2 : 1;                  // bytes per weight
    constexpr int BV = WF16 ? 2 : 1;                  // 16-byte loads per lane, column tile and block
    const uint8_t *b_row[CF];
#pragma unroll
    for (int cf = 0; cf < CF; ++cf)
        b_row[cf] = Wp + ((size_t)min(n0 + cf * 16 + r, N - 1) * Kp + 16 * g) * WB;
    // PM: this lane's pair entries, channel n0 + 16 cf + r, sub-block g PM / 4
    // of each 64-block (the lane's 16 codes lie in one quarter)
    constexpr int H = PM ? PM : 1;
    const f2_t *p_row[PM ? CF : 1];
    if constexpr (PM != 0) {
#pragma unroll
        for (int cf = 0; cf < CF; ++cf)
            p_row[cf] = reinterpret_cast<const f2_t *>(Sp) +
                        (size_t)min(n0 + cf * 16 + r, N - 1) * (Kp / BK) * H + g * H / 4;
    }
    auto load_p = [&](f2_t (&dst)[PM ? CF : 1], int it) {
        if constexpr (PM != 0) {
#pragma unroll
            for (int cf = 0; cf < CF; ++cf) dst[cf] = p_row[cf][(size_t)(k_of(it) / BK) * H];
        }
    };

    auto load_a = [&](u4_t (&dst)[A_PIECES], int it) {
        const int k = k_of(it) + 8 * ppc;
#pragma unroll
        for (int i = 0; i < A_PIECES; ++i) {
            if (KMODE == 0) {
                dst[i] = *reinterpret_cast<const u4_t *>(a_row[i] + k);
            } else if (KMODE == 1) {
                const u4_t v = *reinterpret_cast<const u4_t *>(a_row[i] + min(k, K - 8));
                dst[i] = v & (k < K ? ~0u : 0u);
            } else {
                h8_t t8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const _Float16 v = a_row[i][min(k + e, K - 1)];
                    t8[e] = k + e < K ? v : (_Float16)0.0f;
                }
                dst[i] = __builtin_bit_cast(u4_t, t8);
                // element loads: at most four pieces (32 loads) in flight, so
                // their destination registers fit beside the accumulators
                if (i % 4 == 3) __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    auto load_b = [&](u4_t (&dst)[CF][BV], int it) {
        const size_t k = (size_t)k_of(it) * WB;
#pragma unroll
        for (int cf = 0; cf < CF; ++cf)
#pragma unroll
            for (int v = 0; v < BV; ++v) dst[cf][v] = *reinterpret_cast<const u4_t *>(b_row[cf] + k + 16 * v);
    };
    _Float16 *const a_tiles = reinterpret_cast<_Float16 *>(lds) + (size_t)wave * DEPTH * A_TILE;

    f4_t acc[RF][CF];
#pragma unroll
    for (int i = 0; i < RF; ++i)
#pragma unroll
        for (int j = 0; j < CF; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};
    float rs[RF];              // row sums of this lane's K-elements
#pragma unroll
    for (int i = 0; i < RF; ++i) rs[i] = 0.f;
    const h2_t ones = {(_Float16)1.0f, (_Float16)1.0f};

    u4_t ra[DEPTH][A_PIECES];
    u4_t rb[DEPTH][CF][BV];
    f2_t rp[DEPTH][PM ? CF : 1];
    if (n_it > 0) {            // a wave with no K-block (K < 256) loads nothing
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            load_a(ra[d], min(d, it_last));
            load_b(rb[d], min(d, it_last));
            load_p(rp[d], min(d, it_last));
        }
        // one full wait: the loop header then merges an empty count with the
        // loop's own, and the compiler's in-order count stays exact (the
        // scheduling barriers keep the loads above the wait)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_sched_barrier(0);

        // a do-while (n_pad >= DEPTH here): no guard branch in front of the
        // loop, so the loads above cannot be sunk below the wait
        int base = 0;
        do {
#pragma unroll
            for (int u = 0; u < DEPTH; ++u) {
                const int it = base + u;
                // 1. this block's A into the wave's tile u (the LDS operations of
                //    one wave run in order, so the tile's reads of DEPTH blocks
                //    ago are done)
                _Float16 *At = a_tiles + (size_t)u * A_TILE;
#pragma unroll
                for (int i = 0; i < A_PIECES; ++i)
                    *reinterpret_cast<u4_t *>(At + (8 * i + prow) * AS_STRIDE + 8 * ppc) = ra[u][i];
                // 2. this block's B operands; then both ring slots take block it + DEPTH
                h8_t bw[CF][2];
#pragma unroll
                for (int cf = 0; cf < CF; ++cf) {
                    if constexpr (WF16) {
                        bw[cf][0] = __builtin_bit_cast(h8_t, rb[u][cf][0]);
                        bw[cf][1] = __builtin_bit_cast(h8_t, rb[u][cf][BV - 1]);
                    } else if constexpr (PM != 0) {
                        const float sc = rp[u][cf].y, b = fmaf(-1024.0f, sc, rp[u][cf].x);
                        bw[cf][0] = dequant8_biased(codes_biased(u2_t{rb[u][cf][0][0], rb[u][cf][0][1]}), sc, b);
                        bw[cf][1] = dequant8_biased(codes_biased(u2_t{rb[u][cf][0][2], rb[u][cf][0][3]}), sc, b);
                    } else {
                        bw[cf][0] = codes_biased(u2_t{rb[u][cf][0][0], rb[u][cf][0][1]});
                        bw[cf][1] = codes_biased(u2_t{rb[u][cf][0][2], rb[u][cf][0][3]});
                    }
                }
                load_a(ra[u], min(it + DEPTH, it_last));
                load_b(rb[u], min(it + DEPTH, it_last));
                load_p(rp[u], min(it + DEPTH, it_last));
                // 3. two MFMA steps: lane (r, g) takes K-elements 16 g + 8 s .. +7
                if (it < n_it) {       // uniform; no global load inside
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
                        for (int rf = 0; rf < RF; ++rf) {
                            const h8_t a = *reinterpret_cast<const h8_t *>(
                                At + (rf * 16 + r) * AS_STRIDE + 16 * g + 8 * s2);
                            if constexpr (!WF16 && PM == 0) {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    rs[rf] = dot2(h2_t{a[2 * e], a[2 * e + 1]}, ones, rs[rf]);
                            }
#pragma unroll
                            for (int cf = 0; cf < CF; ++cf)
                                acc[rf][cf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bw[cf][s2], acc[rf][cf], 0, 0, 0);
                        }
                    }
                }
            }
            base += DEPTH;
        } while (base < n_pad);
    }

    // Partial tiles to LDS (over the A tiles, once every wave is done with
    // them): accumulator element i of lane l in tile (rf, cf) is
    // P[rf*16 + 4*(l/16) + i][cf*16 + l%16]. Row sums: lanes r, r + 16,
    // r + 32, r + 48 hold disjoint K-elements of row rf*16 + r.
    __syncthreads();
    float (*red)[BM * RED_STRIDE] = reinterpret_cast<float (*)[BM * RED_STRIDE]>(lds);
    float (*rsum)[BM] = reinterpret_cast<float (*)[BM]>(lds + (size_t)4 * BM * RED_STRIDE * 4);
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

    // Sum the four partials (fixed order), apply the channel pairs and store.
    // Each pass covers 16 whole rows, lane -> 16 consecutive bytes of a row,
    // so one store instruction writes whole rows of the tile contiguously. A
    // split-K slice stores its raw partial tile (plain fp32) at slice
    // blockIdx.y of C.
    constexpr int CPT = BN / 4, RPI = 256 / CPT;
    static_assert(BM % RPI == 0, "whole passes");
    const int c4 = tid % CPT, r0 = tid / CPT;
    const int gc = n0 + 4 * c4;
    const bool raw = gridDim.y > 1 || epi.plain;
    const bool vec_store = (N & 3) == 0 && gc + 4 <= N;
    float *const out_base = static_cast<float *>(C) + (size_t)blockIdx.y * M * N;
    f2_t pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (WF16 || PM != 0) pr[e] = f2_t{0.0f, 0.0f};
        else pr[e] = *reinterpret_cast<const f2_t *>(Sp + (size_t)min(gc + e, N - 1) * 2);
    }
#pragma unroll
    for (int it = 0; it < BM / RPI; ++it) {
        const int row = it * RPI + r0;
        const int gm = m0 + row;
        if (gm >= M) break;
        const float rsm = ((rsum[0][row] + rsum[1][row]) + rsum[2][row]) + rsum[3][row];
        const int o = row * RED_STRIDE + 4 * c4;
        const f4_t p = *reinterpret_cast<const f4_t *>(&red[0][o]) +
                       *reinterpret_cast<const f4_t *>(&red[1][o]) +
                       *reinterpret_cast<const f4_t *>(&red[2][o]) +
                       *reinterpret_cast<const f4_t *>(&red[3][o]);
        f4_t out;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (WF16 || PM != 0) out[e] = p[e];
            else out[e] = fmaf(pr[e].y, p[e], fmaf(-1024.0f, pr[e].y, pr[e].x) * rsm);
        }
        float *dst = out_base + (size_t)gm * N + gc;
        if (!raw && vec_store) {
            epi_put4(epi, C, gm, gc, N, out);
        } else if (!raw) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (gc + e < N) epi_put(epi, C, gm, gc + e, N, out[e]);
        } else if (vec_store) {
            __builtin_nontemporal_store(out, reinterpret_cast<f4_t *>(dst));   // C is not read again here
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (gc + e < N) __builtin_nontemporal_store(out[e], dst + e);
        }
    }
}

template <bool WF16, int PM = 0>
static hipError_t launch_rows(int M, int K, int N, const void *A, const void *Wp, const void *Sp,
                              void *C, const Epilogue &epi, int nsplit, float *part,
                              hipStream_t s) {
    const int Kp = (int)round_up(K, 64);
    const int tiles_n = div_up(N, BN);
    const int tiles = tiles_n * div_up(M, BM);
    void *out = nsplit > 1 ? static_cast<void *>(part) : C;
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(tiles, nsplit), dim3(256), 0, s, M, K, N, Kp, tiles_n,
                           static_cast<const _Float16 *>(A),
                           static_cast<const uint8_t *>(Wp), static_cast<const float *>(Sp), out,
                           epi);
    };
    if constexpr (PM != 0) launch(gemm_rows_kernel<0, false, PM>);   // K % 64 == 0
    else if (K % 64 == 0) launch(gemm_rows_kernel<0, WF16>);
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

hipError_t launch_gemm_int8blk(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, void *C, const Epilogue &epi, int pair_g,
                               int nsplit, float *part, hipStream_t s) {
    return pair_g == 4 ? launch_rows<false, 4>(M, K, N, A, Wp, Sp, C, epi, nsplit, part, s)
         : pair_g == 2 ? launch_rows<false, 2>(M, K, N, A, Wp, Sp, C, epi, nsplit, part, s)
                       : launch_rows<false, 1>(M, K, N, A, Wp, Sp, C, epi, nsplit, part, s);
}

}  // namespace qg
