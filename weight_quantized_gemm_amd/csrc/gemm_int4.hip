// gemm_int4.hip -- prefill GEMM for Int4-Block64 weights on the fp16 matrix
// cores (M above the GEMV threshold).
//
// What is computed (MNN GemmSpeed benchmark page, section "Why Conv1x1 is
// used to measure GEMM"): C = A x deq(B), deq(B)[k][n] = offset + scale * q
// with one [offset, scale] pair per 64 K-elements per channel. The weight is
// formed in fp32 (one fused multiply-add from the fp32 pair) and rounded
// once to fp16; A is fp16 already, so the fp16 operands are exact copies of
// A and the nearest fp16 of each weight. The fp32 MFMA accumulators are never
// narrowed and C is stored as fp32 (the SimdPaddleOCR pull request keeps fp16
// tiles exact and never narrows accumulators before the epilogue).
//
// Decomposition, chosen from what limits this shape on CDNA4 (a 512 x 4096
// output gives each of 256 CUs only 8192 outputs, so operand traffic from L2
// bounds the kernel before the matrix cores do):
//  - a 256-thread workgroup owns a 64 x 128 tile of C (a taller-than-wide
//    tile would read A from L2 twice as often);
//  - its four waves split K into contiguous quarters and each accumulates
//    the whole 64 x 128 tile with v_mfma_f32_32x32x16_f16 (2 x 4 accumulator
//    tiles), so every A and B element is fetched and dequantised once per
//    workgroup;
//  - A rows are fetched with fully coalesced loads (8 rows x 128 bytes per
//    instruction) into a wave-private LDS tile and read back in the operand
//    layout; a wave only reads what it wrote, so no barrier is needed;
//  - a K-block of a 32-channel B tile is one contiguous 1 KiB record already
//    in operand lane order (see the packed layout), fetched three blocks
//    ahead through a register ring;
//  - the four partial tiles meet in LDS and are summed in a fixed order.
// Lane (r, h) = (lane % 32, lane / 32) holds K-elements 32 h + 8 s .. +7 of
// every 64-wide block in MFMA step s, for its A row and B column alike (the K
// order inside an MFMA only has to agree between A and B).
//
// The 256 tiles of a 512 x 4096 output are dealt so that each XCD (the
// hardware deals workgroups to XCDs round-robin) owns a band of four B
// tiles across all row tiles: B is read from HBM once and A stays in L2.
#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

namespace {
constexpr int BM = 64, BN = 128, BK = 64;
constexpr int RF = BM / 32;            // 32-row accumulator tiles per wave
constexpr int CF = BN / 32;            // 32-column accumulator tiles per wave
constexpr int AS_STRIDE = BK + 8;      // halves per LDS row of the A tile (144 bytes)
constexpr int RED_STRIDE = BN + 4;     // floats per LDS row of the reduction
constexpr int RING = 4;                // B register ring (3 blocks ahead)
constexpr size_t AS_BYTES = (size_t)BM * AS_STRIDE * 2;          // one A tile
constexpr size_t RED_BYTES = (size_t)4 * BM * RED_STRIDE * 4;    // all waves
constexpr size_t LDS_BYTES = RED_BYTES > 8 * AS_BYTES ? RED_BYTES : 8 * AS_BYTES;

// Per (channel tile, block) dequantisation constants. Even codes decode as
// x = 1024 + q and odd codes as x = 1024 + 16 q (the nibble is left in
// place), so w = offset + scale * q is x * s_lo + b_lo or x * s_hi + b_hi.
struct DqParams {
    float s_lo, b_lo, s_hi, b_hi;
};

__device__ __forceinline__ DqParams dq_params(f2_t pair) {
    const float off = pair.x, sc = pair.y;
    return {sc, fmaf(-1024.0f, sc, off), sc * 0.0625f, fmaf(-64.0f, sc, off)};
}
}

// 8 Int4 codes (one word, k ascending, low nibble first) -> 8 fp16 weights
// in k order, each one fp32 fused multiply-add rounded once to fp16. m_lo,
// m_hi and magic are the constants 0x000F000F, 0x00F000F0 and 0x64006400 held
// in registers, so each pair of codes costs one v_and_or_b32.
__device__ __forceinline__ h8_t dequant8(unsigned word, const DqParams &p, unsigned m_lo,
                                         unsigned m_hi, unsigned magic) {
    const unsigned w8 = word >> 8;
    const h2_t x0 = as_h2((word & m_lo) | magic);   // codes 0, 4 -> 1024 + q
    const h2_t x1 = as_h2((word & m_hi) | magic);   // codes 1, 5 -> 1024 + 16 q
    const h2_t x2 = as_h2((w8 & m_lo) | magic);     // codes 2, 6
    const h2_t x3 = as_h2((w8 & m_hi) | magic);     // codes 3, 7
    h8_t o;
    o[0] = (_Float16)fmaf((float)x0.x, p.s_lo, p.b_lo);
    o[1] = (_Float16)fmaf((float)x1.x, p.s_hi, p.b_hi);
    o[2] = (_Float16)fmaf((float)x2.x, p.s_lo, p.b_lo);
    o[3] = (_Float16)fmaf((float)x3.x, p.s_hi, p.b_hi);
    o[4] = (_Float16)fmaf((float)x0.y, p.s_lo, p.b_lo);
    o[5] = (_Float16)fmaf((float)x1.y, p.s_hi, p.b_hi);
    o[6] = (_Float16)fmaf((float)x2.y, p.s_lo, p.b_lo);
    o[7] = (_Float16)fmaf((float)x3.y, p.s_hi, p.b_hi);
    return o;
}

__global__ __launch_bounds__(256) void gemm_int4b64_kernel(
    int M, int K, int N, int tiles_m, int tiles_n, int xcd_bands,
    const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ Sp, float *__restrict__ C) {
    __shared__ __align__(16) unsigned char lds[LDS_BYTES];

    // ---- tile of this workgroup ----
    const int L = blockIdx.x;
    int tm, tn;
    if (xcd_bands) {
        // XCD x = L % 8 owns B tiles [x * bw, (x + 1) * bw) for every row tile
        const int bw = tiles_n / 8;
        const int j = L / 8;
        tn = (L % 8) * bw + j % bw;
        tm = j / bw;
    } else {
        tm = L / tiles_n;
        tn = L % tiles_n;
    }
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int r = lane & 31, h = lane >> 5;
    const int nblk = K / BK;
    const int kb0 = wave * nblk / 4, kb1 = (wave + 1) * nblk / 4;   // contiguous quarter
    const int nb = kb1 - kb0;
    const int ntiles_b = (N + 31) / 32;                              // packed 32-channel tiles

    // two A tiles per wave: block i is read from tile i % 2 while block i + 1
    // is written into the other
    _Float16 *As0 = reinterpret_cast<_Float16 *>(lds + (2 * wave) * AS_BYTES);
    _Float16 *As1 = reinterpret_cast<_Float16 *>(lds + (2 * wave + 1) * AS_BYTES);

    // A loader role: 8 rows x 128 bytes per instruction, lane -> (row, 16 B
    // piece); byte offsets from the tile's first row (rows past M are
    // clamped: loaded, never stored).
    const int arow = lane >> 3, apc = lane & 7;
    const char *A_tile = reinterpret_cast<const char *>(A + (size_t)m0 * K);
    unsigned a_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        a_off[i] = (unsigned)(min(8 * i + arow, M - 1 - m0) * K + 8 * apc) * 2u;
    // B: tile index of each accumulator column tile (tiles past N: loaded, never stored)
    size_t b_rec0[CF];
#pragma unroll
    for (int cf = 0; cf < CF; ++cf) b_rec0[cf] = (size_t)min(n0 / 32 + cf, ntiles_b - 1) * nblk;

    auto load_a = [&](u4_t (&dst)[8], int kt) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            dst[i] = *reinterpret_cast<const u4_t *>(A_tile + a_off[i] + (unsigned)kt * (BK * 2));
    };
    auto store_a = [&](_Float16 *As, const u4_t (&src)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<u4_t *>(As + (8 * j + arow) * AS_STRIDE + 8 * apc) = src[j];
    };
    auto read_a = [&](const _Float16 *As, int s, h8_t (&af)[RF]) {
#pragma unroll
        for (int rf = 0; rf < RF; ++rf)
            af[rf] = *reinterpret_cast<const h8_t *>(As + (32 * rf + r) * AS_STRIDE + 32 * h + 8 * s);
    };
    auto load_b = [&](u4_t (&codes)[CF], f2_t (&pairs)[CF], int kt) {
#pragma unroll
        for (int cf = 0; cf < CF; ++cf) {
            const size_t rec = b_rec0[cf] + kt;
            codes[cf] = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(Wp + rec * 1024) + lane);
            pairs[cf] = *reinterpret_cast<const f2_t *>(Sp + rec * 64 + r * 2);
        }
    };

    // decode constants, opaque to the optimiser so they stay in registers
    unsigned m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, magic = 0x64006400u;
    asm volatile("" : "+s"(m_lo), "+s"(m_hi));
    asm volatile("" : "+v"(magic));

    f16_t acc[RF][CF];
#pragma unroll
    for (int i = 0; i < RF; ++i)
#pragma unroll
        for (int j = 0; j < CF; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    if (nb > 0) {
        u4_t an[8];
        u4_t bc[RING][CF];
        f2_t bp[RING][CF];
        DqParams prm[CF];
        h8_t acur[RF], anxt[RF], bcur[CF], bnxt[CF];

        // prologue: A of the first block in LDS, A of the second in flight,
        // B of the first RING - 1 blocks in flight, step (0, 0) operands
        // ready. Ring slots past the last block hold that block again, so
        // every slot always decodes to finite weights.
        load_a(an, kb0);
#pragma unroll
        for (int d = 0; d < RING - 1; ++d) load_b(bc[d], bp[d], kb0 + min(d, nb - 1));
        // the last slot is otherwise first filled inside the loop, and only
        // when that block exists
        if (nb < RING) load_b(bc[RING - 1], bp[RING - 1], kb1 - 1);
        store_a(As0, an);
        if (nb > 1) {
            load_a(an, kb0 + 1);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) an[j] = u4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int cf = 0; cf < CF; ++cf) prm[cf] = dq_params(bp[0][cf]);
        read_a(As0, 0, acur);
#pragma unroll
        for (int cf = 0; cf < CF; ++cf) bcur[cf] = dequant8(bc[0][cf][0], prm[cf], m_lo, m_hi, magic);

        // The block count is padded to a multiple of RING so the unrolled
        // loop has a single exit; a padded block has an all-zero A tile and
        // adds exactly zero to every accumulator.
        const int nb_pad = (nb + RING - 1) / RING * RING;
        for (int base = 0; base < nb_pad; base += RING) {
#pragma unroll
            for (int u = 0; u < RING; ++u) {
                const int i = base + u;
                _Float16 *As_cur = (u & 1) ? As1 : As0;
                _Float16 *As_nxt = (u & 1) ? As0 : As1;
                // block i + 1's A into the other tile (its global loads were
                // issued a block ago), then the loads for blocks i + 2 (A)
                // and i + RING - 1 (B, into the slot block i - 1 has freed)
                store_a(As_nxt, an);
                if (i + 2 < nb) {
                    load_a(an, kb0 + i + 2);
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) an[j] = u4_t{0, 0, 0, 0};
                }
                if (i + RING - 1 < nb)
                    load_b(bc[(u + RING - 1) % RING], bp[(u + RING - 1) % RING], kb0 + i + RING - 1);
                // four MFMA steps; while the matrix cores work on step s the
                // operands of the next step (this block's s + 1, or the next
                // block's step 0) are read and dequantised
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (s < 3) {
                        read_a(As_cur, s + 1, anxt);
#pragma unroll
                        for (int cf = 0; cf < CF; ++cf)
                            bnxt[cf] = dequant8(bc[u][cf][s + 1], prm[cf], m_lo, m_hi, magic);
                    } else {
                        const int un = (u + 1) % RING;
                        read_a(As_nxt, 0, anxt);
#pragma unroll
                        for (int cf = 0; cf < CF; ++cf) {
                            prm[cf] = dq_params(bp[un][cf]);
                            bnxt[cf] = dequant8(bc[un][cf][0], prm[cf], m_lo, m_hi, magic);
                        }
                    }
#pragma unroll
                    for (int rf = 0; rf < RF; ++rf)
#pragma unroll
                        for (int cf = 0; cf < CF; ++cf)
                            acc[rf][cf] = __builtin_amdgcn_mfma_f32_32x32x16_f16(acur[rf], bcur[cf], acc[rf][cf], 0, 0, 0);
                    // one MFMA, then up to seven VALU instructions, eight times
#pragma unroll
                    for (int j = 0; j < RF * CF; ++j) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
                    }
#pragma unroll
                    for (int rf = 0; rf < RF; ++rf) acur[rf] = anxt[rf];
#pragma unroll
                    for (int cf = 0; cf < CF; ++cf) bcur[cf] = bnxt[cf];
                }
            }
        }
    }

    // ---- the four partial tiles to LDS (reusing the A tiles' space) ----
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds) + (size_t)wave * BM * RED_STRIDE;
#pragma unroll
    for (int rf = 0; rf < RF; ++rf)
#pragma unroll
        for (int cf = 0; cf < CF; ++cf)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                red[(32 * rf + 8 * (e >> 2) + 4 * h + (e & 3)) * RED_STRIDE + 32 * cf + r] = acc[rf][cf][e];
    __syncthreads();

    // ---- sum in a fixed order and store: thread -> row tid / 4, 32 columns ----
    const int row = tid >> 2;
    const int c0 = (tid & 3) * 32;
    const int gm = m0 + row;
    if (gm >= M) return;
    const float *red0 = reinterpret_cast<const float *>(lds);
    float *dst = C + (size_t)gm * N + n0 + c0;
    const bool vec_store = (N & 3) == 0 && n0 + c0 + 32 <= N;
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
        const size_t o = (size_t)row * RED_STRIDE + c0 + j;
        const size_t W = (size_t)BM * RED_STRIDE;
        const f4_t sum = *reinterpret_cast<const f4_t *>(red0 + o) +
                         *reinterpret_cast<const f4_t *>(red0 + W + o) +
                         *reinterpret_cast<const f4_t *>(red0 + 2 * W + o) +
                         *reinterpret_cast<const f4_t *>(red0 + 3 * W + o);
        if (vec_store) {
            *reinterpret_cast<f4_t *>(dst + j) = sum;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n0 + c0 + j + e < N) dst[j + e] = sum[e];
        }
    }
}

hipError_t launch_gemm_int4b64(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, float *C, hipStream_t s) {
    const int tiles_m = div_up(M, BM), tiles_n = div_up(N, BN);
    const int xcd_bands = (tiles_n % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL(gemm_int4b64_kernel, dim3(tiles_m * tiles_n), dim3(256), 0, s, M, K, N,
                       tiles_m, tiles_n, xcd_bands, static_cast<const _Float16 *>(A),
                       static_cast<const uint8_t *>(Wp), static_cast<const float *>(Sp), C);
    return hipGetLastError();
}

}  // namespace qg
