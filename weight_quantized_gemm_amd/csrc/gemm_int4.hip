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
// and the per-weight dequantisation work bound the kernel before the matrix
// cores do):
//  - a 512-thread workgroup owns a 64 x 128 tile of C (a taller-than-wide
//    tile would read A from L2 twice as often);
//  - wave (h, q) owns the 64 x 64 half h of the tile for the contiguous K
//    quarter q and accumulates it with v_mfma_f32_32x32x16_f16 (2 x 2
//    accumulator tiles), so every B element is fetched and dequantised once
//    per workgroup; two waves per SIMD let one wave's dequantisation issue
//    while the other's matrix instructions run;
//  - the two waves of a quarter share its A tiles in LDS: each fetches 32 of
//    the 64 rows with fully coalesced loads (8 rows x 128 bytes per
//    instruction) four blocks ahead through a register ring; four LDS tiles
//    per quarter and one barrier per block keep writers behind readers;
//  - a K-block of a 32-channel B tile is one contiguous 1 KiB record already
//    in operand lane order (see the packed layout), fetched three blocks
//    ahead through a register ring and dequantised in registers (one fp32
//    multiply-add per weight, no LDS round trip);
//  - the operands of MFMA step s + 1 are read and dequantised while the
//    matrix cores run step s;
//  - the eight partial tiles meet in LDS and the four K quarters are summed
//    in a fixed order.
// Lane (r, h) = (lane % 32, lane / 32) holds K-elements 32 h + 8 s .. +7 of
// every 64-wide block in MFMA step s, for its A row and B column alike (the K
// order inside an MFMA only has to agree between A and B).
//
// Tiles are dealt to XCDs (the hardware deals workgroups to them
// round-robin, and each has its own L2) as a grid of row bands x column
// bands: each XCD fetches only its bands of A and B. For 512 x 4096 the
// host picks 2 x 4 (A read by four XCDs, B by two), fewer bytes than one
// column band per XCD across all rows.
#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

namespace {
constexpr int BM = kInt4TileM, BN = kInt4TileN, BK = 64;
constexpr int NWAVE = 8;               // (N half, K quarter) per wave
constexpr int WN = BN / 2;             // columns per wave
constexpr int RF = BM / 32;            // 32-row accumulator tiles per wave
constexpr int CF = WN / 32;            // 32-column accumulator tiles per wave
constexpr int AS_STRIDE = BK + 8;      // halves per LDS row of an A tile (144 bytes)
constexpr int RING = 4;                // B register ring (3 blocks ahead) = A tiles per quarter
constexpr int RED_STRIDE = WN + 4;     // floats per LDS row of the reduction
constexpr size_t AS_BYTES = (size_t)BM * AS_STRIDE * 2;                 // one A tile
constexpr size_t A_LDS = (size_t)4 * RING * AS_BYTES;                   // all quarters
constexpr size_t RED_BYTES = (size_t)NWAVE * BM * RED_STRIDE * 4;       // all waves
constexpr size_t LDS_BYTES = RED_BYTES > A_LDS ? RED_BYTES : A_LDS;

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

// HP: one pair per 32-element half of each 64-block (Int4 blocks of 32).
template <bool HP>
__global__ __launch_bounds__(64 * NWAVE) void gemm_int4b64_kernel(
    int M, int K, int N, int tiles_m, int tiles_n, int xcd_rows,
    const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ Sp, void *__restrict__ C, Epilogue epi) {
    __shared__ __align__(16) unsigned char lds[LDS_BYTES];

    // ---- tile of this workgroup ----
    const int L = blockIdx.x;
    int tm, tn;
    if (xcd_rows > 0) {
        // the eight XCDs form an xcd_rows x (8 / xcd_rows) grid over the
        // tiles; XCD x = L % 8 owns row band x / gc and column band x % gc
        const int gc = 8 / xcd_rows;
        const int rb = tiles_m / xcd_rows, cb = tiles_n / gc;
        const int x = L % 8, j = L / 8;
        tm = (x / gc) * rb + j / cb;
        tn = (x % gc) * cb + j % cb;
    } else {
        tm = L / tiles_n;
        tn = L % tiles_n;
    }
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int nh = wave & 1, kq = wave >> 1;      // N half, K quarter
    const int r = lane & 31, h = lane >> 5;
    const int nblk = K / BK;                       // >= 1
    // split-K: this workgroup's blocks are [KB0, KB1) (all of K when
    // gridDim.y == 1) and its output is partial tile blockIdx.y
    const int KB0 = slice_begin(blockIdx.y, nblk, gridDim.y);
    const int KB1 = slice_begin(blockIdx.y + 1, nblk, gridDim.y);
    const int nbs = KB1 - KB0;                     // >= 1: the plan keeps gridDim.y <= nblk
    // partial tiles (split-K) and plain fp32 C take the raw store; otherwise
    // every output goes through the epilogue
    const bool raw = gridDim.y > 1 || epi.plain;
    float *const out = static_cast<float *>(C) + (size_t)blockIdx.y * M * N;
    const int kb0 = KB0 + kq * nbs / 4, kb1 = KB0 + (kq + 1) * nbs / 4;   // contiguous quarter
    const int nb = kb1 - kb0;                      // kb0 is a valid block even when nb == 0
    const int last = max(kb1 - 1, kb0);
    // every wave runs the same number of (padded) blocks: the largest
    // quarter rounded up to the ring, so all waves meet every barrier
    const int nsteps = ((nbs + 3) / 4 + RING - 1) / RING * RING;
    const int ntiles_b = (N + 31) / 32;            // packed 32-channel tiles

    auto a_tile = [&](int slot) {
        return reinterpret_cast<_Float16 *>(lds + (size_t)(kq * RING + slot) * AS_BYTES);
    };

    // A loader role: the two waves of a quarter each fetch 32 of the 64 rows,
    // 8 rows x 128 bytes per instruction, lane -> (row, 16 B piece); byte
    // offsets from the tile's first row (rows past M are clamped: loaded,
    // never stored).
    const int arow = lane >> 3, apc = lane & 7;
    const char *A_tile = reinterpret_cast<const char *>(A + (size_t)m0 * K);
    unsigned a_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a_off[i] = (unsigned)(min(32 * nh + 8 * i + arow, M - 1 - m0) * K + 8 * apc) * 2u;
    // B: packed tile of each accumulator column tile (tiles past N: loaded, never stored)
    size_t b_rec0[CF];
#pragma unroll
    for (int cf = 0; cf < CF; ++cf)
        b_rec0[cf] = (size_t)min(n0 / 32 + CF * nh + cf, ntiles_b - 1) * nblk;

    auto load_a = [&](u4_t (&dst)[4], int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dst[i] = *reinterpret_cast<const u4_t *>(A_tile + a_off[i] + (unsigned)kt * (BK * 2));
    };
    // every word ANDed with a uniform mask (all ones, or zero for a block
    // past the quarter's end): no branch, so no merge point for the
    // compiler's count of outstanding loads
    auto store_a = [&](_Float16 *As, const u4_t (&src)[4], unsigned mask) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u4_t *>(As + (32 * nh + 8 * i + arow) * AS_STRIDE + 8 * apc) = src[i] & mask;
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
            pairs[cf] = *reinterpret_cast<const f2_t *>(HP ? Sp + rec * 128 + h * 64 + r * 2
                                                           : Sp + rec * 64 + r * 2);
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

    u4_t an[RING][4];          // A register ring: stage j holds a block = j mod RING
    u4_t bc[RING][CF];
    f2_t bp[RING][CF];
    DqParams prm[CF];
    h8_t acur[RF], anxt[RF], bcur[CF], bnxt[CF];

    // Every global load below is unconditional, from a block index clamped
    // into the quarter (kb0 is valid even for an empty quarter): with no
    // skipped loads the compiler's in-order count of outstanding loads stays
    // exact, so a wait only ever covers the data it needs. What a clamped
    // load brings is never used: a block past the quarter's end gets an
    // all-zero A tile instead, and adds exactly zero.
    //
    // prologue: block 0's A in tile 0 and blocks 1 .. RING in flight in the
    // A ring, B of blocks 0 .. RING - 1 in flight, step (0, 0) operands ready
    load_a(an[0], kb0);
#pragma unroll
    for (int d = 0; d < RING; ++d) load_b(bc[d], bp[d], min(kb0 + d, last));
    store_a(a_tile(0), an[0], nb > 0 ? ~0u : 0u);
#pragma unroll
    for (int d = 1; d <= RING; ++d) load_a(an[d % RING], min(kb0 + d, last));
    __syncthreads();
#pragma unroll
    for (int cf = 0; cf < CF; ++cf) prm[cf] = dq_params(bp[0][cf]);
    read_a(a_tile(0), 0, acur);
#pragma unroll
    for (int cf = 0; cf < CF; ++cf) bcur[cf] = dequant8(bc[0][cf][0], prm[cf], m_lo, m_hi, magic);

    // Block i uses A tile i % RING and B slot i % RING. A padded block
    // (i >= nb) has an all-zero A tile and adds exactly zero.
    for (int base = 0; base < nsteps; base += RING) {
#pragma unroll
        for (int u = 0; u < RING; ++u) {
            const int i = base + u;
            // block i + 1's A (loaded RING blocks ago) into its tile, which
            // was last read in block i - 3, before the previous barrier; its
            // ring stage then takes block i + 1 + RING
            store_a(a_tile((u + 1) % RING), an[(u + 1) % RING], i + 1 < nb ? ~0u : 0u);
            load_a(an[(u + 1) % RING], min(kb0 + i + 1 + RING, last));
            __syncthreads();
            // four MFMA steps; while the matrix cores work on step s the
            // operands of the next step (this block's s + 1, or the next
            // block's step 0) are read and dequantised
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s < 3) {
                    read_a(a_tile(u), s + 1, anxt);
#pragma unroll
                    for (int cf = 0; cf < CF; ++cf)
                        bnxt[cf] = dequant8(bc[u][cf][s + 1], prm[cf], m_lo, m_hi, magic);
                } else {
                    const int un = (u + 1) % RING;
                    read_a(a_tile(un), 0, anxt);
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
            // slot u is free now (its last use was the dequantisation in
            // step 2): refill it with block i + RING
            load_b(bc[u], bp[u], min(kb0 + i + RING, last));
        }
    }

    // ---- the eight partial tiles to LDS (reusing the A tiles' space) ----
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

    // ---- sum the four K quarters in a fixed order and store:
    //      thread -> row tid / 8, 16 columns ----
    const int row = tid >> 3;
    const int c0 = (tid & 7) * 16;                 // column in the 128-wide tile
    const int gm = m0 + row;
    if (gm >= M) return;
    const int half = c0 / WN, ch = c0 % WN;
    const float *red0 = reinterpret_cast<const float *>(lds);
    float *dst = out + (size_t)gm * N + n0 + c0;
    const bool vec_store = (N & 3) == 0 && n0 + c0 + 16 <= N;
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
        const size_t o = (size_t)row * RED_STRIDE + ch + j;
        const size_t W = (size_t)BM * RED_STRIDE;
        f4_t sum = *reinterpret_cast<const f4_t *>(red0 + (size_t)half * W + o);
#pragma unroll
        for (int q = 1; q < 4; ++q)
            sum += *reinterpret_cast<const f4_t *>(red0 + (size_t)(2 * q + half) * W + o);
        if (!raw && vec_store) {
            epi_put4(epi, C, gm, n0 + c0 + j, N, sum);
        } else if (!raw) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n0 + c0 + j + e < N) epi_put(epi, C, gm, n0 + c0 + j + e, N, sum[e]);
        } else if (vec_store) {
            *reinterpret_cast<f4_t *>(dst + j) = sum;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n0 + c0 + j + e < N) dst[j + e] = sum[e];
        }
    }
}

hipError_t launch_gemm_int4b64(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, void *C, const Epilogue &epi, int half_pairs,
                               int nsplit, float *part, hipStream_t s) {
    const int tiles_m = div_up(M, BM), tiles_n = div_up(N, BN);
    // XCD grid: row bands x column bands = 8, each XCD's L2 then fetches
    // A of its row band and B of its column band; pick the grid the tile
    // counts divide that fetches the fewest bytes (0: plain order)
    int xcd_rows = 0;
    double best = 0;
    const double a_bytes = (double)M * K * 2, b_bytes = (double)N * K * 0.625;
    for (int gr = 1; gr <= 8; gr *= 2) {
        const int gc = 8 / gr;
        if (tiles_m % gr || tiles_n % gc) continue;
        const double fetched = gc * a_bytes + gr * b_bytes;
        if (xcd_rows == 0 || fetched < best) { xcd_rows = gr; best = fetched; }
    }
    void *out = nsplit > 1 ? static_cast<void *>(part) : C;
    auto kernel = half_pairs ? gemm_int4b64_kernel<true> : gemm_int4b64_kernel<false>;
    hipLaunchKernelGGL(kernel, dim3(tiles_m * tiles_n, nsplit), dim3(64 * NWAVE), 0, s,
                       M, K, N, tiles_m, tiles_n, xcd_rows, static_cast<const _Float16 *>(A),
                       static_cast<const uint8_t *>(Wp), static_cast<const float *>(Sp), out, epi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nsplit <= 1) return e;
    return launch_splitk_reduce_f32(part, nsplit, M, N, C, epi, s);
}

}  // namespace qg
