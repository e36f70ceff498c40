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
// output gives each of 256 CUs only 8192 outputs, so the bytes entering a CU
// and the per-weight dequantisation bound the kernel before the matrix cores
// do; each CU's L2 port delivers 64 bytes per clock):
//  - a 256-thread workgroup owns a BM x BN tile of C, one workgroup per CU:
//    128 x 64 once M reaches 128 (each dequantised weight then serves 128
//    rows, which halves the dequantising instructions per matrix
//    instruction: the vector ALUs, not the matrix cores, bound this kernel),
//    64 x 128 below (half the rows of a 128-row tile would be padding), and
//    128 x 128 where those tiles need fewer rounds of the CUs (M >= 1024 at
//    N = 4096): each A byte brought into the CU then serves twice the
//    columns, which the texture unit carrying A into LDS (busy two thirds of
//    the 128 x 64 kernel's life) had limited; its 256 accumulators per lane
//    take all the AGPRs;
//  - each of its four waves (one per SIMD) accumulates the whole tile over
//    one contiguous quarter of K with v_mfma_f32_32x32x16_f16 (BM/32 x BN/32
//    accumulator tiles), so every B element is fetched and dequantised once
//    per workgroup and no operand is shared between waves: the main loop has
//    no barrier, and each SIMD's matrix pipe is fed by its own wave, whose
//    dequantising instructions issue while its matrix instructions run;
//  - a wave's A block (BM rows x 64 K-elements) goes from memory straight
//    into one of the wave's own LDS tiles by DMA (buffer loads with the LDS
//    as destination: no registers and no LDS write instructions, which
//    measured about 6 % of the kernel), fully coalesced (8 rows x 128 bytes
//    per instruction), one (BM = 128, two tiles) or three (BM = 64, four
//    tiles) blocks ahead; rows are stored XOR-swizzled so that the MFMA
//    reads of 32 rows at one K offset hit distinct banks. The compiler does
//    not order the DMA's LDS writes against later reads, so the wave waits
//    for them explicitly before it reads a tile;
//  - a K-block of a 32-channel B tile is one contiguous 1 KiB record already
//    in operand lane order (see the packed layout), fetched four blocks ahead
//    through a register ring and dequantised in registers (one fp32
//    multiply-add per weight, no LDS round trip);
//  - the operands of MFMA step s + 1 are read and dequantised while the
//    matrix cores run step s;
//  - the instructions of one MFMA step stay in one scheduling region, and
//    each dequantised operand is pinned where it is produced, so no matrix
//    instruction waits on a vector instruction moved next to it;
//  - the four partial tiles meet in LDS and are summed in a fixed order (a
//    128 x 128 tile in two chunks of 64 columns).
// Lane (r, h) = (lane % 32, lane / 32) holds K-elements 32 h + 8 s .. +7 of
// every 64-wide block in MFMA step s, for its A row and B column alike (the K
// order inside an MFMA only has to agree between A and B).
//
// The hardware deals workgroups to the XCDs round-robin, and each XCD has
// its own L2. With a multiple of 8 column tiles (512 x 4096: 64) plain
// order gives each XCD an interleaved eighth of the columns for every row
// tile, which measured faster (25.8 against 26.3 us at 512 x 4096 x 4096,
// 96.8 against 100.3 us at 2048 x 4096 x 4096) than the row-band x
// column-band grids that fewer fetched bytes would pick (2 x 4 there: A read
// by four XCDs, B by two). Other column counts (N = 11008: 172 tiles) take
// that grid, where plain order measured slower (140.6 against 138.0 us at
// 1024 x 4096 x 11008).
#include <type_traits>

#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

namespace {
constexpr int BK = 64;
constexpr int NWAVE = 4;               // one K quarter per wave
constexpr int P_RING = 2;              // pair ring (loads two blocks ahead)
constexpr int UNROLL = 4;              // lcm of the rings: every slot a fixed register

// Shape-dependent constants of one tile.
template <int BM_, int BN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int RF = BM / 32;                  // 32-row accumulator tiles per wave
    static constexpr int CF = BN / 32;                  // 32-column accumulator tiles per wave
    // LDS A tiles per wave (a ring: the DMA runs A_TILES - 1 blocks ahead)
    static constexpr int A_TILES = BM == 64 ? 4 : 2;
    // B code ring: loads four blocks ahead
    static constexpr int B_RING = 4;
    static constexpr int A_PIECES = BM * BK / 8 / 64;   // 16-byte A pieces per lane and block
    static constexpr size_t AS_BYTES = (size_t)BM * BK * 2;                 // one A tile
    static constexpr size_t WAVE_LDS = (size_t)A_TILES * AS_BYTES;          // one wave's tiles
    static constexpr size_t LDS_BYTES = (size_t)NWAVE * WAVE_LDS;
    // loads issued after the DMA of the block a wave reads next, by the time
    // it reads it (see the main loop)
    static constexpr int A_WAIT = CF + (A_TILES - 2) * (2 * CF + A_PIECES);
    // loads issued after block 0's codes in the prologue (the pairs of block
    // 1 and the codes of blocks 1 .. B_RING - 1)
    static constexpr int PRO_WAIT = B_RING * CF;
    static_assert(UNROLL % A_TILES == 0 && UNROLL % B_RING == 0, "ring sizes");
    static_assert(A_WAIT <= 63 && PRO_WAIT <= 63, "vmcnt range");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 workgroup");
    // a wave's partial tile (BM x BN fp32) goes through its A tiles' space in
    // NCH chunks of CWID columns
    static constexpr int CWID = (int)(WAVE_LDS / ((size_t)BM * 4));
    static constexpr int NCH = BN / CWID;
    static_assert(NCH * CWID == BN && CWID % 32 == 0 && CWID >= 64, "whole column chunks");
};

// Per (channel tile, block) dequantisation constants. Even codes decode as
// x = 1024 + q and odd codes as x = 1024 + 16 q (the nibble is left in
// place), so w = offset + scale * q is x * s_lo + b_lo or x * s_hi + b_hi.
struct DqParams {
    float s_lo, b_lo, s_hi, b_hi;
};

// keep = 0 (a padded block past the quarter's end) gives all-zero
// constants: every weight of the block dequantises to +0 and adds nothing.
__device__ __forceinline__ DqParams dq_params(f2_t pair, bool keep) {
    const float off = keep ? pair.x : 0.f, sc = keep ? pair.y : 0.f;
    return {sc, fmaf(-1024.0f, sc, off), sc * 0.0625f, fmaf(-64.0f, sc, off)};
}

template <int AUX = 0>
__device__ __forceinline__ u4_t buf_load16(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX));
}
__device__ __forceinline__ f2_t buf_load8(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_bit_cast(f2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}
constexpr int kNonTemporal = 2;   // cache policy of a streamed load (read once per workgroup)

}

// 8 Int4 codes (one word, k ascending, low nibble first) -> 8 fp16 weights
// in k order, each one fp32 fused multiply-add rounded once to fp16. m_lo,
// m_hi and magic are the constants 0x000F000F, 0x00F000F0 and 0x64006400 held
// in registers, so each pair of codes costs one v_and_or_b32. The decode is
// the published magic-exponent conversion of integer codes to fp16 (Kim et
// al., "Who Says Elephants Can't Run", 2022): OR-ing a code into the
// mantissa of 1024.0 gives 1024 + q exactly.
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

// Marks a value as produced here: the optimiser may not sink its
// computation below this point (towards its use in a later MFMA step, where
// it would stall the matrix instruction that reads it).
__device__ __forceinline__ void pin(h8_t &v) { asm volatile("" : "+v"(v)); }

// G: pair entries per 64-block (1; 2: one per 32-element half, blocks of
// 32; 4: one per 16-element quarter, blocks that are odd multiples of 16).
// A lane decodes one 32-element half of each block: with G = 4 its steps 0-1
// and 2-3 take the two quarters' pairs, one 16-byte load for both.
template <class T, int G>
__global__ __launch_bounds__(64 * NWAVE) void gemm_int4b64_kernel(
    int M, int K, int N, int tiles_m, int tiles_n, int xcd_rows,
    const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ Sp, void *__restrict__ C, Epilogue epi) {
    constexpr int BM = T::BM, BN = T::BN, RF = T::RF, CF = T::CF;
    constexpr int A_TILES = T::A_TILES, A_PIECES = T::A_PIECES;
    constexpr int B_RING = T::B_RING;
    constexpr size_t AS_BYTES = T::AS_BYTES;
    __shared__ __align__(16) unsigned char lds[T::LDS_BYTES];

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
    const int kq = uniform(tid >> 6);              // this wave's K quarter
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
    // every wave runs its quarter's blocks rounded up to the unroll, at least
    // one unroll (so no path skips the main loop); blocks past the quarter's
    // end re-load its last block and add exactly zero
    const int nsteps = max((nb + UNROLL - 1) / UNROLL, 1) * UNROLL;
    const int ntiles_b = (N + 31) / 32;            // packed 32-channel tiles

    unsigned char *const a_lds = lds + (size_t)kq * T::WAVE_LDS;
    auto a_tile = [&](int slot) { return a_lds + (size_t)slot * AS_BYTES; };

    // A by LDS DMA: a tile is BM rows of 128 bytes (one block), 16-byte slot
    // j of row rho holding the row's piece j ^ (rho % 8), so that the MFMA
    // reads (32 rows at one piece) fall in distinct banks. DMA instruction i
    // fills rows 8 i .. 8 i + 7: lane l's 16 bytes land in row 8 i + l / 8,
    // slot l % 8, so it fetches piece (l % 8) ^ (l / 8) of that row (rows
    // past M are clamped: loaded, never stored). Per block the buffer's base
    // advances by 128 bytes.
    const int arow = lane >> 3, apc = lane & 7;
    const int arows = min(BM, M - m0);
    unsigned a_off[A_PIECES];
#pragma unroll
    for (int i = 0; i < A_PIECES; ++i)
        a_off[i] = (unsigned)(min(8 * i + arow, arows - 1) * K + 8 * (apc ^ arow)) * 2u;
    // B: records of each accumulator column tile (tiles past N: loaded, never
    // stored), one 1 KiB record and one pair record per block
    constexpr unsigned PREC = 256u * G;           // bytes per pair record
    constexpr int GQ = G == 4 ? 2 : 1;            // pair constants per lane and block
    using PairT = typename std::conditional<G == 4, f4_t, f2_t>::type;
    // (the pair records of the CF tiles are consecutive: one resource over
    // them, each tile at a scalar offset, saves the scalar registers of
    // CF - 1 resources)
    __amdgpu_buffer_rsrc_t b_rs[CF];
    unsigned p_tile[CF];
    const int t0 = min(n0 / 32, ntiles_b - 1);
#pragma unroll
    for (int cf = 0; cf < CF; ++cf) {
        const size_t rec0 = (size_t)min(n0 / 32 + cf, ntiles_b - 1) * nblk;
        b_rs[cf] = byte_rsrc(Wp + rec0 * 1024, (unsigned)nblk * 1024u);
        p_tile[cf] = (unsigned)(min(n0 / 32 + cf, ntiles_b - 1) - t0) * (unsigned)nblk * PREC;
    }
    const __amdgpu_buffer_rsrc_t p_rs = byte_rsrc(reinterpret_cast<const char *>(Sp) + (size_t)t0 * nblk * PREC,
                                                  p_tile[CF - 1] + (unsigned)nblk * PREC);
    const unsigned b_off = (unsigned)lane * 16u;
    const unsigned p_off = G == 4 ? (unsigned)(4 * r + 2 * h) * 8u
                         : G == 2 ? (unsigned)(32 * h + r) * 8u : (unsigned)r * 8u;

    auto dma_a = [&](unsigned char *As, int kt) {
        const __amdgpu_buffer_rsrc_t rs = byte_rsrc(A + (size_t)m0 * K + (size_t)kt * BK,
                                                    (unsigned)arows * K * 2u - (unsigned)kt * (BK * 2));
#pragma unroll
        for (int i = 0; i < A_PIECES; ++i) lds_dma16(rs, As + i * 1024, a_off[i]);
    };
    // MFMA step s: lane (r, h) takes piece 4 h + s of rows 32 rf + r
    auto read_a = [&](const unsigned char *As, int s, h8_t (&af)[RF]) {
#pragma unroll
        for (int rf = 0; rf < RF; ++rf)
            af[rf] = *reinterpret_cast<const h8_t *>(As + (32 * rf + r) * 128 + 16 * ((4 * h + s) ^ (r & 7)));
    };
    auto load_b = [&](u4_t (&codes)[CF], int kt) {
#pragma unroll
        for (int cf = 0; cf < CF; ++cf) codes[cf] = buf_load16<kNonTemporal>(b_rs[cf], b_off, (unsigned)kt * 1024u);
    };
    auto load_p = [&](PairT (&pairs)[CF], int kt) {
#pragma unroll
        for (int cf = 0; cf < CF; ++cf) {
            if constexpr (G == 4)
                pairs[cf] = __builtin_bit_cast(f4_t, buf_load16(p_rs, p_off, p_tile[cf] + (unsigned)kt * PREC));
            else
                pairs[cf] = buf_load8(p_rs, p_off, p_tile[cf] + (unsigned)kt * PREC);
        }
    };
    // a block's dequantisation constants: set 0 for MFMA steps 0-1, set
    // GQ - 1 for steps 2-3
    auto make_prm = [&](const PairT &pp, bool keep, DqParams (&dst)[GQ]) {
        if constexpr (G == 4) {
            dst[0] = dq_params(f2_t{pp.x, pp.y}, keep);
            dst[GQ - 1] = dq_params(f2_t{pp.z, pp.w}, keep);
        } else {
            dst[0] = dq_params(pp, keep);
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

    u4_t bc[B_RING][CF];        // B code ring: slot j % B_RING holds block j
    PairT bp[P_RING][CF];       // pair ring: slot j % 2 holds block j
    DqParams prm[CF][GQ];
    h8_t acur[RF], anxt[RF], bcur[CF], bnxt[CF];

    // Every global load below is unconditional, from a block index clamped
    // into the quarter (kb0 is valid even for an empty quarter): with no
    // skipped loads the compiler's in-order count of outstanding loads stays
    // exact, so a wait only ever covers the data it needs. What a clamped
    // load brings is never used: a block past the quarter's end gets all-zero
    // dequantisation constants instead (every weight +0), and adds exactly
    // zero.
    //
    // prologue: the A of blocks 0 .. A_TILES - 2 (tiles 0 ..), the pairs and
    // codes of block 0, then the pairs of block 1 and the codes of blocks
    // 1 .. B_RING - 1. Only what precedes the last PRO_WAIT loads is waited
    // for (all the DMAs and block 0's B), so block 0 starts while the rest
    // of the rings is still on its way; block 0's step-0 operands ready
#pragma unroll
    for (int d = 0; d < A_TILES - 1; ++d) dma_a(a_tile(d), min(kb0 + d, last));
    load_p(bp[0], kb0);
    load_b(bc[0], kb0);
    load_p(bp[1], min(kb0 + 1, last));
#pragma unroll
    for (int d = 1; d < B_RING; ++d) load_b(bc[d], min(kb0 + d, last));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vm_wait(T::PRO_WAIT));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int cf = 0; cf < CF; ++cf) make_prm(bp[0][cf], nb > 0, prm[cf]);
    read_a(a_tile(0), 0, acur);
#pragma unroll
    for (int cf = 0; cf < CF; ++cf) bcur[cf] = dequant8(bc[0][cf][0], prm[cf][0], m_lo, m_hi, magic);

    // Block i reads A tile i % A_TILES and B slot i % B_RING. At its start
    // the tile of block i - 1, whose reads were all consumed by block i - 1's
    // matrix instructions, takes block i + A_TILES - 1 by DMA. Its step 3
    // reads block i + 1's first operands: that tile's DMA was issued at the
    // start of block i + 2 - A_TILES (or in the prologue, which waited for
    // all its DMAs), and since then each block issued its pair loads, its DMA and its
    // code loads (CF + A_PIECES + CF), this block the pairs and the DMA
    // before the codes: A_WAIT loads may still be outstanding, which the
    // explicit wait below allows (the compiler does not track the DMA's
    // writes to LDS).
    for (int base = 0; base < nsteps; base += UNROLL) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int i = base + u;
            // pair slot i % 2 was last read for block i's constants (end of
            // block i - 1): it takes block i + 2
            load_p(bp[u % P_RING], min(kb0 + i + P_RING, last));
            dma_a(a_tile((u + A_TILES - 1) % A_TILES), min(kb0 + i + A_TILES - 1, last));
            // keep the loads here, ahead of the arithmetic: moved down next to
            // their use they would wait for memory instead of hiding it
            __builtin_amdgcn_sched_barrier(0);
            // four MFMA steps; while the matrix cores work on step s the
            // operands of the next step (this block's s + 1, or the next
            // block's step 0) are read and dequantised
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s < 3) {
                    read_a(a_tile(u % A_TILES), s + 1, anxt);
#pragma unroll
                    for (int cf = 0; cf < CF; ++cf) {
                        bnxt[cf] = dequant8(bc[u % B_RING][cf][s + 1], prm[cf][(s + 1) * GQ / 4],
                                            m_lo, m_hi, magic);
                        pin(bnxt[cf]);
                    }
                } else {
                    const int un = (u + 1) % B_RING;
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_waitcnt(vm_wait(T::A_WAIT));
                    __builtin_amdgcn_sched_barrier(0);
                    read_a(a_tile((u + 1) % A_TILES), 0, anxt);
#pragma unroll
                    for (int cf = 0; cf < CF; ++cf) {
                        make_prm(bp[(u + 1) % P_RING][cf], i + 1 < nb, prm[cf]);
                        bnxt[cf] = dequant8(bc[un][cf][0], prm[cf][0], m_lo, m_hi, magic);
                        pin(bnxt[cf]);
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
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                }
                // one MFMA step per scheduling region: the next step's MFMAs,
                // each on an accumulator of this step, stay RF * CF apart
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int rf = 0; rf < RF; ++rf) acur[rf] = anxt[rf];
#pragma unroll
                for (int cf = 0; cf < CF; ++cf) bcur[cf] = bnxt[cf];
                // slot u % B_RING is free once its last codes were
                // dequantised (step 2): refill it with block i + B_RING
                if (s == 2) {
                    __builtin_amdgcn_sched_barrier(0);
                    load_b(bc[u % B_RING], min(kb0 + i + B_RING, last));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }

    // ---- the four partial tiles meet in LDS. A wave whose own DMAs have
    //      landed (the last ones, of clamped blocks, are never read) writes
    //      its partial tile into its own A tiles, which no other wave uses,
    //      so the waves that finish first do not wait for the last one; after
    //      one barrier every thread sums four rows of one column over the K
    //      quarters in a fixed order and stores them. A wave's partial tile
    //      is column-major in groups of four rows, group R of column col at
    //      slot R ^ (col % 16): the 16 lanes of a 16-byte LDS access, on 16
    //      consecutive columns, then cover all 64 banks, when written from
    //      the accumulator layout and when read back. One store instruction
    //      writes 64 consecutive columns of a row. ----
    constexpr int RG = BM / 4;                     // four-row groups per column
    constexpr int CWID = T::CWID, NCH = T::NCH;
    constexpr int GPP = 64 * NWAVE / CWID;         // row groups per pass
    static_assert(RG % GPP == 0 && RG >= 16, "whole passes, swizzle within the column");
    __builtin_amdgcn_s_waitcnt(vm_wait(0));
    const int col = tid % CWID, g0 = tid / CWID;   // g0 is wave-uniform (CWID >= 64)
    const float *red0 = reinterpret_cast<const float *>(lds);
    constexpr size_t W = T::WAVE_LDS / 4;          // floats per wave's partial tile
    auto sum4 = [&](int R) {
        const size_t o = (size_t)col * BM + 4 * (R ^ (col & 15));
        f4_t v = *reinterpret_cast<const f4_t *>(red0 + o);
#pragma unroll
        for (int q = 1; q < NWAVE; ++q) v += *reinterpret_cast<const f4_t *>(red0 + (size_t)q * W + o);
        return v;
    };
    // A tile wider than the wave's LDS space (BN > CWID) goes through it in
    // column chunks, a barrier before each chunk's writes and each chunk's
    // reads.
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        if (ch > 0) __syncthreads();
        {
            float *mine = reinterpret_cast<float *>(a_lds);
#pragma unroll
            for (int rf = 0; rf < RF; ++rf)
#pragma unroll
                for (int cc = 0; cc < CWID / 32; ++cc)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        // rows 32 rf + 8 g + 4 h + (0 .. 3) of chunk column 32 cc + r
                        const int cf = ch * (CWID / 32) + cc;
                        const int R = 8 * rf + 2 * g + h, lc = 32 * cc + r;
                        *reinterpret_cast<f4_t *>(mine + (size_t)lc * BM + 4 * (R ^ (lc & 15))) =
                            f4_t{acc[rf][cf][4 * g], acc[rf][cf][4 * g + 1], acc[rf][cf][4 * g + 2],
                                 acc[rf][cf][4 * g + 3]};
                    }
        }
        __syncthreads();
        const int gc = n0 + ch * CWID + col;
        // (the two store forms in separate loops, the epilogue one not
        // unrolled: one copy of its code per row group would not stay in the
        // instruction cache). The raw stores are non-temporal: C is not read
        // again here, and streamed past the caches its write-back no longer
        // competes with the next kernel's loads.
        if (raw) {
#pragma unroll
            for (int it = 0; it < RG / GPP; ++it) {
                const int R = it * GPP + g0, gm = m0 + 4 * R;
                if (gm >= M) break;
                const f4_t v = sum4(R);
                if (gc < N) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (gm + e < M) __builtin_nontemporal_store(v[e], out + (size_t)(gm + e) * N + gc);
                }
            }
        } else {
#pragma unroll 1
            for (int it = 0; it < RG / GPP; ++it) {
                const int R = it * GPP + g0, gm = m0 + 4 * R;
                if (gm >= M) break;
                const f4_t v = sum4(R);
                if (gc < N) {
                    for (int e = 0; e < 4 && gm + e < M; ++e) epi_put(epi, C, gm + e, gc, N, v[e]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Skinny prefill (GEMV threshold < M <= 64): few rows, so the weights are the
// bytes that matter (the MNN GemmSpeed page, section "Sample data": small M
// is bound by the weight stream) and a tile of the wide GEMM would be mostly
// padding rows and few workgroups. A 512-thread workgroup owns one 32-channel
// tile of every row (RF 32-row fragments, all of M) over one K slice; its
// eight waves take the slice's 64-blocks round-robin. As in the decode GEMV,
// every weight record and pair of a wave's blocks is requested at once (up to
// 8 NB blocks per workgroup; a longer slice repeats this), so the weight
// stream costs one round trip; A, which every tile reads and the L2 holds,
// goes into LDS by DMA in passes of SK_PB blocks, double-buffered, rows
// XOR-swizzled as in the wide kernel. Per block a wave dequantises its 1 KiB
// record as the wide kernel does and runs four MFMA steps per row fragment;
// the eight waves' partial tiles meet in LDS in a fixed order. Every load is
// unconditional from clamped indices; blocks past the slice get all-zero
// dequantisation constants and add exactly zero.
// ---------------------------------------------------------------------------
constexpr int SK_WAVES = 8;
constexpr int SK_BUF = 64 * 1024;                   // A bytes per pass buffer (two buffers)

template <int RF, int NB>
struct SkinnyCfg {
    static constexpr int MR = 32 * RF;                               // rows staged (M padded)
    static constexpr int PB = SK_BUF / (MR * 128);                   // blocks per pass
    static constexpr int NDMA = PB * MR / 8 / SK_WAVES;              // DMA instructions per wave and pass
    static constexpr int NBW = PB / SK_WAVES;                        // blocks per wave and pass
    static constexpr int SPB = SK_WAVES * NB;                        // blocks per round of weight loads
    static constexpr int NPASS = NB / NBW;                           // passes per round
    static constexpr size_t RED_BYTES = (size_t)SK_WAVES * MR * 32 * 4;  // the waves' partial tiles
    static_assert(NDMA * SK_WAVES * 8 == PB * MR && NBW * SK_WAVES == PB, "whole passes");
    static_assert(NB % NBW == 0, "whole passes per round");
    static_assert(RED_BYTES <= SK_BUF, "reduction fits one A buffer");
    // loads issued after pass 0's DMA when the wave first waits for it (the
    // round's weight records and pairs, then pass 1's DMA), and after pass
    // p's DMA when it waits for that (pass p + 1's DMA)
    static constexpr int WAIT0 = 2 * NB + NDMA;
    static constexpr int WAIT = NDMA;
    static_assert(WAIT0 <= 63, "vmcnt range");
};

// A workgroup barrier without __syncthreads' release fence, which would also
// wait for the LDS DMA just issued for the next pass: the waves' own waits
// cover the DMA they read, and every LDS read before the barrier has been
// consumed; the acquire fence keeps later LDS reads below the barrier.
__device__ __forceinline__ void sk_barrier() {
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int RF, int G, int NB>
__global__ __launch_bounds__(64 * SK_WAVES) void gemm_int4b64_skinny_kernel(
    int M, int K, int N, const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ Sp, void *__restrict__ C, Epilogue epi) {
    using T = SkinnyCfg<RF, NB>;
    constexpr int MR = T::MR, PB = T::PB, NDMA = T::NDMA, NBW = T::NBW, SPB = T::SPB;
    // one array per A buffer: the compiler orders LDS reads after any DMA
    // into the same array (it does not see the explicit waits), and only
    // separate arrays let it tell one buffer's DMA from reads of the other
    __shared__ __align__(16) unsigned char lds0[SK_BUF], lds1[SK_BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int r = lane & 31, h = lane >> 5;
    const int t = blockIdx.x;                                  // 32-channel tile
    const int nblk = K / BK;
    const int KB0 = slice_begin(blockIdx.y, nblk, gridDim.y);
    const int KB1 = slice_begin(blockIdx.y + 1, nblk, gridDim.y);
    const int last = KB1 - 1;
    const bool raw = gridDim.y > 1 || epi.plain;
    float *const out = static_cast<float *>(C) + (size_t)blockIdx.y * M * N;

    constexpr unsigned PREC = 256u * G;
    constexpr int GQ = G == 4 ? 2 : 1;
    using PairT = typename std::conditional<G == 4, f4_t, f2_t>::type;
    const int ntiles_b = (N + 31) / 32;
    const size_t rec0 = (size_t)min(t, ntiles_b - 1) * nblk;
    const __amdgpu_buffer_rsrc_t b_rs = byte_rsrc(Wp + rec0 * 1024, (unsigned)nblk * 1024u);
    const __amdgpu_buffer_rsrc_t p_rs = byte_rsrc(reinterpret_cast<const char *>(Sp) + rec0 * PREC,
                                                  (unsigned)nblk * PREC);
    const unsigned b_off = (unsigned)lane * 16u;
    const unsigned p_off = G == 4 ? (unsigned)(4 * r + 2 * h) * 8u
                         : G == 2 ? (unsigned)(32 * h + r) * 8u : (unsigned)r * 8u;

    // DMA instruction g = wave + 8 q of a pass fills rows 8 (g % (MR / 8)) ..
    // + 7 of its block g / (MR / 8): lane l's 16 bytes land in row
    // rho = 8 (g % (MR / 8)) + l / 8, slot l % 8, and are piece (l % 8) ^ (l / 8)
    // of that row of A (rows past M clamped: loaded, never stored)
    unsigned a_off[NDMA];
#pragma unroll
    for (int q = 0; q < NDMA; ++q) {
        const int g = wave + SK_WAVES * q;
        const int row = 8 * (g % (MR / 8)) + (lane >> 3);
        a_off[q] = (unsigned)(min(row, M - 1) * K + 8 * ((lane & 7) ^ (lane >> 3))) * 2u;
    }
    auto dma = [&](unsigned char *buf, int b0) {    // the pass starting at block b0
#pragma unroll
        for (int q = 0; q < NDMA; ++q) {
            const int g = wave + SK_WAVES * q;
            const int b = min(b0 + g / (MR / 8), last);
            const __amdgpu_buffer_rsrc_t rs =
                byte_rsrc(A + (size_t)b * BK, (unsigned)M * K * 2u - (unsigned)b * (BK * 2));
            lds_dma16(rs, buf + (size_t)g * 1024, a_off[q]);
        }
    };

    unsigned m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, magic = 0x64006400u;
    asm volatile("" : "+s"(m_lo), "+s"(m_hi));
    asm volatile("" : "+v"(magic));

    f16_t acc[RF];
#pragma unroll
    for (int i = 0; i < RF; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

    u4_t bq[NB];
    PairT bp[NB];
    // pass p of a round (blocks s0 + p PB ..): the wave's blocks are k =
    // p NBW + kk, block s0 + wave + 8 k of the round
    auto compute = [&](const unsigned char *buf, int p, int spb) {
#pragma unroll
        for (int kk = 0; kk < NBW; ++kk) {
            const int k = p * NBW + kk;
            const int j = wave + SK_WAVES * k;                 // block within the round
            DqParams prm[GQ];
            if constexpr (G == 4) {
                prm[0] = dq_params(f2_t{bp[k].x, bp[k].y}, j < spb);
                prm[GQ - 1] = dq_params(f2_t{bp[k].z, bp[k].w}, j < spb);
            } else {
                prm[0] = dq_params(bp[k], j < spb);
            }
            const unsigned char *tile = buf + (size_t)(wave + SK_WAVES * kk) * MR * 128;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const h8_t bop = dequant8(bq[k][st], prm[st * GQ / 4], m_lo, m_hi, magic);
#pragma unroll
                for (int rf = 0; rf < RF; ++rf) {
                    const h8_t aop = *reinterpret_cast<const h8_t *>(
                        tile + (32 * rf + r) * 128 + 16 * ((4 * h + st) ^ (r & 7)));
                    acc[rf] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop, acc[rf], 0, 0, 0);
                }
            }
        }
    };

    // Rounds of SPB blocks (usually one). A round issues pass 0's DMA, every
    // weight record and pair of the wave's blocks, and pass 1's DMA; before
    // pass p is read the wave waits for its DMA (loads complete in order:
    // WAIT0 newer loads may stay in flight for pass 0, WAIT for the others,
    // each pass having issued the next one's DMA first; if the compiler moved
    // weight loads below a wait, the count still covers the DMA issued before
    // them), and the barrier makes every wave's share visible; the second
    // barrier keeps a buffer from being refilled while a wave still reads it.
    for (int s0 = KB0; s0 < KB1; s0 += SPB) {                 // workgroup-uniform
        const int spb = min(SPB, KB1 - s0);
        dma(lds0, s0);
#pragma unroll
        for (int k = 0; k < NB; ++k)
            bq[k] = buf_load16<kNonTemporal>(b_rs, b_off, (unsigned)min(s0 + wave + SK_WAVES * k, last) * 1024u);
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const unsigned b = (unsigned)min(s0 + wave + SK_WAVES * k, last);
            if constexpr (G == 4)
                bp[k] = __builtin_bit_cast(f4_t, buf_load16(p_rs, p_off, b * PREC));
            else
                bp[k] = buf_load8(p_rs, p_off, b * PREC);
        }
        dma(lds1, s0 + PB);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vm_wait(T::WAIT0));
        sk_barrier();
        compute(lds0, 0, spb);
        sk_barrier();
#pragma unroll
        for (int p = 1; p < T::NPASS; ++p) {
            if (p * PB >= spb) break;                          // workgroup-uniform
            dma((p & 1) ? lds0 : lds1, s0 + (p + 1) * PB);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vm_wait(T::WAIT));
            sk_barrier();
            compute((p & 1) ? lds1 : lds0, p, spb);
            sk_barrier();
        }
        // the last (clamped) DMA lands before the buffers are refilled or reused
        __builtin_amdgcn_s_waitcnt(vm_wait(0));
        sk_barrier();
    }

    // ---- the eight partial tiles meet in LDS (over the first A buffer),
    //      summed in wave order ----
    float *red = reinterpret_cast<float *>(lds0);
#pragma unroll
    for (int rf = 0; rf < RF; ++rf)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            red[((size_t)wave * MR + 32 * rf + 8 * (e >> 2) + 4 * h + (e & 3)) * 32 + r] = acc[rf][e];
    __syncthreads();
    for (int o = tid; o < MR * 32; o += 64 * SK_WAVES) {
        const int row = o >> 5, col = o & 31;
        const int n = 32 * t + col;
        if (row >= M || n >= N) continue;
        float total = 0.f;
#pragma unroll
        for (int w = 0; w < SK_WAVES; ++w) total += red[((size_t)w * MR + row) * 32 + col];
        if (raw)
            out[(size_t)row * N + n] = total;
        else
            epi_put(epi, C, row, n, N, total);
    }
}

template <int RF, int NB>
static hipError_t launch_skinny_nb(int M, int K, int N, const void *A, const void *Wp, const void *Sp,
                                   void *out, const Epilogue &epi, int pair_g, int nsplit, hipStream_t s) {
    auto kernel = pair_g == 4 ? gemm_int4b64_skinny_kernel<RF, 4, NB>
                : pair_g == 2 ? gemm_int4b64_skinny_kernel<RF, 2, NB> : gemm_int4b64_skinny_kernel<RF, 1, NB>;
    hipLaunchKernelGGL(kernel, dim3(div_up(N, 32), nsplit), dim3(64 * SK_WAVES), 0, s, M, K, N,
                       static_cast<const _Float16 *>(A), static_cast<const uint8_t *>(Wp),
                       static_cast<const float *>(Sp), out, epi);
    return hipGetLastError();
}

// NB, the weight records a wave requests at once: the fewest that cover the
// slice (at least one pass), at most 16 (8 with 64 rows; longer slices take
// several rounds)
template <int RF>
static hipError_t launch_skinny(int M, int K, int N, const void *A, const void *Wp, const void *Sp,
                                void *out, const Epilogue &epi, int pair_g, int nsplit, hipStream_t s) {
    const int per = div_up(K / BK, nsplit);                       // blocks of the longest slice
    const int need = div_up(per, SK_WAVES);
    if (need <= 2) return launch_skinny_nb<RF, 2>(M, K, N, A, Wp, Sp, out, epi, pair_g, nsplit, s);
    if (need <= 4) return launch_skinny_nb<RF, 4>(M, K, N, A, Wp, Sp, out, epi, pair_g, nsplit, s);
    // (with 64 rows, sixteen one-block passes per round would not stay unrolled)
    if (need <= 8 || RF == 2) return launch_skinny_nb<RF, 8>(M, K, N, A, Wp, Sp, out, epi, pair_g, nsplit, s);
    return launch_skinny_nb<RF, RF == 2 ? 8 : 16>(M, K, N, A, Wp, Sp, out, epi, pair_g, nsplit, s);
}

template <class T>
static hipError_t launch_tiles(int M, int K, int N, const void *A, const void *Wp, const void *Sp,
                               void *out, const Epilogue &epi, int pair_g, int nsplit,
                               hipStream_t s) {
    const int tiles_m = div_up(M, T::BM), tiles_n = div_up(N, T::BN);
    // Tile order. With a multiple of 8 column tiles, plain order (XCD x =
    // L % 8 takes the column tiles x, x + 8, ... of every row tile: an
    // interleaved eighth of B, all of A) measured fastest. Otherwise plain
    // order would give each XCD two column sets shifted between row tiles;
    // then the XCDs form a row-band x column-band grid (XCD x owns one band
    // of each, its L2 fetching only A of its row band and B of its column
    // band), the grid the tile counts divide that fetches the fewest bytes.
    int xcd_rows = 0;
    if (tiles_n % 8 != 0) {
        double best = 0;
        const double a_bytes = (double)M * K * 2, b_bytes = (double)N * K * 0.625;
        for (int gr = 1; gr <= 8; gr *= 2) {
            const int gc = 8 / gr;
            if (tiles_m % gr || tiles_n % gc) continue;
            const double fetched = gc * a_bytes + gr * b_bytes;
            if (xcd_rows == 0 || fetched < best) { xcd_rows = gr; best = fetched; }
        }
    }
    auto kernel = pair_g == 4 ? gemm_int4b64_kernel<T, 4>
                : pair_g == 2 ? gemm_int4b64_kernel<T, 2> : gemm_int4b64_kernel<T, 1>;
    hipLaunchKernelGGL(kernel, dim3(tiles_m * tiles_n, nsplit), dim3(64 * NWAVE), 0, s,
                       M, K, N, tiles_m, tiles_n, xcd_rows, static_cast<const _Float16 *>(A),
                       static_cast<const uint8_t *>(Wp), static_cast<const float *>(Sp), out, epi);
    return hipGetLastError();
}

hipError_t launch_gemm_int4b64(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, void *C, const Epilogue &epi, int pair_g,
                               int nsplit, float *part, hipStream_t s) {
    void *out = nsplit > 1 ? static_cast<void *>(part) : C;
    const Int4Tile t = int4_tile(M, N);
    hipError_t e = t.bn == 32 ? (t.bm == 32 ? launch_skinny<1>(M, K, N, A, Wp, Sp, out, epi, pair_g, nsplit, s)
                                            : launch_skinny<2>(M, K, N, A, Wp, Sp, out, epi, pair_g, nsplit, s))
                 : t.bm == 128 && t.bn == 128
        ? launch_tiles<TileCfg<128, 128>>(M, K, N, A, Wp, Sp, out, epi, pair_g, nsplit, s)
                 : t.bm == 128
        ? launch_tiles<TileCfg<128, 64>>(M, K, N, A, Wp, Sp, out, epi, pair_g, nsplit, s)
        : launch_tiles<TileCfg<64, 128>>(M, K, N, A, Wp, Sp, out, epi, pair_g, nsplit, s);
    if (e != hipSuccess || nsplit <= 1) return e;
    return launch_splitk_reduce_f32(part, nsplit, M, N, C, epi, s);
}

}  // namespace qg
