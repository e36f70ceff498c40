// gemv.hip -- streaming GEMV for the decode shape (M = 1, and small M up to
// the dispatch threshold) with Int4-Block64 and Int8-Block0 weights.
//
// What is computed (MNN GemmSpeed benchmark page, section "Why Conv1x1 is
// used to measure GEMM"): C[m][n] = sum_k A[m][k] * (offset + scale * q[n][k]),
// one [offset, scale] pair per (channel, block). Per block the sum is
// regrouped as offset * sum(a) + scale * sum(a * q), so the per-weight work
// is a code decode and a dot product; offset and scale are applied once per
// block. The page's observation that small M is bounded by the GEMV
// bandwidth floor (section "Sample data") makes these kernels HBM streams:
// every weight byte is read exactly once, with load instructions that cover
// 1 KiB of contiguous bytes (64 lanes x 16 bytes), all issued before the
// arithmetic needs them.
//
// Codes become fp16 by a magic-number decode (one v_and_or_b32 per pair of
// 4-bit codes, a byte permute per pair of 8-bit codes): a 4-bit code placed
// in mantissa bits 4..7 under exponent 2^10 reads
// as 1024 + 16 q, in bits 0..3 as 1024 + q; an 8-bit code in bits 0..7 reads
// as 1024 + q. The 1024 bias is removed per block with the block sums of the
// activations, so no per-weight subtract is needed; v_dot2_f32_f16 forms the
// products with fp32 accumulation.
#include <algorithm>
#include <type_traits>

#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

// Adds x over lane pairs (l, l xor 32) with one v_permlane32_swap: on return
// x + y is the pair's sum in both lanes.
__device__ __forceinline__ void swap32(float &x, float &y) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}

// Int4 pair entries (G per 64-block; see the packed layout): lane (c, h)
// decodes channel c's 32-element half h of a block, so it needs one pair
// (G = 1, 2) or the two pairs of its quarters (G = 4, one 16-byte load).
template <int G>
using Int4Pair = typename std::conditional<G == 4, f4_t, f2_t>::type;

template <int G>
__device__ __forceinline__ Int4Pair<G> load_int4_pair(const float *Sp, size_t rec, int c, int h) {
    if constexpr (G == 4)
        return __builtin_nontemporal_load(reinterpret_cast<const f4_t *>(Sp + rec * 256 + (4 * c + 2 * h) * 2));
    else if constexpr (G == 2)
        return __builtin_nontemporal_load(reinterpret_cast<const f2_t *>(Sp + rec * 128 + (32 * h + c) * 2));
    else
        return __builtin_nontemporal_load(reinterpret_cast<const f2_t *>(Sp + rec * 64 + c * 2));
}

// The decode's constants, opaque to the optimiser so that each lives in a
// register once (an instruction here takes at most one scalar operand and
// no literal): the nibble masks 0x000F000F / 0x00F000F0 and the fp16 pair
// 1024.0, 1024.0.
struct Int4Magic {
    unsigned m_lo, m_hi, magic;
};
__device__ __forceinline__ Int4Magic int4_magic() {
    Int4Magic k{0x000F000Fu, 0x00F000F0u, 0x64006400u};
    asm volatile("" : "+s"(k.m_lo), "+s"(k.m_hi));
    asm volatile("" : "+v"(k.magic));
    return k;
}

// One 32-code half of a block against its staged activations (the pieces
// av[d] of words d = 0..3 and, per quarter qh, the even / odd activation sums
// sv[qh]): sum_k a_k (offset + scale q_k), regrouped per pair as offset * sum(a)
// + scale * sum(a * q) with q read off the fp16 magic decode (OR-ing a code
// into the mantissa of 1024.0: 1024 + q for a low nibble, 1024 + 16 q for a
// high one left in place; one v_and_or_b32 per two codes), the 1024 bias
// removed through the sums. Word byte i holds codes 2 i (low nibble) and
// 2 i + 1, so the masked word gives codes (0, 4) and (1, 5), the word shifted
// by 8 codes (2, 6) and (3, 7): the activation pieces' pair order.
template <int G>
__device__ __forceinline__ float int4_half_dot(const u4_t (&av)[4], const unsigned (&word)[4],
                                               const f2_t *sv, const Int4Pair<G> &pp,
                                               const Int4Magic &k) {
    constexpr int GQ = G == 4 ? 2 : 1;
    float total = 0.f;
#pragma unroll
    for (int qh = 0; qh < GQ; ++qh) {
        float Te = 0.f, To = 0.f;
#pragma unroll
        for (int d = qh * 4 / GQ; d < (qh + 1) * 4 / GQ; ++d) {
            const unsigned w = word[d], w8 = w >> 8;
            Te = dot2(as_h2((w & k.m_lo) | k.magic), as_h2(av[d].x), Te);
            Te = dot2(as_h2((w8 & k.m_lo) | k.magic), as_h2(av[d].y), Te);
            To = dot2(as_h2((w & k.m_hi) | k.magic), as_h2(av[d].z), To);
            To = dot2(as_h2((w8 & k.m_hi) | k.magic), as_h2(av[d].w), To);
        }
        float off, sc;
        if constexpr (G == 4) {
            off = qh ? pp.z : pp.x;
            sc = qh ? pp.w : pp.y;
        } else {
            off = pp.x;
            sc = pp.y;
        }
        const float ce = fmaf(-1024.0f, sc, off);
        const float co = fmaf(-64.0f, sc, off);
        total += fmaf(ce, sv[qh].x, fmaf(co, sv[qh].y, fmaf(sc, Te, sc * 0.0625f * To)));
    }
    return total;
}

// Stages one (row, half-block) of activations: the four 16-byte pieces in
// decode pair order into ap, and the even / odd sums of each of its GQ
// quarters-of-a-half into hs.
template <int GQ>
__device__ __forceinline__ void stage_int4_half(const u4_t (&araw)[4], u4_t *ap, f2_t *hs) {
    const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int qh = 0; qh < GQ; ++qh) {
        float se = 0.f, so = 0.f;
#pragma unroll
        for (int w = qh * 4 / GQ; w < (qh + 1) * 4 / GQ; ++w) {
            const u4_t v = araw[w];
            const h2_t p01 = as_h2(v.x), p23 = as_h2(v.y), p45 = as_h2(v.z), p67 = as_h2(v.w);
            const h2_t e0 = {p01.x, p45.x}, e1 = {p23.x, p67.x};
            const h2_t o0 = {p01.y, p45.y}, o1 = {p23.y, p67.y};
            se = dot2(e1, one, dot2(e0, one, se));
            so = dot2(o1, one, dot2(o0, one, so));
            ap[w] = u4_t{as_u(e0), as_u(e1), as_u(o0), as_u(o1)};
        }
        hs[qh] = f2_t{se, so};
    }
}

// ---------------------------------------------------------------------------
// Int4-Block64
// ---------------------------------------------------------------------------
// The Int4-Block64 decode kernel. One 1024-thread workgroup per 32-channel
// tile: every weight load is one whole 1 KiB record of the tile (64 lanes x
// 16 contiguous bytes, all lanes active) and every pair load one whole
// 256-byte pair record, the widest contiguous accesses the packed layout
// offers. K is walked in passes of up to 64 blocks (4096 elements); within a
// pass the blocks are dealt to the 16 waves round-robin and all of a wave's
// loads are issued before the pass's activations are staged. For one row two
// workgroups fit on a CU, so the tiles (about 1.3 per CU for a 7B FFN shape)
// are all resident at once without a cross-workgroup reduction. Lane
// (c, h) = (lane % 32, lane / 32) accumulates channel c, K-half h of its
// blocks; the halves meet with one v_permlane32_swap and the 16 waves'
// partial sums are added in LDS in a fixed order.
constexpr int TILE_WAVES = 16;
constexpr int TILE_PASS = 64;                   // K-blocks per pass
constexpr int TILE_RPW = TILE_PASS / TILE_WAVES;   // blocks per wave and pass

// G: pair entries per 64-block (1, 2 or 4; see load_int4_pair).
// SPLIT: K split over gridDim.z workgroups per tile (its own instantiation:
// the unsplit kernel keeps 53 registers, so two workgroups share a CU).
template <int MR, bool ONE_PASS, int G, bool SPLIT>
__global__ __launch_bounds__(64 * TILE_WAVES) void gemv_int4b64_tile_kernel(
    int M, int K, int N, const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ Sp, void *__restrict__ C, Epilogue epi) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int nblk = K >> 6;
    // split-K: workgroup z of gridDim.z takes the tile's blocks [KB0, KB1)
    // (all of them unless split) and then stores a raw partial tile
    const int KB0 = SPLIT ? slice_begin(blockIdx.z, nblk, gridDim.z) : 0;
    const int KB1 = SPLIT ? slice_begin(blockIdx.z + 1, nblk, gridDim.z) : nblk;
    const int pmax = min(SPLIT ? (nblk + (int)gridDim.z - 1) / (int)gridDim.z : nblk, TILE_PASS);
    constexpr int GQ = G == 4 ? 2 : 1;                                          // sums per half-block
    u4_t *ap = reinterpret_cast<u4_t *>(lds);                                   // [MR][pmax * 8]
    f2_t *hs = reinterpret_cast<f2_t *>(lds + (size_t)MR * pmax * 128);         // [MR][2 pmax][GQ]
    float *part = reinterpret_cast<float *>(lds + (size_t)MR * pmax * (128 + 16 * GQ));
    // part: [TILE_WAVES][MR][32]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int t = blockIdx.x;                // 32-channel tile
    const int m0 = blockIdx.y * MR;
    const int c = lane & 31, h = lane >> 5;
    const Int4Magic magic = int4_magic();

    float acc[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) acc[r] = 0.f;

    // ONE_PASS (K <= 4096) compiles the body once without a loop around it,
    // which keeps the single-pass load schedule straight-line
    for (int b0 = KB0; b0 < (ONE_PASS ? KB0 + 1 : KB1); b0 += TILE_PASS) {   // workgroup-uniform
        const int pb = min(KB1 - b0, TILE_PASS);             // blocks in this pass
        const int nhb = 2 * pb;
        // 1. this pass's activations (one (row, block, half) per thread)
        u4_t araw[4];
        const int ar = tid / nhb, ahb = tid - ar * nhb;
        const bool alive = tid < MR * nhb && m0 + ar < M;
        {
            const u4_t *src = reinterpret_cast<const u4_t *>(
                A + (size_t)(alive ? m0 + ar : 0) * K + (size_t)(alive ? 2 * b0 + ahb : 0) * 32);
#pragma unroll
            for (int w = 0; w < 4; ++w) araw[w] = alive ? src[w] : u4_t{0u, 0u, 0u, 0u};
        }
        // 2. every pair and record load of this wave for the pass
        //    (non-temporal). Loads are unconditional, block index clamped:
        //    with no skipped loads the compiler's in-order count of
        //    outstanding loads stays exact, so each block waits only for its
        //    own data. Clamped blocks are never used.
        Int4Pair<G> pr[TILE_RPW];
        u4_t wq[TILE_RPW];
#pragma unroll
        for (int i = 0; i < TILE_RPW; ++i) {
            const int b = b0 + min(wave + TILE_WAVES * i, pb - 1);
            pr[i] = load_int4_pair<G>(Sp, (size_t)t * nblk + b, c, h);
        }
#pragma unroll
        for (int i = 0; i < TILE_RPW; ++i) {
            const int b = b0 + min(wave + TILE_WAVES * i, pb - 1);
            wq[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u4_t *>(Wp + ((size_t)t * nblk + b) * 1024) + lane);
        }
        // 3. activations to LDS in decode pair order, with even / odd sums
        if (tid < MR * nhb)
            stage_int4_half<GQ>(araw, ap + (size_t)ar * (pmax * 8) + ahb * 4,
                                hs + ((size_t)ar * (2 * pmax) + ahb) * GQ);
        __syncthreads();

        // 4. decode and accumulate this wave's blocks of the pass
#pragma unroll
        for (int i = 0; i < TILE_RPW; ++i) {
            const int bl = wave + TILE_WAVES * i;
            if (bl >= pb) break;                             // wave-uniform
            const int hbg = 2 * bl + h;                      // half-block within the pass
            // row strides, opaque per block: computed here rather than for
            // every (row, block) up front, where they would hold more
            // registers than a 1024-thread workgroup has
            // (with G = 4 the compiler keeps pmax in a vector register and
            // cannot copy it to a scalar one)
            int pm = pmax;
            if constexpr (G == 4)
                asm volatile("" : "+v"(pm));
            else
                asm volatile("" : "+s"(pm));
            const unsigned word[4] = {wq[i][0], wq[i][1], wq[i][2], wq[i][3]};
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                u4_t av[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) av[d] = ap[(size_t)r * (pm * 8) + hbg * 4 + d];
                acc[r] += int4_half_dot<G>(av, word, hs + ((size_t)r * (2 * pm) + hbg) * GQ, pr[i], magic);
            }
        }
        if (!ONE_PASS && b0 + TILE_PASS < KB1) __syncthreads();   // LDS reused by the next pass
    }
    // 5. halves meet (lanes c and c + 32), then per-wave channel sums to LDS
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        float x = acc[r], y = acc[r];
        swap32(x, y);
        if (h == 0) part[(wave * MR + r) * 32 + c] = x + y;
    }
    __syncthreads();

    // 6. add the 16 waves' partial sums in a fixed order and store
    if (tid < MR * 32) {
        const int r = tid >> 5, cc = tid & 31;
        const int n = 32 * t + cc, m = m0 + r;
        float total = 0.f;
#pragma unroll
        for (int w = 0; w < TILE_WAVES; ++w) total += part[(w * MR + r) * 32 + cc];
        if (n < N && m < M) {
            if (SPLIT)
                static_cast<float *>(C)[((size_t)blockIdx.z * M + m) * N + n] = total;   // partial tile
            else if (epi.plain)
                static_cast<float *>(C)[(size_t)m * N + n] = total;
            else
                epi_put(epi, C, m, n, N, total);
        }
    }
}

// MR <= 8 rows (one pass over them), K in passes of up to 64 blocks (one
// pass for K <= 4096), no split: a workgroup of NW waves (eight; sixteen in the case below) per 16
// channels, half of a 32-channel tile, so a
// shape has twice as many workgroups of half the bytes and they spread more
// evenly over the CUs (11008 channels: 688 half tiles, at most 3 per CU
// against an average of 2.7, instead of 344 tiles at most 2 per CU against
// 1.3; 4096 channels: all 256 CUs instead of 128). Lane (c, h, j) =
// (lane % 16, lane / 16 % 2, lane / 32) takes channel c of the half, K-half h
// of block 2 (w + NW i) + j in step i of wave w of NW: one load instruction covers
// the 16 channels' pieces of both halves of two blocks (four 256-byte runs).
// The four lanes of each channel meet by one exchange across 16 lanes and one
// v_permlane32_swap; the waves in LDS in a fixed order.
constexpr int HALF_WAVES = 8;
// Sixteen waves for K in passes when every half tile has a CU of its own:
// twice the loads in flight per CU (measured at M = 1, K = 11008, N = 4096:
// 8.76 us against 9.11 with eight). Where the half tiles outnumber the CUs
// the eight-wave kernel stays: two sixteen-wave workgroups per CU would not
// hold them all at once (K = 4096, N = 11008: 7.9 us against 7.6).
constexpr int HALF_WAVES_WIDE = 16;

template <int MR, bool ONE_PASS, int G, int NW>
__global__ __launch_bounds__(64 * NW) void gemv_int4b64_half_kernel(
    int M, int K, int N, const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ Sp, void *__restrict__ C, Epilogue epi) {
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int RPW = TILE_PASS / (2 * NW);                                  // blocks per wave and pass
    constexpr int AS = (MR * 128 + 64 * NW - 1) / (64 * NW);   // staging slots per thread
    const int nblk = K >> 6;
    const int pmax = min(nblk, TILE_PASS);                                     // blocks per pass
    constexpr int GQ = G == 4 ? 2 : 1;                                         // sums per half-block
    u4_t *ap = reinterpret_cast<u4_t *>(lds);                                  // [MR][pmax * 8]
    f2_t *hs = reinterpret_cast<f2_t *>(lds + (size_t)MR * pmax * 128);        // [MR][2 pmax][GQ]
    float *part = reinterpret_cast<float *>(lds + (size_t)MR * pmax * (128 + 16 * GQ));   // [NW][MR][16]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int t = blockIdx.x >> 1;                   // 32-channel tile
    const int m0 = blockIdx.y * MR;
    const int c16 = lane & 15, h = (lane >> 4) & 1, j = lane >> 5;
    const int c = (blockIdx.x & 1) * 16 + c16;       // channel within the tile
    const Int4Magic magic = int4_magic();
    float acc[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) acc[r] = 0.f;

    // ONE_PASS (K <= 4096) compiles the body once without a loop around it
    for (int b0 = 0; b0 < (ONE_PASS ? 1 : nblk); b0 += TILE_PASS) {   // workgroup-uniform
    const int pb = min(nblk - b0, TILE_PASS);                          // blocks in this pass
    const int nhb = 2 * pb;

    // 1. the pass's activations (one (row, block, half) per thread and slot),
    //    then every pair and record load of this wave, unconditional from
    //    clamped block indices
    // (a wave none of whose threads stages an activation issues no load for
    // the slot: at one row only two of the eight waves do, and the others'
    // clamped loads would sit in the CU's address queue ahead of the weights)
    u4_t araw[AS][4];
#pragma unroll
    for (int sl = 0; sl < AS; ++sl) {
        const int idx = tid + 64 * NW * sl;
        const int ar = idx / nhb, ahb = idx - ar * nhb;
        const bool alive = ar < MR && m0 + ar < M;
        const u4_t *src = reinterpret_cast<const u4_t *>(
            A + (size_t)(alive ? m0 + ar : 0) * K + (size_t)(alive ? 2 * b0 + ahb : 0) * 32);
        if (64 * (NW * sl + wave) < MR * nhb) {     // wave-uniform
#pragma unroll
            for (int w = 0; w < 4; ++w) araw[sl][w] = alive ? src[w] : u4_t{0u, 0u, 0u, 0u};
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) araw[sl][w] = u4_t{0u, 0u, 0u, 0u};
        }
    }
    Int4Pair<G> pr[RPW];
    u4_t wq[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int b = b0 + min(2 * (wave + NW * i) + j, pb - 1);
        pr[i] = load_int4_pair<G>(Sp, (size_t)t * nblk + b, c, h);
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int b = b0 + min(2 * (wave + NW * i) + j, pb - 1);
        wq[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u4_t *>(Wp + ((size_t)t * nblk + b) * 1024) + 32 * h + c);
    }

    // 2. activations to LDS in decode pair order, with even / odd sums (rows
    //    past M are staged as zeros and never stored)
#pragma unroll
    for (int sl = 0; sl < AS; ++sl) {
        const int idx = tid + 64 * NW * sl;
        if (idx < MR * nhb)                  // idx = row * nhb + half-block
            stage_int4_half<GQ>(araw[sl], ap + (size_t)idx * 4, hs + (size_t)idx * GQ);
    }
    __syncthreads();

    // 3. decode and accumulate; a lane whose block lies past the pass (odd
    //    block count) computes on the clamped block and adds zero
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int bl = 2 * (wave + NW * i) + j;
        if (2 * (wave + NW * i) >= pb) break;     // wave-uniform
        const int hbg = 2 * min(bl, pb - 1) + h;
        const unsigned word[4] = {wq[i][0], wq[i][1], wq[i][2], wq[i][3]};
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            u4_t av[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) av[d] = ap[((size_t)r * nhb + hbg) * 4 + d];
            const float v = int4_half_dot<G>(av, word, hs + ((size_t)r * nhb + hbg) * GQ, pr[i], magic);
            acc[r] += bl < pb ? v : 0.f;
        }
    }
    if (!ONE_PASS && b0 + TILE_PASS < nblk) __syncthreads();   // LDS reused by the next pass
    }

    // 4. the K-halves (lanes c and c + 16), then the block parities (lanes
    //    l and l + 32), then the waves in a fixed order
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        float x = acc[r] + __shfl_xor(acc[r], 16);
        float y = x;
        swap32(x, y);
        if (lane < 16) part[(wave * MR + r) * 16 + c16] = x + y;
    }
    __syncthreads();
    if (tid < MR * 16) {
        const int r = tid >> 4, cc = tid & 15;
        const int n = 32 * t + (blockIdx.x & 1) * 16 + cc, m = m0 + r;
        float total = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) total += part[(w * MR + r) * 16 + cc];
        if (n < N && m < M) {
            if (epi.plain) static_cast<float *>(C)[(size_t)m * N + n] = total;
            else epi_put(epi, C, m, n, N, total);
        }
    }
}

// ---------------------------------------------------------------------------
// Int8-Block0
// ---------------------------------------------------------------------------
// One 1024-thread workgroup per 16 channels, one wave per channel. A
// channel's codes are one contiguous run of Kp bytes: lane l reads the
// 16-byte slices l, l + 64, ... of it, so each load instruction is 1 KiB of
// contiguous bytes, and every slice a wave needs is requested before the
// activations are staged. Loads are unconditional with clamped indices
// (slices past the row end reread the last slice and are skipped in the
// arithmetic), which keeps the compiler's in-order count of outstanding
// loads exact. Per channel, sum(a * w) = offset * sum(a) + scale * sum(a * q);
// sum(a) is formed once per workgroup.
//
// Blocked Int8 (PM = 1: a pair per 64-block; PM = 2: per 32-element half;
// PM = 4: per 16-element quarter; K % 64 == 0): the same regrouping per
// 16-code slice, whose codes all lie in one block: the slice adds
// scale * sum(a * (1024 + q)) + (offset - 1024 scale) * sum(a) with its
// block's pair, sum(a) over the slice's 16 activations coming from per-piece
// sums staged in LDS with the activations. Each lane requests its slices'
// pairs (8 bytes, shared by the 4, 2 or 1 lanes of a pair entry) with its
// codes.
constexpr int I8_WAVES = 16;

template <int MR, int NCH, int PM>
__global__ __launch_bounds__(64 * I8_WAVES) void gemv_int8b0_kernel(
    int M, int K, int N, int Kp, const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    const f2_t *__restrict__ Sp, void *__restrict__ C, Epilogue epi) {
    extern __shared__ __align__(16) unsigned char lds[];
    _Float16 *As = reinterpret_cast<_Float16 *>(lds);                      // [MR][Kp], zero past K
    float *ssum = reinterpret_cast<float *>(lds + (size_t)MR * Kp * 2);    // [MR][I8_WAVES]
    float *psum = ssum + MR * I8_WAVES;                                    // PM: [MR][Kp / 8]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int m0 = blockIdx.y * MR;
    const int Np = (N + 3) & ~3;
    const int n = blockIdx.x * I8_WAVES + wave;
    const int nc = min(n, Np - 1);
    const int nchunk = Kp >> 4;              // 16-byte slices per channel

    // 0. the activation pieces this thread stages, requested first: loads
    //    complete in order, so staged after the weights they would wait for
    //    the wave's whole weight stream (when at most two per thread; else
    //    they are loaded in step 2)
    const int pieces = Kp >> 3;
    constexpr int AS = (MR * NCH * 128 + 64 * I8_WAVES - 1) / (64 * I8_WAVES);   // >= slots needed
    constexpr bool A_FIRST = AS <= 2;
    const bool vec_a = (K & 7) == 0;
    u4_t araw[A_FIRST ? AS : 1];
    if constexpr (A_FIRST) {
#pragma unroll
        for (int sl = 0; sl < AS; ++sl) {
            const int p = tid + 64 * I8_WAVES * sl;
            const int r = p / pieces, c = p - r * pieces;
            araw[sl] = u4_t{0u, 0u, 0u, 0u};
            if (vec_a && p < MR * pieces && m0 + r < M && c * 8 < K)
                araw[sl] = *reinterpret_cast<const u4_t *>(A + (size_t)(m0 + r) * K + (size_t)c * 8);
        }
    }

    // 1. this wave's code slices and pair
    u4_t wq[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int ci = min(lane + 64 * i, nchunk - 1);
        wq[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u4_t *>(Wp + (size_t)nc * Kp + (size_t)ci * 16));
    }
    // slice ci's pair: entry ci >> SH of the channel's nchunk >> SH entries
    constexpr int SH = PM == 4 ? 0 : PM == 2 ? 1 : 2;
    f2_t pb[PM ? NCH : 1];
    if constexpr (PM != 0) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int ci = min(lane + 64 * i, nchunk - 1);
            pb[i] = Sp[(size_t)nc * (nchunk >> SH) + (ci >> SH)];
        }
    }
    const f2_t pr = PM ? f2_t{0.f, 0.f} : Sp[nc];

    // 2. activations to LDS (zero past K), and their row sums
    float part[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) part[r] = 0.f;
    const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    if (vec_a) {
        for (int p = tid, sl = 0; p < MR * pieces; p += 64 * I8_WAVES, ++sl) {
            const int r = p / pieces, c = p - r * pieces;
            u4_t v = {0u, 0u, 0u, 0u};
            if constexpr (A_FIRST)
                v = araw[sl < AS ? sl : 0];
            else if (m0 + r < M && c * 8 < K)
                v = *reinterpret_cast<const u4_t *>(A + (size_t)(m0 + r) * K + (size_t)c * 8);
            *reinterpret_cast<u4_t *>(As + (size_t)r * Kp + (size_t)c * 8) = v;
            float sp = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) sp = dot2(as_h2(v[i]), one, sp);
            if (PM) psum[p] = sp;            // p = r * pieces + c
#pragma unroll
            for (int rr = 0; rr < MR; ++rr) part[rr] += (rr == r) ? sp : 0.f;
        }
    } else {
        for (int e = tid; e < MR * Kp; e += 64 * I8_WAVES) {
            const int r = e / Kp, k = e - r * Kp;
            const _Float16 v = (m0 + r < M && k < K) ? A[(size_t)(m0 + r) * K + k] : (_Float16)0.0f;
            As[e] = v;
#pragma unroll
            for (int rr = 0; rr < MR; ++rr) part[rr] += (rr == r) ? (float)v : 0.f;
        }
    }
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        float v = part[r];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0) ssum[r * I8_WAVES + wave] = v;
    }
    __syncthreads();

    // 3. sum(a * (1024 + q)) per row over this lane's slices
    float T[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) T[r] = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int ci = lane + 64 * i;
        if (ci >= nchunk) break;
        float Ts[MR];                        // PM: this slice's sum(a * (1024 + q))
#pragma unroll
        for (int r = 0; r < MR; ++r) Ts[r] = 0.f;
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
            const unsigned word = wq[i][wi];
            // bytes (q0, q1) and (q2, q3) under 0x64: halves 1024 + q
            const h2_t x0 = as_h2(__builtin_amdgcn_perm(0x64646464u, word, 0x04010400u));
            const h2_t x1 = as_h2(__builtin_amdgcn_perm(0x64646464u, word, 0x04030402u));
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const u2_t av = *reinterpret_cast<const u2_t *>(As + (size_t)r * Kp + ci * 16 + wi * 4);
                float &t = PM ? Ts[r] : T[r];
                t = dot2(x0, as_h2(av.x), t);
                t = dot2(x1, as_h2(av.y), t);
            }
        }
        if constexpr (PM != 0) {
            const float c1b = fmaf(-1024.0f, pb[i].y, pb[i].x);
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const float2 ps = *reinterpret_cast<const float2 *>(psum + (size_t)r * (Kp >> 3) + 2 * ci);
                T[r] = fmaf(pb[i].y, Ts[r], fmaf(c1b, ps.x + ps.y, T[r]));
            }
        }
    }
    // 4. per row: reduce over the wave, then offset * sum(a) + scale * sum(a q)
    //    with sum(a q) = T - 1024 sum(a)
    const float c1 = fmaf(-1024.0f, pr.y, pr.x);
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        float v = T[r];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0 && n < N && m0 + r < M) {
            float sa = 0.f;
#pragma unroll
            for (int w = 0; w < I8_WAVES; ++w) sa += ssum[r * I8_WAVES + w];
            const float out = PM ? v : fmaf(c1, sa, pr.y * v);
            if (epi.plain) static_cast<float *>(C)[(size_t)(m0 + r) * N + n] = out;
            else epi_put(epi, C, m0 + r, n, N, out);
        }
    }
}

// ---------------------------------------------------------------------------
// fp16-weight GEMV (the float mode at FP16 precision): the Int8-Block0
// structure with fp16 channel rows [Np][Kp]. One wave per channel reads its
// row as 16-byte slices l, l + 64, ... (eight weights each; 1 KiB of
// contiguous bytes per load instruction), all requested before the
// activations are staged in LDS; each weight pair meets its activation pair
// in one v_dot2 (products exact in fp32, fp32 sums).
// ---------------------------------------------------------------------------
template <int MR, int NCH>
__global__ __launch_bounds__(64 * I8_WAVES) void gemv_f16_kernel(
    int M, int K, int N, int Kp, const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    void *__restrict__ C, Epilogue epi) {
    extern __shared__ __align__(16) unsigned char lds[];
    _Float16 *As = reinterpret_cast<_Float16 *>(lds);   // [MR][Kp], zero past K
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int m0 = blockIdx.y * MR;
    const int Np = (N + 3) & ~3;
    const int n = blockIdx.x * I8_WAVES + wave;
    const int nc = min(n, Np - 1);
    const int nslice = Kp >> 3;              // 16-byte slices per channel

    // 0. with two or more rows, the activation pieces this thread stages,
    //    requested before the weights (as in the Int8 kernel: loads complete
    //    in order). Measured, one box: M = 2 and 4 at K = N = 4096 8.1 -> 7.6
    //    and 9.6 -> 9.3 us, but M = 1 6.83 -> 7.0 us, so one row keeps the
    //    weights first.
    const int pieces = Kp >> 3;
    constexpr int AS = (MR * NCH * 64 + 64 * I8_WAVES - 1) / (64 * I8_WAVES);   // >= slots needed
    constexpr bool A_FIRST = MR > 1 && AS <= 2;
    const bool vec_a = (K & 7) == 0;
    u4_t araw[A_FIRST ? AS : 1];
    if constexpr (A_FIRST) {
#pragma unroll
        for (int sl = 0; sl < AS; ++sl) {
            const int p = tid + 64 * I8_WAVES * sl;
            const int r = p / pieces, c = p - r * pieces;
            araw[sl] = u4_t{0u, 0u, 0u, 0u};
            if (vec_a && p < MR * pieces && m0 + r < M && c * 8 < K)
                araw[sl] = *reinterpret_cast<const u4_t *>(A + (size_t)(m0 + r) * K + (size_t)c * 8);
        }
    }

    // 1. this wave's weight slices (clamped: slices past the row end reread
    //    the last slice and are skipped in the arithmetic)
    u4_t wq[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int ci = min(lane + 64 * i, nslice - 1);
        wq[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u4_t *>(Wp + ((size_t)nc * Kp + (size_t)ci * 8) * 2));
    }

    // 2. activations to LDS, zero past K
    if (vec_a) {
        for (int p = tid, sl = 0; p < MR * pieces; p += 64 * I8_WAVES, ++sl) {
            const int r = p / pieces, c = p - r * pieces;
            u4_t v = {0u, 0u, 0u, 0u};
            if constexpr (A_FIRST)
                v = araw[sl < AS ? sl : 0];
            else if (m0 + r < M && c * 8 < K)
                v = *reinterpret_cast<const u4_t *>(A + (size_t)(m0 + r) * K + (size_t)c * 8);
            *reinterpret_cast<u4_t *>(As + (size_t)r * Kp + (size_t)c * 8) = v;
        }
    } else {
        for (int e = tid; e < MR * Kp; e += 64 * I8_WAVES) {
            const int r = e / Kp, k = e - r * Kp;
            As[e] = (m0 + r < M && k < K) ? A[(size_t)(m0 + r) * K + k] : (_Float16)0.0f;
        }
    }
    __syncthreads();

    // 3. sum(a * w) per row over this lane's slices
    float T[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) T[r] = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int ci = lane + 64 * i;
        if (ci >= nslice) break;
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const u4_t av = *reinterpret_cast<const u4_t *>(As + (size_t)r * Kp + (size_t)ci * 8);
#pragma unroll
            for (int wi = 0; wi < 4; ++wi) T[r] = dot2(as_h2(wq[i][wi]), as_h2(av[wi]), T[r]);
        }
    }
    // 4. per row: reduce over the wave and store
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        float v = T[r];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0 && n < N && m0 + r < M) {
            if (epi.plain) static_cast<float *>(C)[(size_t)(m0 + r) * N + n] = v;
            else epi_put(epi, C, m0 + r, n, N, v);
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static int rows_per_pass(int M, int K, int kp_bytes_per_row) {
    // Rows of A staged in LDS at once (up to all M <= 8, so that the weights
    // stream once): they and the reduction space fit in kGemvLds bytes.
    (void)K;
    int mr = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
    while (mr > 1 && (size_t)mr * kp_bytes_per_row > kGemvLds - 2048) mr >>= 1;
    return mr;
}

template <int MR, int G>
static hipError_t gemv_int4_tile(int M, int K, int N, const void *A, const void *Wp,
                                 const void *Sp, void *C, const Epilogue &epi, int nsplit,
                                 hipStream_t s) {
    const int per = div_up(K / 64, nsplit);                // most blocks of a slice
    const int pmax = std::min(per, TILE_PASS);
    const size_t lds = (size_t)MR * pmax * (128 + 16 * (G == 4 ? 2 : 1)) +
                       (size_t)TILE_WAVES * MR * 32 * sizeof(float);
    dim3 grid(div_up(N, 32), div_up(M, MR), nsplit);
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(64 * TILE_WAVES), lds, s, M, K, N,
                           static_cast<const _Float16 *>(A), static_cast<const uint8_t *>(Wp),
                           static_cast<const float *>(Sp), C, epi);
    };
    if (nsplit > 1) {
        if (per <= TILE_PASS) go(gemv_int4b64_tile_kernel<MR, true, G, true>);
        else go(gemv_int4b64_tile_kernel<MR, false, G, true>);
    } else {
        if (per <= TILE_PASS) go(gemv_int4b64_tile_kernel<MR, true, G, false>);
        else go(gemv_int4b64_tile_kernel<MR, false, G, false>);
    }
    return hipGetLastError();
}

template <int MR>
static hipError_t gemv_int4_tile(int M, int K, int N, const void *A, const void *Wp,
                                 const void *Sp, void *C, const Epilogue &epi, int pair_g,
                                 int nsplit, hipStream_t s) {
    return pair_g == 4 ? gemv_int4_tile<MR, 4>(M, K, N, A, Wp, Sp, C, epi, nsplit, s)
         : pair_g == 2 ? gemv_int4_tile<MR, 2>(M, K, N, A, Wp, Sp, C, epi, nsplit, s)
                       : gemv_int4_tile<MR, 1>(M, K, N, A, Wp, Sp, C, epi, nsplit, s);
}

static hipError_t gemv_int4_rows(int M, int K, int N, const void *A, const void *Wp,
                                 const void *Sp, void *C, const Epilogue &epi, int pair_g,
                                 int nsplit, hipStream_t s);

hipError_t launch_gemv_int4b64(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, void *C, const Epilogue &epi, int pair_g,
                               int nsplit, float *part, hipStream_t s) {
    if (nsplit <= 1) return gemv_int4_rows(M, K, N, A, Wp, Sp, C, epi, pair_g, 1, s);
    const hipError_t e = gemv_int4_rows(M, K, N, A, Wp, Sp, part, epi, pair_g, nsplit, s);
    if (e != hipSuccess) return e;
    return launch_splitk_reduce_f32(part, nsplit, M, N, C, epi, s);
}

static hipError_t gemv_int4_rows(int M, int K, int N, const void *A, const void *Wp,
                                 const void *Sp, void *C, const Epilogue &epi, int pair_g,
                                 int nsplit, hipStream_t s) {
    if (nsplit <= 1) {
        // one pass over the rows: half tiles
        auto half = [&](auto mr) {
            constexpr int MR = decltype(mr)::value;
            const bool one = K <= 64 * TILE_PASS;
            const long long groups = (long long)div_up(N, 16) * div_up(M, MR);
            const int nw = !one && groups <= kSplitTargetCUs ? HALF_WAVES_WIDE : HALF_WAVES;
            const size_t lds = (size_t)MR * std::min(K / 64, TILE_PASS) * (128 + 16 * (pair_g == 4 ? 2 : 1)) +
                               (size_t)nw * MR * 16 * sizeof(float);
            auto go = [&](auto kernel) {
                hipLaunchKernelGGL(kernel, dim3(div_up(N, 16), div_up(M, MR)), dim3(64 * nw),
                                   lds, s, M, K, N, static_cast<const _Float16 *>(A),
                                   static_cast<const uint8_t *>(Wp), static_cast<const float *>(Sp),
                                   C, epi);
            };
            constexpr int W8 = HALF_WAVES, W16 = HALF_WAVES_WIDE;
            auto pick = [&](auto one_pass, auto waves) {
                constexpr bool OP = decltype(one_pass)::value;
                constexpr int NWV = decltype(waves)::value;
                if (pair_g == 4) go(gemv_int4b64_half_kernel<MR, OP, 4, NWV>);
                else if (pair_g == 2) go(gemv_int4b64_half_kernel<MR, OP, 2, NWV>);
                else go(gemv_int4b64_half_kernel<MR, OP, 1, NWV>);
            };
            if (one) pick(std::true_type{}, std::integral_constant<int, W8>{});
            else if (nw == W16) pick(std::false_type{}, std::integral_constant<int, W16>{});
            else pick(std::false_type{}, std::integral_constant<int, W8>{});
            return hipGetLastError();
        };
        switch (M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8) {
        case 8: return half(std::integral_constant<int, 8>{});
        case 4: return half(std::integral_constant<int, 4>{});
        case 2: return half(std::integral_constant<int, 2>{});
        default: return half(std::integral_constant<int, 1>{});
        }
    }
    // all rows in one pass (at most 88 KiB of LDS for eight), so the weights stream once
    switch (M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8) {
    case 8: return gemv_int4_tile<8>(M, K, N, A, Wp, Sp, C, epi, pair_g, nsplit, s);
    case 4: return gemv_int4_tile<4>(M, K, N, A, Wp, Sp, C, epi, pair_g, nsplit, s);
    case 2: return gemv_int4_tile<2>(M, K, N, A, Wp, Sp, C, epi, pair_g, nsplit, s);
    default: return gemv_int4_tile<1>(M, K, N, A, Wp, Sp, C, epi, pair_g, nsplit, s);
    }
}

template <int MR, int NCH, int PM>
static hipError_t gemv_int8_mr(int M, int K, int N, int Kp, const void *A, const void *Wp,
                               const void *Sp, void *C, const Epilogue &epi, hipStream_t s) {
    dim3 grid(div_up(N, I8_WAVES), div_up(M, MR));
    const size_t lds = (size_t)MR * Kp * sizeof(_Float16) + (size_t)MR * I8_WAVES * sizeof(float) +
                       (PM ? (size_t)MR * (Kp / 8) * sizeof(float) : 0);
    hipLaunchKernelGGL((gemv_int8b0_kernel<MR, NCH, PM>), grid, dim3(64 * I8_WAVES), lds, s, M, K,
                       N, Kp, static_cast<const _Float16 *>(A), static_cast<const uint8_t *>(Wp),
                       static_cast<const f2_t *>(Sp), C, epi);
    return hipGetLastError();
}

template <int MR, int PM>
static hipError_t gemv_int8_k(int M, int K, int N, int Kp, const void *A, const void *Wp,
                              const void *Sp, void *C, const Epilogue &epi, hipStream_t s) {
    // slices per lane: Kp / 1024, rounded up to a power of two (K <= 16384;
    // blocked Int8: K <= 8192, eight slices and their pairs)
    const int nch = div_up(Kp, 1024);
    if (nch <= 1) return gemv_int8_mr<MR, 1, PM>(M, K, N, Kp, A, Wp, Sp, C, epi, s);
    if (nch <= 2) return gemv_int8_mr<MR, 2, PM>(M, K, N, Kp, A, Wp, Sp, C, epi, s);
    if (nch <= 4) return gemv_int8_mr<MR, 4, PM>(M, K, N, Kp, A, Wp, Sp, C, epi, s);
    if (PM || nch <= 8) return gemv_int8_mr<MR, 8, PM>(M, K, N, Kp, A, Wp, Sp, C, epi, s);
    return gemv_int8_mr<MR, 16, 0>(M, K, N, Kp, A, Wp, Sp, C, epi, s);
}

template <int PM>
static hipError_t gemv_int8_rows(int M, int K, int N, const void *A, const void *Wp,
                                 const void *Sp, void *C, const Epilogue &epi, hipStream_t s) {
    const int Kp = (int)round_up(K, 64);
    // the dispatcher sends at most four rows here (the tiled kernel wins
    // above); per row: the fp16 activations, and the piece sums when blocked
    switch (rows_per_pass(M < 4 ? M : 4, K, Kp * 2 + (PM ? Kp / 2 : 0))) {
    case 4: return gemv_int8_k<4, PM>(M, K, N, Kp, A, Wp, Sp, C, epi, s);
    case 2: return gemv_int8_k<2, PM>(M, K, N, Kp, A, Wp, Sp, C, epi, s);
    default: return gemv_int8_k<1, PM>(M, K, N, Kp, A, Wp, Sp, C, epi, s);
    }
}

hipError_t launch_gemv_int8b0(int M, int K, int N, const void *A, const void *Wp,
                              const void *Sp, void *C, const Epilogue &epi, hipStream_t s) {
    return gemv_int8_rows<0>(M, K, N, A, Wp, Sp, C, epi, s);
}

hipError_t launch_gemv_int8blk(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, void *C, const Epilogue &epi, int pair_g,
                               hipStream_t s) {
    return pair_g == 4 ? gemv_int8_rows<4>(M, K, N, A, Wp, Sp, C, epi, s)
         : pair_g == 2 ? gemv_int8_rows<2>(M, K, N, A, Wp, Sp, C, epi, s)
                       : gemv_int8_rows<1>(M, K, N, A, Wp, Sp, C, epi, s);
}

template <int MR, int NCH>
static hipError_t gemv_f16_mr(int M, int K, int N, int Kp, const void *A, const void *Wp, void *C,
                              const Epilogue &epi, hipStream_t s) {
    dim3 grid(div_up(N, I8_WAVES), div_up(M, MR));
    const size_t lds = (size_t)MR * Kp * sizeof(_Float16);
    hipLaunchKernelGGL((gemv_f16_kernel<MR, NCH>), grid, dim3(64 * I8_WAVES), lds, s, M, K, N, Kp,
                       static_cast<const _Float16 *>(A), static_cast<const uint8_t *>(Wp), C, epi);
    return hipGetLastError();
}

template <int MR>
static hipError_t gemv_f16_k(int M, int K, int N, int Kp, const void *A, const void *Wp, void *C,
                             const Epilogue &epi, hipStream_t s) {
    // slices per lane: Kp / 512, rounded up to a power of two (K <= 8192)
    const int nch = div_up(Kp, 512);
    if (nch <= 1) return gemv_f16_mr<MR, 1>(M, K, N, Kp, A, Wp, C, epi, s);
    if (nch <= 2) return gemv_f16_mr<MR, 2>(M, K, N, Kp, A, Wp, C, epi, s);
    if (nch <= 4) return gemv_f16_mr<MR, 4>(M, K, N, Kp, A, Wp, C, epi, s);
    if (nch <= 8) return gemv_f16_mr<MR, 8>(M, K, N, Kp, A, Wp, C, epi, s);
    return gemv_f16_mr<MR, 16>(M, K, N, Kp, A, Wp, C, epi, s);
}

hipError_t launch_gemv_f16(int M, int K, int N, const void *A, const void *Wp, void *C,
                           const Epilogue &epi, hipStream_t s) {
    const int Kp = (int)round_up(K, 64);
    switch (rows_per_pass(M, K, Kp * 2)) {
    case 8: return gemv_f16_k<8>(M, K, N, Kp, A, Wp, C, epi, s);
    case 4: return gemv_f16_k<4>(M, K, N, Kp, A, Wp, C, epi, s);
    case 2: return gemv_f16_k<2>(M, K, N, Kp, A, Wp, C, epi, s);
    default: return gemv_f16_k<1>(M, K, N, Kp, A, Wp, C, epi, s);
    }
}

}  // namespace qg
