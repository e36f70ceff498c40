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
// activations are decoded once per block slot and reused for all channels;
// for Int4 they are read straight from global memory (the 8 KiB row stays in
// L1/L2), issued ahead of the weight stream so their latency hides under it.
// Codes become fp16 by a magic-number decode (one byte permute per pair of
// codes): a 4-bit code placed in mantissa bits 4..7 under exponent 2^10 reads
// as 1024 + 16 q; an 8-bit code in bits 0..7 reads as 1024 + q. The bias is removed per block with the
// block sum of the activations, so no per-weight subtract is needed.
// The partial sums of the 64 lanes are combined by a transposing butterfly
// (each exchange step halves the values a lane holds) before the store.
#include <algorithm>

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

// Same contract as wave_transpose_sum, with every exchange done in
// registers: v_permlane32_swap / v_permlane16_swap for lane distances 32 and
// 16, DPP row_ror:8, row_half_mirror and quad permutes below that. Each
// exchange pairs a lane with one whose bit of that step differs, so the
// halving bookkeeping is the same as for xor partners.
__device__ __forceinline__ void swap32(float &x, float &y) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float &x, float &y) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF, true));
}
// partner of bit 3: row_ror:8; bit 2: row_half_mirror; bit 1: quad_perm
// [2,3,0,1]; bit 0: quad_perm [1,0,3,2]
template <int BIT>
__device__ __forceinline__ float partner(float v) {
    if constexpr (BIT == 3) return dpp<0x128>(v);
    else if constexpr (BIT == 2) return dpp<0x141>(v);
    else if constexpr (BIT == 1) return dpp<0x4E>(v);
    else return dpp<0xB1>(v);
}

template <int NV, int STEP = 0>
__device__ __forceinline__ void dpp_halve(float (&v)[NV], int lane, int &idx) {
    constexpr int L = Log2<NV>::value;
    if constexpr (STEP < L) {
        constexpr int half = NV >> (STEP + 1);
        constexpr int bit = 5 - STEP;
        const bool up = (lane >> bit) & 1;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            float x = v[i], y = v[i + half];
            if constexpr (bit == 5) {
                swap32(x, y);
                v[i] = x + y;
            } else if constexpr (bit == 4) {
                swap16(x, y);
                v[i] = x + y;
            } else {
                const float keep = up ? y : x;
                const float send = up ? x : y;
                v[i] = keep + partner<bit>(send);
            }
        }
        if (up) idx += half;
        dpp_halve<NV, STEP + 1>(v, lane, idx);
    }
}

// ---------------------------------------------------------------------------
// Int4-Block64
//
// Packed records (see the layout notes in qgemm_internal.h): record (t, b) of
// a 32-channel tile holds, for each half h of block b, the 16 code bytes of
// each channel; four consecutive channels of one half are a 64-byte run. A
// wave owns groups of 4 channels (so every CU gets the same number of bytes,
// to within one group) and reads a group with lanes
//   lane = 8 bb + 4 h + c:  channel c of the group, half h, block 8 i + bb
// for load i = 0..7 (64 blocks = K 4096 per pass), i.e. 16 runs of 64 bytes
// per 1 KiB load. The activations of every (block, half) are staged once per
// workgroup in LDS, already in the pair order the decode needs, with their
// even / odd position sums.
// ---------------------------------------------------------------------------
constexpr int GEMV_LOADS = 8;            // 1 KiB loads per group per pass
constexpr int GEMV_PASS_BLOCKS = 64;     // K-blocks per pass

// Reduces v[0..NV) over lane bits 5..2 (the lanes sharing lane & 3); NV <= 8.
// Bit 2 goes first, with DPP row_shr:4 (lanes with bit 2 set receive the sum),
// then bits 5, 4, 3 transpose-halve (permlane32 / permlane16 swaps, row_ror:8:
// all keep bits 0..2). On return, lanes with bit 2 set and zero unused bits
// among 3..5 hold value `idx`.
template <int NV>
__device__ __forceinline__ float group_transpose_sum(float (&v)[NV], int lane, int &idx) {
    constexpr int L = Log2<NV>::value;
    static_assert((1 << L) == NV && L <= 3, "NV must be a power of two <= 8");
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] += dpp<0x114>(v[i]);   // row_shr:4
    idx = 0;
    dpp_halve<NV>(v, lane, idx);
    float s = v[0];
#pragma unroll
    for (int bit = 5 - L; bit >= 3; --bit) {
        if (bit == 5) { float x = s, y = s; swap32(x, y); s = x + y; }
        else if (bit == 4) { float x = s, y = s; swap16(x, y); s = x + y; }
        else s += partner<3>(s);
    }
    return s;
}

template <int MR, int MAXG, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_int4b64_kernel(
    int M, int K, int N, const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ Sp, float *__restrict__ C) {
    // LDS: per row, per 8-group w: 16 bytes {(a0,a4),(a2,a6),(a1,a5),(a3,a7)};
    // per row, per (block, half): {sum a_even, sum a_odd}.
    extern __shared__ __align__(16) unsigned char lds[];
    const int nblk = K >> 6;
    const int nhb = nblk * 2;
    const int pk = min(K, GEMV_PASS_BLOCKS * 64);                     // K per pass
    u4_t *ap = reinterpret_cast<u4_t *>(lds);                         // [MR][pk/8]
    f2_t *hs = reinterpret_cast<f2_t *>(lds + (size_t)MR * pk * 2);   // [MR][pk/32]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int m0 = blockIdx.y * MR;
    const int G = (N + 3) >> 2;
    const long long nwg = gridDim.x;
    const int gs = (int)((long long)blockIdx.x * G / nwg);
    const int ge = (int)((long long)(blockIdx.x + 1) * G / nwg);
    const int g0 = uniform(gs + wave);
    const bool active = g0 < ge;

    const int cc = lane & 3, hh = (lane >> 2) & 1, bb = lane >> 3;
    const unsigned magic = 0x64646464u;
    constexpr int NV0 = MAXG * MR;
    constexpr int NV = NV0 <= 1 ? 1 : (NV0 <= 2 ? 2 : (NV0 <= 4 ? 4 : 8));
    static_assert(NV0 <= 8, "at most 8 outputs per lane");
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.f;

    for (int pass = 0; pass * GEMV_PASS_BLOCKS < nblk; ++pass) {
        // 1. this pass's activations, one (row, block, half) item per thread
        //    and slot, loaded first so they do not queue behind the weights
        const int hb0 = pass * GEMV_PASS_BLOCKS * 2;
        const int nh = min(nhb - hb0, GEMV_PASS_BLOCKS * 2);
        constexpr int SLOTS = (MR * GEMV_PASS_BLOCKS * 2 + 64 * WAVES - 1) / (64 * WAVES);
        u4_t araw[SLOTS][4];
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
            const int it = tid + sl * 64 * WAVES;
            const int r = it / nh, hbl = it - r * nh;
            const bool live = it < MR * nh && m0 + r < M;
            const u4_t *src = reinterpret_cast<const u4_t *>(
                A + (size_t)(live ? m0 + r : 0) * K + (live ? hb0 + hbl : 0) * 32);
#pragma unroll
            for (int w = 0; w < 4; ++w) araw[sl][w] = live ? src[w] : u4_t{0u, 0u, 0u, 0u};
        }
        // 2. every weight and pair load of this pass (non-temporal: read once)
        u4_t wq[MAXG][GEMV_LOADS];
        f2_t pr[MAXG][GEMV_LOADS];
#pragma unroll
        for (int gi = 0; gi < MAXG; ++gi) {
            const int g = g0 + WAVES * gi;
            const int t = g >> 3, q = g & 7;
#pragma unroll
            for (int i = 0; i < GEMV_LOADS; ++i) {
                const int b = pass * GEMV_PASS_BLOCKS + 8 * i + bb;
                if (active && g < ge && b < nblk) {
                    const size_t rec = (size_t)t * nblk + b;
                    wq[gi][i] = __builtin_nontemporal_load(
                        reinterpret_cast<const u4_t *>(Wp + rec * 1024 + (size_t)(32 * hh + 4 * q + cc) * 16));
                    pr[gi][i] = __builtin_nontemporal_load(
                        reinterpret_cast<const f2_t *>(Sp + rec * 64 + (4 * q + cc) * 2));
                } else {
                    wq[gi][i] = u4_t{0u, 0u, 0u, 0u};
                    pr[gi][i] = f2_t{0.f, 0.f};
                }
            }
        }
        // 3. activations to LDS in decode pair order, with even / odd sums
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
            const int it = tid + sl * 64 * WAVES;
            if (it < MR * nh) {
                const int r = it / nh, hbl = it - r * nh;
                float se = 0.f, so = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const u4_t v = araw[sl][w];
                    const h2_t p01 = as_h2(v.x), p23 = as_h2(v.y), p45 = as_h2(v.z), p67 = as_h2(v.w);
                    const h2_t e0 = {p01.x, p45.x}, e1 = {p23.x, p67.x};
                    const h2_t o0 = {p01.y, p45.y}, o1 = {p23.y, p67.y};
                    const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
                    se = dot2(e1, one, dot2(e0, one, se));
                    so = dot2(o1, one, dot2(o0, one, so));
                    ap[(size_t)r * (pk >> 3) + hbl * 4 + w] = u4_t{as_u(e0), as_u(e1), as_u(o0), as_u(o1)};
                }
                hs[(size_t)r * (pk >> 5) + hbl] = f2_t{se, so};
            }
        }
        __syncthreads();

        // 4. decode and accumulate
        if (active) {
#pragma unroll
            for (int i = 0; i < GEMV_LOADS; ++i) {
                const int bl = 8 * i + bb;                  // block within the pass
                const int hbl = 2 * bl + hh;
                if (pass * GEMV_PASS_BLOCKS + bl >= nblk) continue;
                u4_t av[MR][4];
                f2_t sv[MR];
#pragma unroll
                for (int r = 0; r < MR; ++r) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) av[r][w] = ap[(size_t)r * (pk >> 3) + hbl * 4 + w];
                    sv[r] = hs[(size_t)r * (pk >> 5) + hbl];
                }
#pragma unroll
                for (int gi = 0; gi < MAXG; ++gi) {
                    float Te[MR], To[MR];
#pragma unroll
                    for (int r = 0; r < MR; ++r) Te[r] = To[r] = 0.f;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const unsigned word = wq[gi][i][d];
                        // one byte permute puts code byte (q_even | q_odd << 4)
                        // under the fp16 exponent 2^10; masking keeps 1024 + q_even
                        // or 1024 + 16 q_odd
                        const unsigned y0 = __builtin_amdgcn_perm(magic, word, 0x04020400u);
                        const unsigned y1 = __builtin_amdgcn_perm(magic, word, 0x04030401u);
                        const h2_t e0 = as_h2(y0 & 0xFF0FFF0Fu), e1 = as_h2(y1 & 0xFF0FFF0Fu);
                        const h2_t o0 = as_h2(y0 & 0xFFF0FFF0u), o1 = as_h2(y1 & 0xFFF0FFF0u);
#pragma unroll
                        for (int r = 0; r < MR; ++r) {
                            Te[r] = dot2(e0, as_h2(av[r][d].x), Te[r]);
                            Te[r] = dot2(e1, as_h2(av[r][d].y), Te[r]);
                            To[r] = dot2(o0, as_h2(av[r][d].z), To[r]);
                            To[r] = dot2(o1, as_h2(av[r][d].w), To[r]);
                        }
                    }
                    const float off = pr[gi][i].x, sc = pr[gi][i].y;
                    // Te = 1024 s_even + sum(a q_even), To = 1024 s_odd + 16 sum(a q_odd)
                    const float ce = fmaf(-1024.0f, sc, off);
                    const float co = fmaf(-64.0f, sc, off);
                    const float so16 = sc * 0.0625f;
#pragma unroll
                    for (int r = 0; r < MR; ++r)
                        acc[gi * MR + r] += fmaf(ce, sv[r].x, fmaf(co, sv[r].y, fmaf(sc, Te[r], so16 * To[r])));
                }
            }
        }
        if ((pass + 1) * GEMV_PASS_BLOCKS < nblk) __syncthreads();   // LDS reused next pass
    }
    if (!active) return;

    int idx;
    const float total = group_transpose_sum<NV>(acc, lane, idx);
    constexpr int USED = Log2<NV>::value;   // lane bits 5 .. 6-USED carry idx
    const int rest_mask = ((1 << (3 - USED)) - 1) << 3;   // bits 3 .. 5-USED
    if ((lane & 4) && (lane & rest_mask) == 0 && idx < NV0) {
        const int r = idx % MR;
        const int gi = idx / MR;
        const int g = g0 + WAVES * gi;
        const int n = 4 * g + cc;
        const int m = m0 + r;
        if (g < ge && n < N && m < M) C[(size_t)m * N + n] = total;
    }
}

// The decode kernel for K <= 4096. One 1024-thread workgroup per 32-channel
// tile: every weight load is one whole 1 KiB record of the tile (64 lanes x
// 16 contiguous bytes, all lanes active) and every pair load one whole
// 256-byte pair record, the widest contiguous accesses the packed layout
// offers. The tile's K-blocks are dealt to the 16 waves round-robin and all
// of a wave's loads are issued before the activations are staged. For one
// row two workgroups fit on a CU, so the tiles (about 1.3 per CU for a 7B
// FFN shape) are all resident at once without a cross-workgroup reduction.
// Lane (c, h) = (lane % 32, lane / 32) accumulates channel c, K-half h of its
// blocks; the halves meet with one v_permlane32_swap and the 16 waves'
// partial sums are added in LDS in a fixed order.
constexpr int TILE_WAVES = 16;
constexpr int TILE_RPW = 64 / TILE_WAVES;      // blocks per wave (K <= 4096)

template <int MR>
__global__ __launch_bounds__(64 * TILE_WAVES) void gemv_int4b64_tile_kernel(
    int M, int K, int N, const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ Sp, float *__restrict__ C) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int nblk = K >> 6;                 // 1 .. 64
    const int nhb = nblk * 2;
    u4_t *ap = reinterpret_cast<u4_t *>(lds);                                   // [MR][K/8]
    f2_t *hs = reinterpret_cast<f2_t *>(lds + (size_t)MR * K * 2);              // [MR][nhb]
    float *part = reinterpret_cast<float *>(lds + (size_t)MR * K * 2 + (size_t)MR * nhb * 8);
    // part: [TILE_WAVES][MR][32]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int t = blockIdx.x;                // 32-channel tile
    const int m0 = blockIdx.y * MR;
    const int c = lane & 31, h = lane >> 5;

    // 1. activations for this workgroup (one (row, block, half) per thread)
    u4_t araw[4];
    const int ar = tid / nhb, ahb = tid - ar * nhb;
    const bool alive = tid < MR * nhb && m0 + ar < M;
    {
        const u4_t *src = reinterpret_cast<const u4_t *>(
            A + (size_t)(alive ? m0 + ar : 0) * K + (alive ? ahb : 0) * 32);
#pragma unroll
        for (int w = 0; w < 4; ++w) araw[w] = alive ? src[w] : u4_t{0u, 0u, 0u, 0u};
    }
    // 2. every pair and record load of this wave (non-temporal). Loads are
    //    unconditional, block index clamped: with no skipped loads the
    //    compiler's in-order count of outstanding loads stays exact, so each
    //    block waits only for its own data. Clamped blocks are never used.
    f2_t pr[TILE_RPW];
    u4_t wq[TILE_RPW];
#pragma unroll
    for (int i = 0; i < TILE_RPW; ++i) {
        const int b = min(wave + TILE_WAVES * i, nblk - 1);
        pr[i] = __builtin_nontemporal_load(
            reinterpret_cast<const f2_t *>(Sp + ((size_t)t * nblk + b) * 64 + c * 2));
    }
#pragma unroll
    for (int i = 0; i < TILE_RPW; ++i) {
        const int b = min(wave + TILE_WAVES * i, nblk - 1);
        wq[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u4_t *>(Wp + ((size_t)t * nblk + b) * 1024) + lane);
    }
    // 3. activations to LDS in decode pair order, with even / odd sums
    if (tid < MR * nhb) {
        float se = 0.f, so = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const u4_t v = araw[w];
            const h2_t p01 = as_h2(v.x), p23 = as_h2(v.y), p45 = as_h2(v.z), p67 = as_h2(v.w);
            const h2_t e0 = {p01.x, p45.x}, e1 = {p23.x, p67.x};
            const h2_t o0 = {p01.y, p45.y}, o1 = {p23.y, p67.y};
            const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
            se = dot2(e1, one, dot2(e0, one, se));
            so = dot2(o1, one, dot2(o0, one, so));
            ap[(size_t)ar * (K >> 3) + ahb * 4 + w] = u4_t{as_u(e0), as_u(e1), as_u(o0), as_u(o1)};
        }
        hs[(size_t)ar * nhb + ahb] = f2_t{se, so};
    }
    __syncthreads();

    // 4. decode and accumulate this wave's blocks
    const unsigned magic = 0x64646464u;
    float acc[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < TILE_RPW; ++i) {
        const int b = wave + TILE_WAVES * i;
        if (b >= nblk) break;                            // wave-uniform
        const int hbg = 2 * b + h;
        const float off = pr[i].x, sc = pr[i].y;
        const float ce = fmaf(-1024.0f, sc, off);
        const float co = fmaf(-64.0f, sc, off);
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            float Te = 0.f, To = 0.f;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const u4_t av = ap[(size_t)r * (K >> 3) + hbg * 4 + d];
                const unsigned word = wq[i][d];
                const unsigned y0 = __builtin_amdgcn_perm(magic, word, 0x04020400u);
                const unsigned y1 = __builtin_amdgcn_perm(magic, word, 0x04030401u);
                Te = dot2(as_h2(y0 & 0xFF0FFF0Fu), as_h2(av.x), Te);
                Te = dot2(as_h2(y1 & 0xFF0FFF0Fu), as_h2(av.y), Te);
                To = dot2(as_h2(y0 & 0xFFF0FFF0u), as_h2(av.z), To);
                To = dot2(as_h2(y1 & 0xFFF0FFF0u), as_h2(av.w), To);
            }
            const f2_t sv = hs[(size_t)r * nhb + hbg];
            acc[r] += fmaf(ce, sv.x, fmaf(co, sv.y, fmaf(sc, Te, sc * 0.0625f * To)));
        }
    }
    // 5. halves meet (lanes c and c + 32), then per-wave channel sums to LDS
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        float x = acc[r], y = acc[r];
        swap32(x, y);
        if (h == 0) part[(wave * MR + r) * 32 + c] = x + y;
    }
    __syncthreads();

    // 6. add the eight waves' partial sums in a fixed order and store
    if (tid < MR * 32) {
        const int r = tid >> 5, cc = tid & 31;
        const int n = 32 * t + cc, m = m0 + r;
        float total = 0.f;
#pragma unroll
        for (int w = 0; w < TILE_WAVES; ++w) total += part[(w * MR + r) * 32 + cc];
        if (n < N && m < M) C[(size_t)m * N + n] = total;
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
constexpr int I8_WAVES = 16;

template <int MR, int NCH>
__global__ __launch_bounds__(64 * I8_WAVES) void gemv_int8b0_kernel(
    int M, int K, int N, int Kp, const _Float16 *__restrict__ A, const uint8_t *__restrict__ Wp,
    const f2_t *__restrict__ Sp, float *__restrict__ C) {
    extern __shared__ __align__(16) unsigned char lds[];
    _Float16 *As = reinterpret_cast<_Float16 *>(lds);                      // [MR][Kp], zero past K
    float *ssum = reinterpret_cast<float *>(lds + (size_t)MR * Kp * 2);    // [MR][I8_WAVES]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int m0 = blockIdx.y * MR;
    const int Np = (N + 3) & ~3;
    const int n = blockIdx.x * I8_WAVES + wave;
    const int nc = min(n, Np - 1);
    const int nchunk = Kp >> 4;              // 16-byte slices per channel

    // 1. this wave's code slices and pair
    u4_t wq[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int ci = min(lane + 64 * i, nchunk - 1);
        wq[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u4_t *>(Wp + (size_t)nc * Kp + (size_t)ci * 16));
    }
    const f2_t pr = Sp[nc];

    // 2. activations to LDS (zero past K), and their row sums
    float part[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) part[r] = 0.f;
    const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    if ((K & 7) == 0) {
        const int pieces = Kp >> 3;
        for (int p = tid; p < MR * pieces; p += 64 * I8_WAVES) {
            const int r = p / pieces, c = p - r * pieces;
            u4_t v = {0u, 0u, 0u, 0u};
            if (m0 + r < M && c * 8 < K)
                v = *reinterpret_cast<const u4_t *>(A + (size_t)(m0 + r) * K + (size_t)c * 8);
            *reinterpret_cast<u4_t *>(As + (size_t)r * Kp + (size_t)c * 8) = v;
            float sp = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) sp = dot2(as_h2(v[i]), one, sp);
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
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
            const unsigned word = wq[i][wi];
            // bytes (q0, q1) and (q2, q3) under 0x64: halves 1024 + q
            const h2_t x0 = as_h2(__builtin_amdgcn_perm(0x64646464u, word, 0x04010400u));
            const h2_t x1 = as_h2(__builtin_amdgcn_perm(0x64646464u, word, 0x04030402u));
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const u2_t av = *reinterpret_cast<const u2_t *>(As + (size_t)r * Kp + ci * 16 + wi * 4);
                T[r] = dot2(x0, as_h2(av.x), T[r]);
                T[r] = dot2(x1, as_h2(av.y), T[r]);
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
            C[(size_t)(m0 + r) * N + n] = fmaf(c1, sa, pr.y * v);
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static int rows_per_pass(int M, int K, int kp_bytes_per_row) {
    // Rows of A staged in LDS at once: they and 1 KiB of reduction space fit
    // in 64 KiB of LDS.
    (void)K;
    int mr = M >= 4 ? 4 : (M >= 2 ? 2 : 1);
    while (mr > 1 && mr * kp_bytes_per_row > 65536 - 1024) mr >>= 1;
    return mr;
}

// Compute units of the current device (cached per device ordinal).
static int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] <= 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cached[dev] = v;
    }
    return cached[dev];
}

template <int MR, int MAXG>
static hipError_t gemv_int4(int M, int K, int N, const void *A, const void *Wp, const void *Sp,
                            float *C, hipStream_t s) {
    constexpr int WAVES = 4;
    const int G = (N + 3) / 4;
    const int nwg = std::max(cu_count(), div_up(G, WAVES * MAXG));
    const int pass_k = std::min(K, GEMV_PASS_BLOCKS * 64);
    const size_t lds = (size_t)MR * pass_k * 2 + (size_t)MR * (pass_k / 32) * sizeof(f2_t);
    dim3 grid(nwg, div_up(M, MR));
    hipLaunchKernelGGL((gemv_int4b64_kernel<MR, MAXG, WAVES>), grid, dim3(64 * WAVES), lds, s, M, K,
                       N, static_cast<const _Float16 *>(A), static_cast<const uint8_t *>(Wp),
                       static_cast<const float *>(Sp), C);
    return hipGetLastError();
}

template <int MR>
static hipError_t gemv_int4_tile(int M, int K, int N, const void *A, const void *Wp,
                                 const void *Sp, float *C, hipStream_t s) {
    const size_t lds = (size_t)MR * K * 2 + (size_t)MR * (K / 32) * sizeof(f2_t) +
                       (size_t)TILE_WAVES * MR * 32 * sizeof(float);
    dim3 grid(div_up(N, 32), div_up(M, MR));
    hipLaunchKernelGGL((gemv_int4b64_tile_kernel<MR>), grid, dim3(64 * TILE_WAVES), lds, s, M, K,
                       N, static_cast<const _Float16 *>(A), static_cast<const uint8_t *>(Wp),
                       static_cast<const float *>(Sp), C);
    return hipGetLastError();
}

hipError_t launch_gemv_int4b64(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, float *C, hipStream_t s) {
    if (K <= 4096) {
        switch (M >= 4 ? 4 : (M >= 2 ? 2 : 1)) {
        case 4: return gemv_int4_tile<4>(M, K, N, A, Wp, Sp, C, s);
        case 2: return gemv_int4_tile<2>(M, K, N, A, Wp, Sp, C, s);
        default: return gemv_int4_tile<1>(M, K, N, A, Wp, Sp, C, s);
        }
    }
    switch (M >= 4 ? 4 : (M >= 2 ? 2 : 1)) {
    case 4: return gemv_int4<4, 2>(M, K, N, A, Wp, Sp, C, s);
    case 2: return gemv_int4<2, 2>(M, K, N, A, Wp, Sp, C, s);
    default: return gemv_int4<1, 3>(M, K, N, A, Wp, Sp, C, s);
    }
}

template <int MR, int NCH>
static hipError_t gemv_int8_mr(int M, int K, int N, int Kp, const void *A, const void *Wp,
                               const void *Sp, float *C, hipStream_t s) {
    dim3 grid(div_up(N, I8_WAVES), div_up(M, MR));
    const size_t lds = (size_t)MR * Kp * sizeof(_Float16) + (size_t)MR * I8_WAVES * sizeof(float);
    hipLaunchKernelGGL((gemv_int8b0_kernel<MR, NCH>), grid, dim3(64 * I8_WAVES), lds, s, M, K, N,
                       Kp, static_cast<const _Float16 *>(A), static_cast<const uint8_t *>(Wp),
                       static_cast<const f2_t *>(Sp), C);
    return hipGetLastError();
}

template <int MR>
static hipError_t gemv_int8_k(int M, int K, int N, int Kp, const void *A, const void *Wp,
                              const void *Sp, float *C, hipStream_t s) {
    // slices per lane: Kp / 1024, rounded up to a power of two (K <= 16384)
    const int nch = div_up(Kp, 1024);
    if (nch <= 1) return gemv_int8_mr<MR, 1>(M, K, N, Kp, A, Wp, Sp, C, s);
    if (nch <= 2) return gemv_int8_mr<MR, 2>(M, K, N, Kp, A, Wp, Sp, C, s);
    if (nch <= 4) return gemv_int8_mr<MR, 4>(M, K, N, Kp, A, Wp, Sp, C, s);
    if (nch <= 8) return gemv_int8_mr<MR, 8>(M, K, N, Kp, A, Wp, Sp, C, s);
    return gemv_int8_mr<MR, 16>(M, K, N, Kp, A, Wp, Sp, C, s);
}

hipError_t launch_gemv_int8b0(int M, int K, int N, const void *A, const void *Wp,
                              const void *Sp, float *C, hipStream_t s) {
    const int Kp = (int)round_up(K, 64);
    switch (rows_per_pass(M, K, Kp * 2)) {
    case 4: return gemv_int8_k<4>(M, K, N, Kp, A, Wp, Sp, C, s);
    case 2: return gemv_int8_k<2>(M, K, N, Kp, A, Wp, Sp, C, s);
    default: return gemv_int8_k<1>(M, K, N, Kp, A, Wp, Sp, C, s);
    }
}

}  // namespace qg
