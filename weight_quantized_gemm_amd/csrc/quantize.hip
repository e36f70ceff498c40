// quantize.hip -- the weight export step on the GPU: float weights [N][K] ->
// 4- or 8-bit codes and [offset, scale] pairs, written either in the
// canonical layout or straight into the packed layouts the GEMM kernels read.
//
// MNN GemmSpeed page, section "Why Conv1x1 is used to measure GEMM": the
// weights are quantised offline (the converter's export), asymmetrically,
// one [offset, scale] pair per (channel, block of K). Per block the offset is
// the minimum, the scale (maximum - minimum) / (2^bits - 1) and a weight's
// code rint((w - offset) / scale) clamped to [0, 2^bits - 1]. The kernel
// takes every step in the same IEEE double operations as the host quantiser
// (the pair from double, rounded to float; the quotient from the stored
// float pair, in double, rounded half to even), so its codes and pairs equal
// the host's bit for bit.
//
// One wave per channel. Lane l of a 64-element chunk holds k = 64 j + l; the
// chunks are loaded eight at a time, every load unconditional from a clamped
// index, and the codes leave as 32-bit words assembled across lanes.
#include "kernels_common.h"

#pragma clang fp contract(off)

namespace qg {
namespace {

constexpr int kQWaves = 4;     // channels (waves) per workgroup
constexpr int kQUnroll = 8;    // 64-element chunks loaded per batch

struct QParams {
    const float *W;
    int K, N;
    int rows;        // channels the grid covers: N (canonical) or the padded Np (packed)
    int nkc;         // 64-element chunks per row: ceil(K / 64)
    int block, nblk; // K-elements per pair and pairs per channel
    int kp;          // packed Int8-Block0 row length
    uint8_t *q;      // codes
    float *pairs;    // pairs
    int tail_off, tail_len;   // floats of the packed pair buffer past the last pair (zeroed)
};

__device__ inline float wave_min(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m));
    return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

__device__ inline uint32_t group_or(uint32_t x, int lanes) {
    // OR over aligned groups of `lanes` (4 or 8) lanes
    x |= __shfl_xor(x, 1);
    x |= __shfl_xor(x, 2);
    if (lanes == 8) x |= __shfl_xor(x, 4);
    return x;
}

// The pair of one block from its reduced minimum and maximum.
__device__ inline float2 block_pair(float lo, float hi, int qmax, bool bad, bool live) {
    float2 p;
    p.x = lo;
    p.y = (float)(((double)hi - (double)lo) / (double)qmax);
    if (bad) p.x = p.y = __builtin_nanf("");   // a non-finite weight poisons its block
    if (!live) p.x = p.y = 0.0f;               // padding channels of a packed buffer
    return p;
}

// Code of one weight from its block's stored float pair: rint of the double
// quotient (w - offset) / scale, clamped. rcp = 1 / scale, correctly rounded
// to float (once per block). The float estimate t = RN(RN(w - offset) * rcp)
// carries three roundings, so |t - exact| <= 3 * 2^-24 * 255 < 5e-5 for every
// code range here, and the double quotient is within 2^-50 of the exact one.
// Unless t lies within 2^-12 of a half-integer (or is not finite), all three
// round to the same integer, and the float estimate's is returned; otherwise
// the double quotient decides. The result is the double path's in every case.
__device__ inline int code_of(float w, float2 p, float rcp, int qmax) {
    if (p.y == 0.0f) return 0;
    const float t = (w - p.x) * rcp;
    const float rt = rintf(t);
    float r;
    if (fabsf(t - rt) < 0.5f - 0x1p-12f) {
        r = rt;
    } else {
        r = (float)rint(((double)w - (double)p.x) / (double)p.y);
    }
    r = r < 0.0f ? 0.0f : (r > (float)qmax ? (float)qmax : r);
    return (int)r;
}

// Stores the codes of chunk kc (k = 64 kc + lane) of channel n. Every lane
// calls it (the word assembly crosses lanes); codes past K arrive as 0.
template <int OUT, int BITS>
__device__ inline void store_codes(const QParams &p, int n, int kc, int lane, int code) {
    const int k = kc * 64 + lane;
    if (OUT == QGEMM_F32) {           // canonical layout (the format's own slot is unused here)
        if (BITS == 8) {
            if (k < p.K) p.q[(size_t)n * p.K + k] = (uint8_t)code;
        } else if ((p.K & 7) == 0) {
            // rows start on 4-byte boundaries: one word per 8 codes
            const uint32_t x = group_or((uint32_t)code << (4 * (lane & 7)), 8);
            if ((lane & 7) == 0 && k < p.K)
                *reinterpret_cast<uint32_t *>(p.q + (size_t)n * (p.K / 2) + k / 2) = x;
        } else {
            uint32_t x = (uint32_t)code << (4 * (lane & 1));
            x |= __shfl_xor(x, 1);
            if ((lane & 1) == 0 && k < p.K) p.q[(size_t)n * (p.K / 2) + k / 2] = (uint8_t)x;
        }
    } else if (OUT == QGEMM_INT4_B64) {
        // record (n / 32, kc); piece 32 h + (n % 32) holds canonical bytes
        // [16 h, 16 h + 16) of the block, word w of it codes 32 h + 8 w + [0, 8)
        const uint32_t x = group_or((uint32_t)code << (4 * (lane & 7)), 8);
        const int G = lane >> 3, h = G >> 2, w = G & 3;
        const size_t rec = (size_t)(n >> 5) * p.nkc + kc;
        if ((lane & 7) == 0)
            *reinterpret_cast<uint32_t *>(p.q + rec * 1024 + (size_t)(32 * h + (n & 31)) * 16 + 4 * w) = x;
    } else if (OUT == QGEMM_INT8_B0 || OUT == QGEMM_INT8_BLOCK_BASE) {
        const uint32_t x = group_or((uint32_t)code << (8 * (lane & 3)), 4);
        if ((lane & 3) == 0)
            *reinterpret_cast<uint32_t *>(p.q + (size_t)n * p.kp + k) = x;
    } else {                          // W4A8
        // word of k0 = 64 kc + 32 s + 16 h + 8 w: byte i = q[k0 + i] | q[k0 + 4 + i] << 4
        const uint32_t x = group_or((uint32_t)code << (8 * (lane & 3) + 4 * ((lane >> 2) & 1)), 8);
        const int G = lane >> 3, s = G >> 2, h = (G >> 1) & 1, w = G & 1;
        const size_t rec = (size_t)(n >> 5) * p.nkc + kc;
        if ((lane & 7) == 0)
            *reinterpret_cast<uint32_t *>(p.q + rec * 1024 + (size_t)(32 * h + (n & 31)) * 16 + 8 * s + 4 * w) = x;
    }
}

// OUT: QGEMM_F32 stands for the canonical layout, else the packed layout of
// that format (the other Int4 block sizes pack as QGEMM_INT4_B64 with
// REPEAT). B64: one pair per 64-block; else blocks of p.block elements (all
// of K for the per-channel formats), each reduced before its codes.
template <int OUT, int BITS, bool B64, bool REPEAT>
__global__ __launch_bounds__(64 * kQWaves) void quantize_kernel(QParams p) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * kQWaves + (threadIdx.x >> 6);
    if (blockIdx.x == 0 && threadIdx.x < 64)
        for (int i = lane; i < p.tail_len; i += 64) p.pairs[p.tail_off + i] = 0.0f;
    if (n >= p.rows) return;                       // whole waves only
    const bool live = n < p.N;
    const float *row = p.W + (size_t)(live ? n : p.N - 1) * p.K;
    constexpr int qmax = (1 << BITS) - 1;

    if (B64) {
        // K % 64 == 0: chunk kc is block kc
        for (int j0 = 0; j0 < p.nkc; j0 += kQUnroll) {
            float v[kQUnroll];
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) v[u] = row[min((j0 + u) * 64 + lane, p.K - 1)];
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) {
                const int kc = j0 + u;
                if (kc >= p.nkc) break;            // uniform
                const bool bad = __ballot(!__builtin_isfinite(v[u])) != 0;
                float lo = wave_min(v[u]), hi = wave_max(v[u]);
                if (lo == 0.0f || hi == 0.0f) {
                    // equal extremes differ only in the sign of zero: the first zero
                    // in k order is the one a sequential scan keeps
                    const unsigned long long z = __ballot(v[u] == 0.0f);
                    const float z0 = __shfl(v[u], __builtin_ctzll(z));
                    lo = lo == 0.0f ? z0 : lo;
                    hi = hi == 0.0f ? z0 : hi;
                }
                const float2 pr = block_pair(lo, hi, qmax, bad, live);
                const float rcp = 1.0f / pr.y;     // IEEE division, once per block
                const int code = (live && !bad) ? code_of(v[u], pr, rcp, qmax) : 0;
                store_codes<OUT, BITS>(p, n, kc, lane, code);
                if (lane == 0) {
                    const size_t pi = (OUT == QGEMM_F32 || OUT == QGEMM_INT8_BLOCK_BASE)
                                          ? (size_t)n * p.nkc + kc
                                          : ((size_t)(n >> 5) * p.nkc + kc) * 32 + (n & 31);
                    reinterpret_cast<float2 *>(p.pairs)[pi] = pr;
                }
            }
        }
        return;
    }

    // blocks of several chunks: each block's minimum and maximum, then its codes
    const int cpb = (p.block + 63) / 64;           // chunks per block
    for (int blk = 0; blk < p.nblk; ++blk) {
        const int c0 = blk * cpb, c1 = min(c0 + cpb, p.nkc);
        const int kend = min((blk + 1) * p.block, p.K);
        float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
        bool bad_lane = false;
        for (int j0 = c0; j0 < c1; j0 += kQUnroll) {
            float v[kQUnroll];
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) v[u] = row[min((j0 + u) * 64 + lane, p.K - 1)];
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) {
                const bool valid = live && (j0 + u) * 64 + lane < kend;
                lo = valid ? fminf(lo, v[u]) : lo;
                hi = valid ? fmaxf(hi, v[u]) : hi;
                bad_lane |= valid && !__builtin_isfinite(v[u]);
            }
        }
        const bool bad = __ballot(bad_lane) != 0;
        lo = wave_min(lo);
        hi = wave_max(hi);
        if ((lo == 0.0f || hi == 0.0f) && !bad) {
            // an extreme of 0: the first zero in k order carries the sign a
            // sequential scan keeps (rare, so found by a second scan)
            for (int kc = c0; kc < c1; ++kc) {
                const int k = kc * 64 + lane;
                const float v = row[min(k, p.K - 1)];
                const unsigned long long z = __ballot(k < kend && v == 0.0f);
                if (z) {
                    const float z0 = __shfl(v, __builtin_ctzll(z));
                    lo = lo == 0.0f ? z0 : lo;
                    hi = hi == 0.0f ? z0 : hi;
                    break;
                }
            }
        }
        const float2 pr = block_pair(lo, hi, qmax, bad, live);
        const float rcp = 1.0f / pr.y;             // IEEE division, once per block
        for (int j0 = c0; j0 < c1; j0 += kQUnroll) {
            float v[kQUnroll];
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) v[u] = row[min((j0 + u) * 64 + lane, p.K - 1)];
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) {
                const int kc = j0 + u;
                if (kc >= c1) break;                   // uniform
                const bool valid = live && !bad && kc * 64 + lane < kend;
                store_codes<OUT, BITS>(p, n, kc, lane, valid ? code_of(v[u], pr, rcp, qmax) : 0);
            }
        }
        float2 *pp = reinterpret_cast<float2 *>(p.pairs);
        if (OUT == QGEMM_F32) {
            if (lane == 0) pp[(size_t)n * p.nblk + blk] = pr;
        } else if (REPEAT && OUT == QGEMM_INT8_BLOCK_BASE) {
            // blocked Int8: the pair in every 64-block entry of the block
            for (int b = c0 + lane; b < c1; b += 64) pp[(size_t)n * p.nkc + b] = pr;
        } else if (REPEAT) {
            // packed as Int4-Block64: the pair in every 64-block record of the block
            for (int b = c0 + lane; b < c1; b += 64) pp[((size_t)(n >> 5) * p.nkc + b) * 32 + (n & 31)] = pr;
        } else if (lane == 0) {
            pp[n] = pr;
        }
    }
}

// ---------------------------------------------------------------------------
// Four weights per lane (K % 4 == 0): lane l of a 256-element chunk j holds
// k = 256 j + 4 l .. + 3 (one 16-byte load), so a 64-block spans 16 lanes and
// its reduction four cross-lane steps, and each load moves four times the
// bytes. G > 0: blocks of 4 G elements (32, 64, 128 or 256), G lanes each, a
// whole number of them per chunk. G == 0: blocks of whole chunks (a multiple
// of 256 elements, or all of K), reduced over a first pass and coded in a
// second. Same arithmetic, same results as quantize_kernel.
// ---------------------------------------------------------------------------
template <int G>
__device__ inline float group_min(float v) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) v = fminf(v, __shfl_xor(v, m));
    return v;
}
template <int G>
__device__ inline float group_max(float v) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}
template <int G>
__device__ inline int group_imin(int v) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) v = min(v, __shfl_xor(v, m));
    return v;
}

// Stores the four codes of lane `lane` in chunk j of channel n (k0 = 256 j +
// 4 lane). Every lane calls it (the W4A8 words pair lanes).
template <int OUT, int BITS>
__device__ inline void store_codes4(const QParams &p, int n, int j, int lane, const int (&c)[4]) {
    const int k0 = 256 * j + 4 * lane;
    if (OUT == QGEMM_F32) {
        if (BITS == 8) {
            if (k0 < p.K)
                *reinterpret_cast<uint32_t *>(p.q + (size_t)n * p.K + k0) =
                    (uint32_t)c[0] | (uint32_t)c[1] << 8 | (uint32_t)c[2] << 16 | (uint32_t)c[3] << 24;
        } else if (k0 < p.K) {
            *reinterpret_cast<uint16_t *>(p.q + (size_t)n * (p.K / 2) + k0 / 2) =
                (uint16_t)(c[0] | c[1] << 4 | c[2] << 8 | c[3] << 12);
        }
    } else if (OUT == QGEMM_INT4_B64) {
        // record (n / 32, k0 / 64); piece 32 h + n % 32 holds canonical bytes
        // [16 h, 16 h + 16) of the 64-block
        const int o = k0 & 63, h = o >> 5;
        const size_t rec = (size_t)(n >> 5) * p.nkc + (k0 >> 6);
        if (k0 < p.K)
            *reinterpret_cast<uint16_t *>(p.q + rec * 1024 + (size_t)(32 * h + (n & 31)) * 16 + (o & 31) / 2) =
                (uint16_t)(c[0] | c[1] << 4 | c[2] << 8 | c[3] << 12);
    } else if (OUT == QGEMM_INT8_B0 || OUT == QGEMM_INT8_BLOCK_BASE) {
        if (k0 < p.kp)
            *reinterpret_cast<uint32_t *>(p.q + (size_t)n * p.kp + k0) =
                (uint32_t)c[0] | (uint32_t)c[1] << 8 | (uint32_t)c[2] << 16 | (uint32_t)c[3] << 24;
    } else {                          // W4A8
        // word of k8 = 64 kc + 32 s + 16 h + 8 w: byte i = q[k8 + i] | q[k8 + 4 + i] << 4,
        // the even lane's codes low, the odd lane's high
        const uint32_t b4 = (uint32_t)c[0] | (uint32_t)c[1] << 8 | (uint32_t)c[2] << 16 | (uint32_t)c[3] << 24;
        const uint32_t x = b4 | (__shfl_xor(b4, 1) << 4);
        const int o = k0 & 63, s = o >> 5, h = (o >> 4) & 1, w = (o >> 3) & 1;
        const size_t rec = (size_t)(n >> 5) * p.nkc + (k0 >> 6);
        if ((lane & 1) == 0 && k0 < p.kp)
            *reinterpret_cast<uint32_t *>(p.q + rec * 1024 + (size_t)(32 * h + (n & 31)) * 16 + 8 * s + 4 * w) = x;
    }
}

template <int OUT, int BITS, int G>
__global__ __launch_bounds__(64 * kQWaves) void quantize_vec_kernel(QParams p) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * kQWaves + (threadIdx.x >> 6);
    if (blockIdx.x == 0 && threadIdx.x < 64)
        for (int i = lane; i < p.tail_len; i += 64) p.pairs[p.tail_off + i] = 0.0f;
    if (n >= p.rows) return;                       // whole waves only
    const bool live = n < p.N;
    const float *row = p.W + (size_t)(live ? n : p.N - 1) * p.K;
    constexpr int qmax = (1 << BITS) - 1;
    const int nch = (p.K + 255) / 256;             // chunks per row
    float2 *pp = reinterpret_cast<float2 *>(p.pairs);
    auto load4 = [&](int j) {
        return *reinterpret_cast<const f4_t *>(row + min(256 * j + 4 * lane, p.K - 4));
    };

    if (G > 0) {
        for (int j0 = 0; j0 < nch; j0 += kQUnroll) {
            f4_t v[kQUnroll];
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) v[u] = load4(j0 + u);
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) {
                const int j = j0 + u;
                if (j >= nch) break;               // uniform
                const f4_t x = v[u];
                // blocks of whole groups: K % (4 G) == 0, so a group is all in or all past K
                const bool valid = live && 256 * j + 4 * lane < p.K;
                const bool fin = __builtin_isfinite(x[0]) && __builtin_isfinite(x[1]) &&
                                 __builtin_isfinite(x[2]) && __builtin_isfinite(x[3]);
                const unsigned long long badm = __ballot(valid && !fin);
                const unsigned long long gmask = G == 64 ? ~0ull : ((1ull << G) - 1) << (lane & ~(G - 1));
                const bool bad = (badm & gmask) != 0;
                float lo = group_min<G>(fminf(fminf(x[0], x[1]), fminf(x[2], x[3])));
                float hi = group_max<G>(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
                if (__ballot(lo == 0.0f || hi == 0.0f) != 0) {
                    // equal extremes differ only in the sign of zero: the first zero
                    // in k order (key 2 k + sign) is the one a sequential scan keeps
                    int key = 0x7fffffff;
#pragma unroll
                    for (int e = 3; e >= 0; --e)
                        if (x[e] == 0.0f) key = (8 * lane + 2 * e) | (__builtin_signbitf(x[e]) ? 1 : 0);
                    key = group_imin<G>(key);
                    const float z0 = (key & 1) ? -0.0f : 0.0f;
                    lo = lo == 0.0f ? z0 : lo;
                    hi = hi == 0.0f ? z0 : hi;
                }
                const float2 pr = block_pair(lo, hi, qmax, bad, live);
                const float rcp = 1.0f / pr.y;     // IEEE division, once per block
                int c[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) c[e] = (valid && !bad) ? code_of(x[e], pr, rcp, qmax) : 0;
                store_codes4<OUT, BITS>(p, n, j, lane, c);
                const int k0 = 256 * j + 4 * lane;
                if (OUT == QGEMM_F32) {
                    if ((lane & (G - 1)) == 0 && k0 < p.K) pp[(size_t)n * p.nblk + k0 / (4 * G)] = pr;
                } else if (OUT == QGEMM_INT8_BLOCK_BASE && G > 0 && G <= 8) {
                    // blocked Int8, blocks of 16 or 32: entry (channel, 64-block,
                    // quarter or half)
                    constexpr int H = G > 0 ? 16 / G : 1;          // entries per 64-block
                    if ((lane & (G - 1)) == 0 && k0 < p.K)
                        pp[((size_t)n * p.nkc + (k0 >> 6)) * H + ((k0 & 63) / (4 * G))] = pr;
                } else if (OUT == QGEMM_INT8_BLOCK_BASE) {
                    // blocked Int8: the block's pair in each of its 64-block entries
                    if ((lane & 15) == 0 && k0 < p.K) pp[(size_t)n * p.nkc + (k0 >> 6)] = pr;
                } else if (OUT == QGEMM_INT4_B64 && G > 0 && G <= 8) {
                    // blocks of 16 or 32: records of 1024 or 512 bytes, the
                    // quarter's or half's entry of the channel
                    constexpr int H = G > 0 ? 16 / G : 1;          // entries per 64-block
                    if ((lane & (G - 1)) == 0 && k0 < p.K)
                        pp[int4_pair_entry((size_t)(n >> 5) * p.nkc + (k0 >> 6), n & 31,
                                           (k0 & 63) / (4 * G), H) / 2] = pr;
                } else if (OUT == QGEMM_INT4_B64) {
                    // packed as Int4-Block64: the block's pair in each of its 64-block records
                    if ((lane & 15) == 0 && k0 < p.K) pp[((size_t)(n >> 5) * p.nkc + (k0 >> 6)) * 32 + (n & 31)] = pr;
                } else if (lane == 0) {
                    pp[n] = pr;                    // per-channel formats: the one block is all of K
                }
            }
        }
        return;
    }

    // blocks of whole chunks (or all of K): reduce, then code
    const int cpb = (p.block + 255) / 256;         // chunks per block
    for (int blk = 0; blk < p.nblk; ++blk) {
        const int c0 = blk * cpb, c1 = min(c0 + cpb, nch);
        const int kend = min((blk + 1) * p.block, p.K);
        float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
        bool bad_lane = false;
        for (int j0 = c0; j0 < c1; j0 += kQUnroll) {
            f4_t v[kQUnroll];
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) v[u] = load4(j0 + u);
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) {
                const bool valid = live && 256 * (j0 + u) + 4 * lane < kend;   // K % 4 == 0
                const f4_t x = v[u];
                lo = valid ? fminf(lo, fminf(fminf(x[0], x[1]), fminf(x[2], x[3]))) : lo;
                hi = valid ? fmaxf(hi, fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]))) : hi;
                bad_lane |= valid && !(__builtin_isfinite(x[0]) && __builtin_isfinite(x[1]) &&
                                       __builtin_isfinite(x[2]) && __builtin_isfinite(x[3]));
            }
        }
        const bool bad = __ballot(bad_lane) != 0;
        lo = wave_min(lo);
        hi = wave_max(hi);
        if ((lo == 0.0f || hi == 0.0f) && !bad) {
            // an extreme of 0: the first zero in k order carries the sign a
            // sequential scan keeps (rare, so found by a second scan)
            for (int j = c0; j < c1; ++j) {
                const f4_t x = load4(j);
                int key = 0x7fffffff;
#pragma unroll
                for (int e = 3; e >= 0; --e)
                    if (x[e] == 0.0f && 256 * j + 4 * lane + e < kend)
                        key = (8 * lane + 2 * e) | (__builtin_signbitf(x[e]) ? 1 : 0);
                key = group_imin<64>(key);
                if (key != 0x7fffffff) {
                    const float z0 = (key & 1) ? -0.0f : 0.0f;
                    lo = lo == 0.0f ? z0 : lo;
                    hi = hi == 0.0f ? z0 : hi;
                    break;
                }
            }
        }
        const float2 pr = block_pair(lo, hi, qmax, bad, live);
        const float rcp = 1.0f / pr.y;             // IEEE division, once per block
        for (int j0 = c0; j0 < c1; j0 += kQUnroll) {
            f4_t v[kQUnroll];
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) v[u] = load4(j0 + u);
#pragma unroll
            for (int u = 0; u < kQUnroll; ++u) {
                const int j = j0 + u;
                if (j >= c1) break;                    // uniform
                const bool valid = live && !bad && 256 * j + 4 * lane < kend;
                int c[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) c[e] = valid ? code_of(v[u][e], pr, rcp, qmax) : 0;
                store_codes4<OUT, BITS>(p, n, j, lane, c);
            }
        }
        if (OUT == QGEMM_F32) {
            if (lane == 0) pp[(size_t)n * p.nblk + blk] = pr;
        } else if (OUT == QGEMM_INT8_BLOCK_BASE) {
            // blocked Int8: the pair in every 64-block entry of the block
            const int b0 = blk * (p.block / 64), b1 = min(b0 + p.block / 64, p.nkc);
            for (int b = b0 + lane; b < b1; b += 64) pp[(size_t)n * p.nkc + b] = pr;
        } else if (OUT == QGEMM_INT4_B64) {
            // packed as Int4-Block64: the pair in every 64-block record of the block
            const int b0 = blk * (p.block / 64), b1 = min(b0 + p.block / 64, p.nkc);
            for (int b = b0 + lane; b < b1; b += 64) pp[((size_t)(n >> 5) * p.nkc + b) * 32 + (n & 31)] = pr;
        } else if (lane == 0) {
            pp[n] = pr;
        }
    }
}

template <int OUT, int BITS>
hipError_t launch_vec(const QParams &p, int G, hipStream_t s) {
    const dim3 grid(div_up(p.rows, kQWaves)), block(64 * kQWaves);
    switch (G) {
    case 4: hipLaunchKernelGGL((quantize_vec_kernel<OUT, BITS, 4>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((quantize_vec_kernel<OUT, BITS, 8>), grid, block, 0, s, p); break;
    case 16: hipLaunchKernelGGL((quantize_vec_kernel<OUT, BITS, 16>), grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL((quantize_vec_kernel<OUT, BITS, 32>), grid, block, 0, s, p); break;
    case 64: hipLaunchKernelGGL((quantize_vec_kernel<OUT, BITS, 64>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((quantize_vec_kernel<OUT, BITS, 0>), grid, block, 0, s, p); break;
    }
    return hipGetLastError();
}

template <int OUT, int BITS, bool B64, bool REPEAT>
hipError_t launch(const QParams &p, hipStream_t s) {
    const int grid = div_up(p.rows, kQWaves);
    hipLaunchKernelGGL((quantize_kernel<OUT, BITS, B64, REPEAT>), dim3(grid), dim3(64 * kQWaves), 0,
                       s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int K, int N, qgemm_format f, bool packed, const float *W, void *q,
                           float *pairs, const Geometry &g, hipStream_t s) {
    QParams p{};
    p.W = W;
    p.K = K;
    p.N = N;
    p.rows = packed ? g.Np : N;
    p.nkc = div_up(K, 64);
    p.block = g.block;
    p.nblk = g.nblk;
    p.kp = g.Kp;
    p.q = static_cast<uint8_t *>(q);
    p.pairs = pairs;
    const bool i8blk = kernel_format(f) == QGEMM_INT8_BLOCK_BASE;
    if (packed && (f == QGEMM_INT8_B0 || i8blk)) {
        // the packed pair buffer is padded to its alignment past the last pair
        p.tail_off = f == QGEMM_INT8_B0 ? g.Np * 2 : g.Np * p.nkc * pair_groups(g.block) * 2;
        p.tail_len = (int)(g.s_bytes / sizeof(float)) - p.tail_off;
    }
    if ((K & 3) == 0) {
        // four weights per lane: blocks of 16 to 256 elements (powers of two)
        // as lane groups, or blocks of whole 256-element chunks (and all of K)
        // over two passes
        const int G = (g.block == 16 || g.block == 32 || g.block == 64 || g.block == 128 ||
                       g.block == 256) ? g.block / 4 : 0;
        if (G > 0 || g.block % 256 == 0 || g.block == K) {
            if (!packed) {
                if (f == QGEMM_INT8_B0 || i8blk) return launch_vec<QGEMM_F32, 8>(p, G, s);
                return launch_vec<QGEMM_F32, 4>(p, G, s);
            }
            if (f == QGEMM_INT8_B0) return launch_vec<QGEMM_INT8_B0, 8>(p, G, s);
            if (i8blk) return launch_vec<QGEMM_INT8_BLOCK_BASE, 8>(p, G, s);
            if (f == QGEMM_W4A8) return launch_vec<QGEMM_W4A8, 4>(p, G, s);
            return launch_vec<QGEMM_INT4_B64, 4>(p, G, s);
        }
    }
    if (g.block % 64 != 0 && g.block != K) return hipErrorInvalidValue;   // blocks of 16, 32: lanes of four
    const bool b64 = g.block == 64;
    if (!packed) {
        if (f == QGEMM_INT8_B0 || i8blk) return launch<QGEMM_F32, 8, false, false>(p, s);
        return b64 ? launch<QGEMM_F32, 4, true, false>(p, s)
                   : launch<QGEMM_F32, 4, false, false>(p, s);   // W4A8 and the other Int4 blocks
    }
    if (f == QGEMM_INT8_B0) return launch<QGEMM_INT8_B0, 8, false, false>(p, s);
    if (i8blk) return launch<QGEMM_INT8_BLOCK_BASE, 8, false, true>(p, s);   // blocks of 64 x odd > 1
    if (f == QGEMM_W4A8) return launch<QGEMM_W4A8, 4, false, false>(p, s);
    return b64 ? launch<QGEMM_INT4_B64, 4, true, false>(p, s)
               : launch<QGEMM_INT4_B64, 4, false, true>(p, s);   // Int4-Block0, other blocks
}

}  // namespace qg
