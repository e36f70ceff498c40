// w4a8.hip -- the W4A8 path: per-row dynamic int8 quantisation of the fp16
// activations, then an exact s8 x s8 -> s32 product (on the int8 matrix
// cores for prefill, with v_dot4 in a GEMV for decode-sized M) and an fp32
// rescale epilogue.
//
// MNN GemmSpeed benchmark page, section "Test cases and registration", mode 3
// (Int4-Block0 W4A8): per-channel 4-bit weights are unpacked to int8, the
// activations are dynamically quantised to int8 and an S8 x S8 -> S32 GEMM
// runs. The page fixes no formula; the reading implemented here:
//   sa[m] = max_k |A[m][k]| / 127 (fp32, correctly rounded division),
//   qa[m][k] = clamp(rint(A[m][k] / sa[m]), -127, 127) (ties to even),
//   a zero row gives sa = 0 and qa = 0, S[m] = sum_k qa[m][k];
//   D[m][n] = sum_k qa[m][k] * q[n][k] with q the zero-extended code in [0, 15];
//   C[m][n] = sa[m] * (scale[n] * D[m][n] + offset[n] * S[m]),
// which is sum_k (sa qa) (offset + scale q) regrouped so the inner loop is
// pure integer arithmetic.
#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

// ---------------------------------------------------------------------------
// Activation quantisation: one 256-thread workgroup per row. The row of qa
// has Kq = roundup(K, 128) bytes, zero past K, so the GEMM can stage 128-wide
// K slices without bounds cases.
// ---------------------------------------------------------------------------
// clamp(rint(a / s), -127, 127) with a / s the correctly rounded fp32
// quotient, formed from rs = RN(1 / s) with one residual correction:
// y = RN(a * rs), q = y + rs * (a - y * s) (two fused multiply-adds). For
// every fp16 a with |a| <= amax and s = RN(amax / 127) this q is bit-identical
// to the IEEE division (checked exhaustively on the CPU by the test suite).
__device__ __forceinline__ int quant1(float a, float s, float rs) {
    const float y = a * rs;
    const float e = fmaf(-y, s, a);
    const float q = fmaf(e, rs, y);
    return (int)fminf(fmaxf(rintf(q), -127.0f), 127.0f);   // ties to even
}

__device__ __forceinline__ float block_max(float v, float *red4) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
}

__device__ __forceinline__ void block_sum_store(int v, int *red4, int32_t *dst) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) *dst = red4[0] + red4[1] + red4[2] + red4[3];
}

// K % 8 == 0 and Kq <= 2048 * NPT: one 256-thread workgroup per row (four
// waves per row, sixteen per CU at M = 1024, so a SIMD starts quantising as
// soon as the chunks of one of its waves have arrived). Thread t requests
// the row's 8-element chunks t, t + 256, ... at once (clamped, so every load
// is unconditional); the maximum and the sum meet in LDS once each.
template <int NPT>
__global__ __launch_bounds__(256) void w4a8_actquant_row_kernel(int K, int Kq,
                                                                const _Float16 *__restrict__ A,
                                                                int8_t *__restrict__ qa,
                                                                float *__restrict__ sa,
                                                                int32_t *__restrict__ S) {
    __shared__ float red_f[4];
    __shared__ int red_i[4];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const _Float16 *row = A + (size_t)m * K;
    int8_t *qrow = qa + (size_t)m * Kq;
    const int nch = K >> 3, nchq = Kq >> 3;
    h8_t v[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i)
        v[i] = *reinterpret_cast<const h8_t *>(row + 8 * min(tid + 256 * i, nch - 1));
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        float c = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) c = fmaxf(c, fabsf((float)v[i][e]));
        mx = tid + 256 * i < nch ? fmaxf(mx, c) : mx;
    }
    const float amax = block_max(mx, red_f);
    const float s = amax / 127.0f;           // IEEE division, one rounding
    const float rs = 1.0f / s;               // IEEE division, one rounding
    int sum = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int c = tid + 256 * i;
        if (c >= nchq) continue;
        unsigned lo = 0u, hi = 0u;
        if (c < nch && amax != 0.0f) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int qi = quant1((float)v[i][e], s, rs);
                sum += qi;
                const unsigned byte = (unsigned)(qi & 0xff);
                if (e < 4) lo |= byte << (8 * e);
                else hi |= byte << (8 * (e - 4));
            }
        }
        *reinterpret_cast<u2_t *>(qrow + 8 * c) = u2_t{lo, hi};
    }
    if (tid == 0) sa[m] = amax != 0.0f ? s : 0.0f;
    block_sum_store(sum, red_i, S + m);
}

// Any even K: two passes over the row, element by element.
__global__ __launch_bounds__(256) void w4a8_actquant_kernel(int K, int Kq,
                                                            const _Float16 *__restrict__ A,
                                                            int8_t *__restrict__ qa,
                                                            float *__restrict__ sa,
                                                            int32_t *__restrict__ S) {
    __shared__ float red_f[4];
    __shared__ int red_i[4];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const _Float16 *row = A + (size_t)m * K;
    int8_t *qrow = qa + (size_t)m * Kq;
    float amax = 0.0f;
    for (int k = tid; k < K; k += 256) amax = fmaxf(amax, fabsf((float)row[k]));
    amax = block_max(amax, red_f);
    const float s = amax / 127.0f;
    const float rs = 1.0f / s;
    int sum = 0;
    for (int k = tid; k < Kq; k += 256) {
        int qi = 0;
        if (k < K && amax != 0.0f) qi = quant1((float)row[k], s, rs);
        sum += qi;
        qrow[k] = (int8_t)qi;
    }
    if (tid == 0) sa[m] = amax != 0.0f ? s : 0.0f;
    block_sum_store(sum, red_i, S + m);
}

hipError_t launch_w4a8_actquant(int M, int K, int Kq, const void *A, int8_t *qa, float *sa,
                                int32_t *S, hipStream_t s) {
    const _Float16 *a = static_cast<const _Float16 *>(A);
    const dim3 rows(M);
    if ((K & 7) == 0 && Kq <= 2048 * 1)
        hipLaunchKernelGGL(w4a8_actquant_row_kernel<1>, rows, dim3(256), 0, s, K, Kq, a, qa, sa, S);
    else if ((K & 7) == 0 && Kq <= 2048 * 2)
        hipLaunchKernelGGL(w4a8_actquant_row_kernel<2>, rows, dim3(256), 0, s, K, Kq, a, qa, sa, S);
    else if ((K & 7) == 0 && Kq <= 2048 * 4)
        hipLaunchKernelGGL(w4a8_actquant_row_kernel<4>, rows, dim3(256), 0, s, K, Kq, a, qa, sa, S);
    else if ((K & 7) == 0 && Kq <= 2048 * 8)
        hipLaunchKernelGGL(w4a8_actquant_row_kernel<8>, rows, dim3(256), 0, s, K, Kq, a, qa, sa, S);
    else
        hipLaunchKernelGGL(w4a8_actquant_kernel, rows, dim3(256), 0, s, K, Kq, a, qa, sa, S);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// int8 GEMM. A 512-thread workgroup owns a 128 x 256 tile of C; wave w owns
// the 128 x 32 column block 32 w and runs every K step with
// v_mfma_i32_32x32x32_i8 (4 accumulator tiles). Shapes whose 128 x 128
// tiles fit one round of the CUs take those instead (two rows of four
// waves, each wave 64 x 32): twice the workgroups, so fewer K slices. Each wave loads only its own
// weight record, so no weight byte enters a CU twice; two waves per SIMD
// overlap one wave's loads and LDS reads with the other's matrix work. (The
// wave grid is a parameter: a 2 x 4 grid of 64 x 64 wave tiles halves the
// LDS reads of A but loads every weight record twice, and measured slower.)
//  - qa is staged in LDS 128 K-columns (one 128-byte run per row) at a time,
//    four stages deep, loaded three stages ahead through a register ring;
//    one barrier per stage;
//  - a K-block of a 32-channel weight record is one contiguous 1 KiB load
//    already in operand lane order, loaded three stages ahead; the int4
//    codes become int8 operands with one mask (and one shift) per word;
//  - every global load is unconditional with clamped indices (rows past M,
//    channels past N, stages past the end read valid data that is never
//    stored or, for padded stages, meets an all-zero A tile), which keeps
//    the compiler's in-order count of outstanding loads exact;
//  - the epilogue applies C = sa * (scale * D + offset * S) with the row
//    scales and sums staged in LDS; for a plain fp32 C each wave passes its
//    results through LDS in 64 x 32 blocks so that every lane stores
//    16-byte pieces of rows: storing the accumulator layout directly (one
//    float per lane down a column) made the store phase a third of the
//    kernel's time at 1024 x 3072 x 8192.
// Lane (r, h) = (lane % 32, lane / 32) holds K-elements 32 s + 16 h .. +15 of
// each 64-wide block in step s for its A row and B column alike.
// ---------------------------------------------------------------------------
namespace {
constexpr int WBM = kW4A8TileM, WSK = kW4A8StageK;
constexpr int WNW = 8;                    // waves
// Wave grid: WGM_ rows x (8 / WGM_) columns of (128 / WGM_) x 32 wave tiles,
// so the tile is 128 x 256 (one row of waves) or 128 x 128 (two).
template <int WGM_>
struct W4Grid {
    static constexpr int WGM = WGM_, WGN = WNW / WGM_;
    static constexpr int WBN = 32 * WGN;                 // tile columns
    static constexpr int WRF = WBM / (32 * WGM);         // 32-row fragments per wave
    static constexpr int WCF = 1;                        // 32-column fragments per wave
    static_assert(WRF % 2 == 0 && WRF * WCF <= 4 && WBN == kW4A8TileN / WGM_, "wave tile of 64k x 32 rows");
};
constexpr int WAROW = WSK + 16;           // bytes per LDS row of an A stage (144)
constexpr int WRING = 4;                  // stages: LDS A tiles = A and B register ring slots
constexpr size_t WAS_BYTES = (size_t)WBM * WAROW;
}

__device__ __forceinline__ i4_t unpack_codes(unsigned w0, unsigned w1) {
    const unsigned m = 0x0F0F0F0Fu;
    return i4_t{(int)(w0 & m), (int)((w0 >> 4) & m), (int)(w1 & m), (int)((w1 >> 4) & m)};
}

template <bool DEBUG_D, int WGM_>
__global__ __launch_bounds__(64 * WNW) void w4a8_gemm_kernel(
    int M, int N, int Kq, int nkc, int tiles_n, const int8_t *__restrict__ qa,
    const float *__restrict__ sa, const int32_t *__restrict__ S, const uint8_t *__restrict__ Wp,
    const f2_t *__restrict__ Sp, void *__restrict__ C, Epilogue epi, int32_t *__restrict__ D) {
    using G = W4Grid<WGM_>;
    constexpr int WGM = G::WGM, WGN = G::WGN, WBN = G::WBN, WRF = G::WRF, WCF = G::WCF;
    __shared__ __align__(16) int8_t As[WRING * WAS_BYTES];
    __shared__ float sa_s[WBM];
    __shared__ int S_s[WBM];

    // ---- tile of this workgroup: plain row-major order. The hardware deals
    //      workgroups to the eight XCDs round-robin, so with a multiple of 8
    //      column tiles each XCD takes an interleaved eighth of the columns
    //      of every row tile; this measured faster than giving each XCD a
    //      contiguous band of column tiles (37.8 against 36.9 us at
    //      1024 x 3072 x 8192, one box) ----
    const int L = blockIdx.x;
    const int tm = L / tiles_n, tn = L % tiles_n;
    const int m0 = tm * WBM, n0 = tn * WBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;   // wave tile rows 32 WRF wm.., columns 32 WCF wn..
    const int r = lane & 31, h = lane >> 5;
    // split-K: slice blockIdx.y of gridDim.y takes stages [st0, st0 + nst) of
    // the Kq / WSK (the plan keeps gridDim.y <= Kq / WSK, so nst >= 1)
    const int nst_all = Kq / WSK;
    const int st0 = slice_begin(blockIdx.y, nst_all, gridDim.y);
    const int nst = slice_begin(blockIdx.y + 1, nst_all, gridDim.y) - st0;
    const int nsteps = (nst + WRING - 1) / WRING * WRING;
    const int ntiles_b = (N + 31) / 32;

    if (tid < WBM) {
        const int gm = min(m0 + tid, M - 1);
        sa_s[tid] = sa[gm];
        S_s[tid] = S[gm];
    }

    // A loader role: 2 x (8 lanes x 16 bytes per row), rows tid / 8 and 64 + tid / 8
    size_t a_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = tid + 512 * i;
        a_off[i] = (size_t)min(m0 + (idx >> 3), M - 1) * Kq + (size_t)(idx & 7) * 16;
    }
    auto load_a = [&](u4_t (&dst)[2], int st) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dst[i] = *reinterpret_cast<const u4_t *>(qa + a_off[i] + (size_t)(st0 + st) * WSK);
    };
    auto a_tile = [&](int slot) { return As + (size_t)slot * WAS_BYTES; };
    auto store_a = [&](int8_t *T, const u4_t (&src)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 512 * i;
            *reinterpret_cast<u4_t *>(T + (idx >> 3) * WAROW + (idx & 7) * 16) = src[i];
        }
    };
    // the same, with every word ANDed with a uniform mask (all ones, or zero
    // for a stage past the end): no branch, so no merge point for the
    // compiler's count of outstanding loads
    auto store_a_masked = [&](int8_t *T, const u4_t (&src)[2], unsigned mask) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 512 * i;
            *reinterpret_cast<u4_t *>(T + (idx >> 3) * WAROW + (idx & 7) * 16) = src[i] & mask;
        }
    };
    // B: the records of the wave's two 32-channel tiles, two K-blocks per stage
    size_t b_rec0[WCF];
#pragma unroll
    for (int cf = 0; cf < WCF; ++cf)
        b_rec0[cf] = (size_t)min(n0 / 32 + WCF * wn + cf, ntiles_b - 1) * nkc;
    auto load_b = [&](u4_t (&dst)[2][WCF], int st) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int cf = 0; cf < WCF; ++cf) {
                const size_t rec = b_rec0[cf] + min(2 * (st0 + st) + kk, nkc - 1);
                dst[kk][cf] = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(Wp + rec * 1024) + lane);
            }
    };

    i16_t acc[WRF][WCF];
#pragma unroll
    for (int a = 0; a < WRF; ++a)
#pragma unroll
        for (int b = 0; b < WCF; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[a][b][j] = 0;

    u4_t an[WRING][2];
    u4_t bq[WRING][2][WCF];

    // prologue: stage 0 in LDS tile 0, stages 1 .. WRING of A and 0 .. WRING - 1
    // of B in flight (clamped past the end: never used)
    load_a(an[0], 0);
#pragma unroll
    for (int d = 0; d < WRING; ++d) load_b(bq[d], min(d, nst - 1));
    store_a(a_tile(0), an[0]);
#pragma unroll
    for (int d = 1; d <= WRING; ++d) load_a(an[d % WRING], min(d, nst - 1));
    // Let the prologue's loads land before the loop: the loop header merges
    // this path with the back edge, and the compiler may have issued these
    // loads in any order, so without this wait it would count the slot the
    // loop reads first as the newest load and drain everything every stage.
    // The scheduling barriers keep the loads above the wait (the wait alone
    // does not stop the scheduler from sinking loads below it).
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);

    // a do-while (nsteps >= WRING always): with no guard branch in front of
    // the loop, the compiler cannot sink the prologue's loads below the wait
    // into a preheader of their own
    int base = 0;
    do {
#pragma unroll
        for (int u = 0; u < WRING; ++u) {
            const int i = base + u;
            // stage i + 1's A into its tile (last read in stage i - 3, before
            // the previous barrier), then its ring slot takes stage i + 1 + WRING
            store_a_masked(a_tile((u + 1) % WRING), an[(u + 1) % WRING], i + 1 < nst ? ~0u : 0u);
            load_a(an[(u + 1) % WRING], min(i + 1 + WRING, nst - 1));
            __syncthreads();
            const int8_t *T = a_tile(u) + (32 * WRF * wm + r) * WAROW + 16 * h;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    i4_t af[WRF], bf[WCF];
#pragma unroll
                    for (int rf = 0; rf < WRF; ++rf)
                        af[rf] = *reinterpret_cast<const i4_t *>(T + 32 * rf * WAROW + 64 * kk + 32 * s);
#pragma unroll
                    for (int cf = 0; cf < WCF; ++cf)
                        bf[cf] = unpack_codes(bq[u][kk][cf][2 * s], bq[u][kk][cf][2 * s + 1]);
#pragma unroll
                    for (int rf = 0; rf < WRF; ++rf)
#pragma unroll
                        for (int cf = 0; cf < WCF; ++cf)
                            acc[rf][cf] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[rf], bf[cf],
                                                                                acc[rf][cf], 0, 0, 0);
                }
            // B slot u is free: refill it with stage i + WRING
            load_b(bq[u], min(i + WRING, nst - 1));
        }
        base += WRING;
    } while (base < nsteps);

    // ---- epilogue: C = sa * (scale * D + offset * S), or this slice's D ----
    // Plain fp32 C of a whole 64 x 32 wave block: through LDS (over the A
    // tiles, a private 64 x 36-float region per wave) so that each lane
    // stores 16-byte pieces of rows instead of single floats down a column.
    const bool staged = gridDim.y == 1 && !DEBUG_D && epi.plain && (N & 3) == 0 &&
                        (reinterpret_cast<uintptr_t>(C) & 15) == 0;
    if (staged) {
        __syncthreads();   // every wave is done with the A tiles
        float *stg = reinterpret_cast<float *>(As) + wave * (64 * 36);
#pragma unroll
        for (int cf = 0; cf < WCF; ++cf)
#pragma unroll
            for (int rh = 0; rh < WRF / 2; ++rh) {
                const int c0 = n0 + 32 * WCF * wn + 32 * cf;
                const int rb = 32 * WRF * wm + 64 * rh;     // first tile row of this 64-row block
                if (m0 + rb + 64 > M || c0 + 32 > N) {
                    // a ragged block: element stores (uniform branch per wave)
                    const int col = c0 + r;
                    if (col >= N) continue;
                    const f2_t pr = Sp[col];
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const int rl = rb + 32 * q + 8 * (j >> 2) + 4 * h + (j & 3);
                            if (m0 + rl >= M) continue;
                            static_cast<float *>(C)[(size_t)(m0 + rl) * N + col] =
                                sa_s[rl] * fmaf(pr.y, (float)acc[2 * rh + q][cf][j], pr.x * (float)S_s[rl]);
                        }
                    continue;
                }
                const f2_t pr = Sp[c0 + r];
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int rw = 32 * q + 8 * (j >> 2) + 4 * h + (j & 3);
                        const int rl = rb + rw;
                        stg[rw * 36 + r] = sa_s[rl] * fmaf(pr.y, (float)acc[2 * rh + q][cf][j], pr.x * (float)S_s[rl]);
                    }
                // the wave's own LDS writes precede its reads (one wave's LDS
                // operations complete in order); its next block's writes
                // follow these reads likewise
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int rw = 8 * i + (lane >> 3), c4 = lane & 7;
                    const f4_t v = *reinterpret_cast<const f4_t *>(stg + rw * 36 + 4 * c4);
                    __builtin_nontemporal_store(v, reinterpret_cast<f4_t *>(static_cast<float *>(C) + (size_t)(m0 + rb + rw) * N + c0 + 4 * c4));
                }
            }
        return;
    }
#pragma unroll
    for (int cf = 0; cf < WCF; ++cf) {
        const int col = n0 + 32 * WCF * wn + 32 * cf + r;
        if (col >= N) continue;
        if (gridDim.y > 1) {       // exact int32 partial tile; the reduce finishes
            int32_t *dp = D + (size_t)blockIdx.y * M * N;
#pragma unroll
            for (int rf = 0; rf < WRF; ++rf)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int row = m0 + 32 * WRF * wm + 32 * rf + 8 * (j >> 2) + 4 * h + (j & 3);
                    if (row < M) dp[(size_t)row * N + col] = acc[rf][cf][j];
                }
            continue;
        }
        const f2_t pr = Sp[col];
#pragma unroll
        for (int rf = 0; rf < WRF; ++rf) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int rl = 32 * WRF * wm + 32 * rf + 8 * (j >> 2) + 4 * h + (j & 3);
                const int row = m0 + rl;
                if (row >= M) continue;
                const int d = acc[rf][cf][j];
                if (DEBUG_D) D[(size_t)row * N + col] = d;
                const float out = sa_s[rl] * fmaf(pr.y, (float)d, pr.x * (float)S_s[rl]);
                if (epi.plain) static_cast<float *>(C)[(size_t)row * N + col] = out;
                else epi_put(epi, C, row, col, N, out);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// W4A8 GEMV (M up to the GEMV limit, the decode shape): one 1024-thread
// workgroup per 32-channel tile and pass of MR rows, reading the same 1 KiB
// records as the GEMM.
//  1. Each thread requests its share of the MR activation rows, then its
//     wave's weight records (kc = w, w + 16, ...; whole records, clamped into
//     the tile). Loads complete in order, so waiting for the activations
//     leaves the records in flight.
//  2. FUSED (one or two rows): the fp16 rows are quantised into LDS (16 / MR
//     waves per row) with the same arithmetic as the standalone quantiser
//     (row maximum, sa = amax / 127, quant1), so the codes, sa and S equal its
//     results bit for bit. Otherwise the standalone quantiser has run and its
//     codes are copied into LDS (every workgroup requantising many rows would
//     cost more than the separate launch).
//  3. Lane (c, h) = (lane % 32, lane / 32) holds 32 codes of channel c per
//     record (k = 64 kc + 32 s + 16 h + [0, 16) for s = 0, 1), unpacks them to
//     int8 with one mask and one shift-mask per word, and meets the codes of
//     each row (LDS broadcast reads) in v_dot4: exact int32 sums.
//  4. The two halves h, then the 16 waves' partial sums, are added in a fixed
//     order; the epilogue is C = sa (scale D + offset S) as in the GEMM.
// FUSED: every workgroup quantises its rows itself (a few KiB, read from L2),
// so the call is one launch and qa never leaves the chip; with the debug
// outputs requested, the workgroups of tile 0 also store qa, sa and S.
// ---------------------------------------------------------------------------
constexpr int WG_WAVES = 16;
// LDS for MR quantised rows of Kp bytes (the wave partial sums reuse it).
constexpr size_t kW4A8GemvLds = kGemvLds;

// SPLIT: the tile's records [KC0, KC1) of slice blockIdx.z (gridDim.z
// slices), and an int32 partial tile into D ([gridDim.z][M][N]) instead of C;
// only with the standalone quantiser's codes.
template <int MR, int NREC, bool FUSED, bool DEBUG_D, bool SPLIT>
__global__ __launch_bounds__(64 * WG_WAVES) void w4a8_gemv_kernel(
    int M, int K, int N, int Kq, int nkc, const _Float16 *__restrict__ A, int8_t *__restrict__ qa,
    float *__restrict__ sa, int32_t *__restrict__ S, const uint8_t *__restrict__ Wp,
    const f2_t *__restrict__ Sp, void *__restrict__ C, Epilogue epi, int32_t *__restrict__ D) {
    constexpr int WPR = WG_WAVES / MR;                       // waves per activation row
    constexpr int TPR = 64 * WPR;                            // threads per activation row
    // per thread: fp16 pairs of its row (FUSED), or 16-byte pieces of the codes
    constexpr int AP = FUSED ? (NREC * MR / 2 > 1 ? NREC * MR / 2 : 1)
                             : (NREC * MR / 16 > 1 ? NREC * MR / 16 : 1);
    extern __shared__ __align__(16) uint8_t lds[];           // qa [MR][Kp], then partial sums
    __shared__ float amax_w[WG_WAVES];
    __shared__ int sum_w[WG_WAVES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int c = lane & 31, h = lane >> 5;
    const int t = blockIdx.x;
    const int m0 = blockIdx.y * MR;
    const int Kp = nkc * 64, npair = K >> 1;
    static_assert(!(SPLIT && (FUSED || DEBUG_D)), "a split GEMV uses the standalone quantiser");
    const int KC0 = SPLIT ? slice_begin(blockIdx.z, nkc, gridDim.z) : 0;
    const int KC1 = SPLIT ? slice_begin(blockIdx.z + 1, nkc, gridDim.z) : nkc;

    // 1. this thread's activations (rows past M repeat row M - 1, never
    //    stored), then this wave's records
    const int ar = wave / WPR, at = tid - ar * TPR;
    unsigned ap[FUSED ? AP : 1];
    u4_t qp[FUSED ? 1 : AP];
    if (FUSED) {
        const unsigned *arow = reinterpret_cast<const unsigned *>(A + (size_t)min(m0 + ar, M - 1) * K);
#pragma unroll
        for (int j = 0; j < AP; ++j) ap[j] = arow[min(at + TPR * j, npair - 1)];
    } else {
        // piece i of the MR code rows' records [KC0, KC1): row i / per_row,
        // bytes 64 KC0 + 16 (i % per_row)
        const int per_row = 4 * (KC1 - KC0);
#pragma unroll
        for (int j = 0; j < AP; ++j) {
            const int i = min(tid + 64 * WG_WAVES * j, MR * per_row - 1);
            const int r = i / per_row;
            qp[j] = *reinterpret_cast<const u4_t *>(qa + (size_t)min(m0 + r, M - 1) * Kq + 64 * KC0 +
                                                     16 * (i - r * per_row));
        }
    }
    u4_t rec[NREC];
#pragma unroll
    for (int i = 0; i < NREC; ++i) {
        const int kc = min(KC0 + wave + WG_WAVES * i, KC1 - 1);
        rec[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u4_t *>(Wp + ((size_t)t * nkc + kc) * 1024) + lane);
    }

    // 2. the codes of the MR rows into LDS
    if (!FUSED) {
        const int per_row = 4 * (KC1 - KC0);
#pragma unroll
        for (int j = 0; j < AP; ++j) {
            const int i = tid + 64 * WG_WAVES * j;
            const int r = i / per_row;
            if (i < MR * per_row)
                *reinterpret_cast<u4_t *>(lds + r * Kp + 64 * KC0 + 16 * (i - r * per_row)) = qp[j];
        }
        __syncthreads();
    } else {
        // quantise: maximum, then codes (zero past K) and sums
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < AP; ++j) {
            const _Float16 *hv = reinterpret_cast<const _Float16 *>(&ap[j]);
            const float m2 = fmaxf(fabsf((float)hv[0]), fabsf((float)hv[1]));
            amax = at + TPR * j < npair ? fmaxf(amax, m2) : amax;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        if (lane == 0) amax_w[wave] = amax;
        __syncthreads();
        float rmax = 0.0f;
#pragma unroll
        for (int w = 0; w < WPR; ++w) rmax = fmaxf(rmax, amax_w[ar * WPR + w]);
        const float s = rmax / 127.0f;           // IEEE division, one rounding
        const float rs = 1.0f / s;               // IEEE division, one rounding
        int sum = 0;
#pragma unroll
        for (int j = 0; j < AP; ++j) {
            const int i = at + TPR * j;
            const _Float16 *hv = reinterpret_cast<const _Float16 *>(&ap[j]);
            int q0 = 0, q1 = 0;
            if (i < npair && rmax != 0.0f) {
                q0 = quant1((float)hv[0], s, rs);
                q1 = quant1((float)hv[1], s, rs);
            }
            sum += q0 + q1;
            if (2 * i < Kp)
                *reinterpret_cast<unsigned short *>(lds + ar * Kp + 2 * i) =
                    (unsigned short)((q0 & 0xff) | ((q1 & 0xff) << 8));
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
        if (lane == 0) sum_w[wave] = sum;
        __syncthreads();
        if (DEBUG_D && t == 0) {
            // the standalone quantiser's outputs: qa rows of Kq bytes, sa, S
            for (int i = tid; i < MR * Kq; i += 64 * WG_WAVES) {
                const int r = i / Kq, k = i - r * Kq;
                if (m0 + r < M) qa[(size_t)(m0 + r) * Kq + k] = k < Kp ? (int8_t)lds[r * Kp + k] : 0;
            }
            if (tid < MR && m0 + tid < M) {
                float mx = 0.0f;
                int S_r = 0;
                for (int w = 0; w < WPR; ++w) {
                    mx = fmaxf(mx, amax_w[tid * WPR + w]);
                    S_r += sum_w[tid * WPR + w];
                }
                sa[m0 + tid] = mx != 0.0f ? mx / 127.0f : 0.0f;
                S[m0 + tid] = S_r;
            }
        }
    }

    // 3. exact int32 dot products against the codes in LDS
    int acc[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) acc[r] = 0;
#pragma unroll
    for (int i = 0; i < NREC; ++i) {
        const int kc = KC0 + wave + WG_WAVES * i;
        const int kk = 64 * min(kc, KC1 - 1) + 16 * h;
        const i4_t b0 = unpack_codes(rec[i][0], rec[i][1]);   // k = 64 kc + 16 h + [0, 16)
        const i4_t b1 = unpack_codes(rec[i][2], rec[i][3]);   // k = 64 kc + 32 + 16 h + [0, 16)
        if (kc < KC1) {        // uniform; no global load inside
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const i4_t a0 = *reinterpret_cast<const i4_t *>(lds + r * Kp + kk);
                const i4_t a1 = *reinterpret_cast<const i4_t *>(lds + r * Kp + kk + 32);
                int v = acc[r];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v = __builtin_amdgcn_sdot4(a0[e], b0[e], v, false);
                    v = __builtin_amdgcn_sdot4(a1[e], b1[e], v, false);
                }
                acc[r] = v;
            }
        }
    }

    // 4. halves, then waves, in a fixed order; then the epilogue
    __syncthreads();                                   // the codes are no longer read
    int *red = reinterpret_cast<int *>(lds);           // [WG_WAVES][MR][32]
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        const int v = acc[r] + __shfl_xor(acc[r], 32);
        if (h == 0) red[(wave * MR + r) * 32 + c] = v;
    }
    __syncthreads();
    if (tid >= MR * 32) return;
    const int r = tid >> 5, n = 32 * t + (tid & 31), m = m0 + r;
    if (n >= N || m >= M) return;
    int d = 0;
#pragma unroll
    for (int w = 0; w < WG_WAVES; ++w) d += red[(w * MR + r) * 32 + (tid & 31)];
    if (SPLIT) {
        D[((size_t)blockIdx.z * M + m) * N + n] = d;      // exact partial; the reduce finishes
        return;
    }
    float sa_r;
    int S_r = 0;
    if (FUSED) {
        float mx = 0.0f;
#pragma unroll
        for (int w = 0; w < WPR; ++w) {
            mx = fmaxf(mx, amax_w[r * WPR + w]);
            S_r += sum_w[r * WPR + w];
        }
        sa_r = mx != 0.0f ? mx / 127.0f : 0.0f;
    } else {
        sa_r = sa[m];
        S_r = S[m];
    }
    if (DEBUG_D) D[(size_t)m * N + n] = d;
    const f2_t pr = Sp[n];
    const float out = sa_r * fmaf(pr.y, (float)d, pr.x * (float)S_r);
    if (epi.plain) static_cast<float *>(C)[(size_t)m * N + n] = out;
    else epi_put(epi, C, m, n, N, out);
}

// Fusing the quantisation pays for one or two rows; more rows use the
// standalone quantiser's codes.
template <int MR, int NREC>
constexpr bool w4a8_gemv_fused() { return MR == 1 || (MR == 2 && NREC <= 8); }

template <int MR, int NREC>
static void w4a8_gemv_launch(dim3 grid, size_t lds, hipStream_t s, int M, int K, int N, int Kq,
                             int nkc, const void *A, int8_t *qa, float *sa, int32_t *S,
                             const void *Wp, const void *Sp, void *C, const Epilogue &epi,
                             int32_t *D) {
    constexpr bool F = w4a8_gemv_fused<MR, NREC>();
    const _Float16 *a = static_cast<const _Float16 *>(A);
    const uint8_t *w = static_cast<const uint8_t *>(Wp);
    const f2_t *p = static_cast<const f2_t *>(Sp);
    if (grid.z > 1)            // D is the partial-tile buffer
        hipLaunchKernelGGL((w4a8_gemv_kernel<MR, NREC, false, false, true>), grid, dim3(64 * WG_WAVES),
                           lds, s, M, K, N, Kq, nkc, a, qa, sa, S, w, p, C, epi, D);
    else if (D)
        hipLaunchKernelGGL((w4a8_gemv_kernel<MR, NREC, F, true, false>), grid, dim3(64 * WG_WAVES), lds, s,
                           M, K, N, Kq, nkc, a, qa, sa, S, w, p, C, epi, D);
    else
        hipLaunchKernelGGL((w4a8_gemv_kernel<MR, NREC, F, false, false>), grid, dim3(64 * WG_WAVES), lds, s,
                           M, K, N, Kq, nkc, a, qa, sa, S, w, p, C, epi, D);
}

template <int MR>
static hipError_t w4a8_gemv_mr(int M, int K, int N, int Kq, const void *A, int8_t *qa, float *sa,
                               int32_t *S, const void *Wp, const void *Sp, void *C,
                               const Epilogue &epi, int32_t *D, int nsplit, int32_t *part,
                               hipStream_t s) {
    const int nkc = (int)round_up(K, 64) / 64;
    const dim3 grid(div_up(N, 32), div_up(M, MR), nsplit);
    const size_t codes = (size_t)MR * nkc * 64, sums = (size_t)WG_WAVES * MR * 32 * sizeof(int);
    const size_t lds = codes > sums ? codes : sums;
    const int nrec = div_up(div_up(nkc, nsplit), WG_WAVES);   // K <= 16384: at most 16
    const bool fused = nsplit == 1 && (nrec <= 1   ? w4a8_gemv_fused<MR, 1>()
                                       : nrec <= 2 ? w4a8_gemv_fused<MR, 2>()
                                       : nrec <= 4 ? w4a8_gemv_fused<MR, 4>()
                                       : nrec <= 8 ? w4a8_gemv_fused<MR, 8>()
                                                   : w4a8_gemv_fused<MR, 16>());
    if (nsplit > 1) D = part;  // the kernel writes partial tiles; the reduce writes C (and D)
    if (!fused) {
        const hipError_t e = launch_w4a8_actquant(M, K, Kq, A, qa, sa, S, s);
        if (e != hipSuccess) return e;
    }
    if (nrec <= 1) w4a8_gemv_launch<MR, 1>(grid, lds, s, M, K, N, Kq, nkc, A, qa, sa, S, Wp, Sp, C, epi, D);
    else if (nrec <= 2) w4a8_gemv_launch<MR, 2>(grid, lds, s, M, K, N, Kq, nkc, A, qa, sa, S, Wp, Sp, C, epi, D);
    else if (nrec <= 4) w4a8_gemv_launch<MR, 4>(grid, lds, s, M, K, N, Kq, nkc, A, qa, sa, S, Wp, Sp, C, epi, D);
    else if (nrec <= 8) w4a8_gemv_launch<MR, 8>(grid, lds, s, M, K, N, Kq, nkc, A, qa, sa, S, Wp, Sp, C, epi, D);
    else w4a8_gemv_launch<MR, 16>(grid, lds, s, M, K, N, Kq, nkc, A, qa, sa, S, Wp, Sp, C, epi, D);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void w4a8_splitk_reduce_kernel(
    const int32_t *__restrict__ part, int nsplit, int M, int N, const float *__restrict__ sa,
    const int32_t *__restrict__ S, const f2_t *__restrict__ Sp, void *__restrict__ C, Epilogue epi,
    int32_t *__restrict__ D);
static hipError_t launch_w4a8_gemv_rows(int M, int K, int N, int Kq, const void *A, int8_t *qa,
                                        float *sa, int32_t *S, const void *Wp, const void *Sp,
                                        void *C, const Epilogue &epi, int32_t *D_debug, int nsplit,
                                        int32_t *part, hipStream_t s);

hipError_t launch_w4a8_gemv(int M, int K, int N, int Kq, const void *A, int8_t *qa, float *sa,
                            int32_t *S, const void *Wp, const void *Sp, void *C,
                            const Epilogue &epi, int32_t *D_debug, int nsplit, int32_t *part,
                            hipStream_t s) {
    if (nsplit > 1) {
        hipError_t e = launch_w4a8_gemv_rows(M, K, N, Kq, A, qa, sa, S, Wp, Sp, C, epi, D_debug,
                                             nsplit, part, s);
        if (e != hipSuccess) return e;
        const size_t mn = (size_t)M * N;
        hipLaunchKernelGGL(w4a8_splitk_reduce_kernel, dim3((unsigned)((mn + 255) / 256)), dim3(256),
                           0, s, part, nsplit, M, N, sa, S, static_cast<const f2_t *>(Sp), C, epi,
                           D_debug);
        return hipGetLastError();
    }
    return launch_w4a8_gemv_rows(M, K, N, Kq, A, qa, sa, S, Wp, Sp, C, epi, D_debug, 1, nullptr, s);
}

static hipError_t launch_w4a8_gemv_rows(int M, int K, int N, int Kq, const void *A, int8_t *qa,
                                        float *sa, int32_t *S, const void *Wp, const void *Sp,
                                        void *C, const Epilogue &epi, int32_t *D_debug, int nsplit,
                                        int32_t *part, hipStream_t s) {
    // rows per pass: up to M (at most 8), as long as their codes fit the LDS
    const size_t Kp = round_up(K, 64);
    int mr = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
    while (mr > 1 && (size_t)mr * Kp > (size_t)kW4A8GemvLds) mr >>= 1;
    switch (mr) {
    case 1: return w4a8_gemv_mr<1>(M, K, N, Kq, A, qa, sa, S, Wp, Sp, C, epi, D_debug, nsplit, part, s);
    case 2: return w4a8_gemv_mr<2>(M, K, N, Kq, A, qa, sa, S, Wp, Sp, C, epi, D_debug, nsplit, part, s);
    case 4: return w4a8_gemv_mr<4>(M, K, N, Kq, A, qa, sa, S, Wp, Sp, C, epi, D_debug, nsplit, part, s);
    default: return w4a8_gemv_mr<8>(M, K, N, Kq, A, qa, sa, S, Wp, Sp, C, epi, D_debug, nsplit, part, s);
    }
}

// Split-K reduction: D = sum of the int32 partial tiles (exact in any order),
// then the same rescale and epilogue as the unsplit kernel, so the result is
// bit-identical to it.
__global__ __launch_bounds__(256) void w4a8_splitk_reduce_kernel(
    const int32_t *__restrict__ part, int nsplit, int M, int N, const float *__restrict__ sa,
    const int32_t *__restrict__ S, const f2_t *__restrict__ Sp, void *__restrict__ C, Epilogue epi,
    int32_t *__restrict__ D) {
    const size_t mn = (size_t)M * N;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= mn) return;
    int d = part[i];
    for (int z = 1; z < nsplit; ++z) d += part[(size_t)z * mn + i];
    const int m = (int)(i / (size_t)N), n = (int)(i - (size_t)m * N);
    if (D) D[i] = d;
    const f2_t pr = Sp[n];
    const float out = sa[m] * fmaf(pr.y, (float)d, pr.x * (float)S[m]);
    if (epi.plain) static_cast<float *>(C)[i] = out;
    else epi_put(epi, C, m, n, N, out);
}

template <int WGM_>
static hipError_t launch_w4a8_gemm_grid(int M, int K, int N, int Kq, const int8_t *qa, const float *sa,
                                        const int32_t *S, const void *Wp, const void *Sp, void *C,
                                        const Epilogue &epi, int32_t *D_debug, int nsplit, int32_t *part,
                                        hipStream_t s) {
    const int nkc = (int)round_up(K, 64) / 64;
    const int tiles_m = div_up(M, WBM), tiles_n = div_up(N, W4Grid<WGM_>::WBN);
    if (nsplit > 1) {
        hipLaunchKernelGGL((w4a8_gemm_kernel<false, WGM_>), dim3(tiles_m * tiles_n, nsplit), dim3(64 * WNW),
                           0, s, M, N, Kq, nkc, tiles_n, qa, sa, S,
                           static_cast<const uint8_t *>(Wp), static_cast<const f2_t *>(Sp), C, epi,
                           part);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const size_t mn = (size_t)M * N;
        hipLaunchKernelGGL(w4a8_splitk_reduce_kernel, dim3((unsigned)((mn + 255) / 256)), dim3(256),
                           0, s, part, nsplit, M, N, sa, S, static_cast<const f2_t *>(Sp), C, epi,
                           D_debug);
        return hipGetLastError();
    }
    dim3 grid(tiles_m * tiles_n);
    if (D_debug)
        hipLaunchKernelGGL((w4a8_gemm_kernel<true, WGM_>), grid, dim3(64 * WNW), 0, s, M, N, Kq, nkc,
                           tiles_n, qa, sa, S, static_cast<const uint8_t *>(Wp),
                           static_cast<const f2_t *>(Sp), C, epi, D_debug);
    else
        hipLaunchKernelGGL((w4a8_gemm_kernel<false, WGM_>), grid, dim3(64 * WNW), 0, s, M, N, Kq, nkc,
                           tiles_n, qa, sa, S, static_cast<const uint8_t *>(Wp),
                           static_cast<const f2_t *>(Sp), C, epi, D_debug);
    return hipGetLastError();
}

hipError_t launch_w4a8_gemm(int M, int K, int N, int Kq, const int8_t *qa, const float *sa,
                            const int32_t *S, const void *Wp, const void *Sp, void *C,
                            const Epilogue &epi, int32_t *D_debug, int nsplit, int32_t *part,
                            hipStream_t s) {
    return w4a8_tile_n(M, N) == kW4A8TileN
               ? launch_w4a8_gemm_grid<1>(M, K, N, Kq, qa, sa, S, Wp, Sp, C, epi, D_debug, nsplit, part, s)
               : launch_w4a8_gemm_grid<2>(M, K, N, Kq, qa, sa, S, Wp, Sp, C, epi, D_debug, nsplit, part, s);
}

}  // namespace qg
