// qgemm_internal.h -- layouts and kernel launchers shared by the library's
// own translation units (never installed, never used by the oracle).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qgemm.h"

namespace qg {

inline size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }
inline int div_up(int x, int m) { return (x + m - 1) / m; }

// Every packed buffer is padded to a multiple of this many bytes.
constexpr size_t kPackAlign = 256;

// ---------------------------------------------------------------------------
// Packed layouts (host packer <-> kernels).
//
// INT4_B64 (and every Int4 format without A8: Int4-Block0 and the other
// block sizes store each pair in every 64-block it covers), nblk = K / 64,
// Np = roundup(N, 32), tiles t of 32 channels:
//   weights: 1 KiB records, record (t, b) at (t * nblk + b) * 1024; its
//            16-byte piece h * 32 + c holds canonical bytes [32 b + 16 h, +16)
//            (the codes of k = 64 b + 32 h .. 64 b + 32 h + 31) of channel
//            32 t + c. Piece order is the lane order of a 32 x 32 MFMA operand
//            (lane = 32 h + c), so one K-block of a 32-channel tile is a single
//            contiguous 1 KiB load; four consecutive channels of one half are
//            a contiguous 64-byte run.
//   pairs:   256-byte records, record (t, b) at (t * nblk + b) * 256 holding
//            {offset, scale} of channels 32 t .. 32 t + 31 for block b.
//            Int4 with blocks that are odd multiples of 32 (a pair per half
//            of each 64-block): 512-byte records, entry (h, c) of record
//            (t, b) at (t * nblk + b) * 512 + (32 h + c) * 8 for K-elements
//            64 b + 32 h .. + 31 of channel 32 t + c. Other multiples of 16
//            (a pair per quarter): 1024-byte records, entry (c, j) at
//            (t * nblk + b) * 1024 + (4 c + j) * 8 for K-elements 64 b + 16 j
//            .. + 15 (int4_pair_entry).
// INT8_B0, Kp = roundup(K, 64), Np = roundup(N, 4):
//   weights: [Np][Kp] bytes (canonical rows, zero padded);
//   pairs:   [Np][2] floats.
// W4A8, Kp = roundup(K, 64), nkc = Kp / 64, Np = roundup(N, 32):
//   weights: 1 KiB records, record (g, kc) at (g * nkc + kc) * 1024 for the
//            channels 32 g .. 32 g + 31 and k in [64 kc, 64 kc + 64); its
//            16-byte piece 32 h + c belongs to channel 32 g + c and holds, for
//            s = 0, 1, the codes of k = 64 kc + 32 s + 16 h + [0, 16) in bytes
//            [8 s, 8 s + 8): byte i of word w (k0 = 64 kc + 32 s + 16 h + 8 w)
//            is q[k0 + i] | q[k0 + 4 + i] << 4, so masking a word with
//            0x0F0F0F0F / shifting it by 4 gives the codes of k0..k0+3 /
//            k0+4..k0+7 in natural order as int8. Piece order is the lane order
//            of a 32 x 32 x 32 int8 MFMA operand (lane = 32 h + c).
//   pairs:   [Np][2] floats.
// F32: weights = B float [K][N] unchanged; no pairs.
// ---------------------------------------------------------------------------
struct Geometry {
    int K = 0, N = 0;
    int Kp = 0;        // K padded to the kernels' step (64) where relevant
    int Np = 0;        // N padded to the channel group
    int nblk = 0;      // pairs per channel
    int block = 0;     // K-elements per pair (0 for float weights)
    size_t w_bytes = 0, s_bytes = 0;
};

qgemm_status geometry(int K, int N, qgemm_format f, Geometry *g);

// Pair entries per 64-element K step in the packed pair layouts of the
// blocked formats: one per 64-block when 64 divides the block size, one per
// 32-element half when 32 does, else one per 16-element quarter (block sizes
// that are multiples of 16). Every entry holds the pair of the block that
// contains its K-elements.
inline int pair_groups(int block) { return block % 64 == 0 ? 1 : block % 32 == 0 ? 2 : 4; }

// Float offset of entry (channel c of the 32-channel tile, sub-block sub) of
// pair record rec in an Int4 packed pair buffer: records of 256 G bytes;
// entry c (G = 1), 32 sub + c (G = 2), or 4 c + sub (G = 4: the two quarters
// of one 32-element half, which one lane decodes, are one 16-byte piece).
__host__ __device__ inline size_t int4_pair_entry(size_t rec, int c, int sub, int G) {
    return rec * 64 * (size_t)G + (size_t)(G == 4 ? 4 * c + sub : 32 * sub + c) * 2;
}

// Int4 with a block size given in the format id (QGEMM_INT4_BLOCK(b)); the
// id carries b, which geometry() checks against K.
constexpr int kMaxBlock = 1 << 24;
inline bool is_int4_blocked(int f) {
    return f > QGEMM_INT4_BLOCK_BASE && f <= QGEMM_INT4_BLOCK_BASE + kMaxBlock;
}
// Int8 with a block size in the format id (QGEMM_INT8_BLOCK(b)).
inline bool is_int8_blocked(int f) {
    return f > QGEMM_INT8_BLOCK_BASE && f <= QGEMM_INT8_BLOCK_BASE + kMaxBlock;
}
// The format the kernels see: every Int4 weight format (Block64, Block0 and
// the other block sizes) is packed as Int4-Block64, its pairs repeated in
// each 64-block of their block; every blocked Int8 format is packed as
// channel rows of codes with a pair per 64-block (per 32-element half for
// blocks of 32), named QGEMM_INT8_BLOCK_BASE here.
inline qgemm_format kernel_format(qgemm_format f) {
    if (f == QGEMM_INT4_B0 || is_int4_blocked(f)) return QGEMM_INT4_B64;
    if (is_int8_blocked(f)) return QGEMM_INT8_BLOCK_BASE;
    return f;
}

constexpr int kGemvMaxM = 8;          // largest M the GEMV kernels take
constexpr int kGemvF16MaxK = 8192;   // fp16-weight GEMV: 16 slices of 8 per lane
constexpr int kGemvI8BlkMaxK = 8192; // blocked Int8 GEMV: eight code slices and pairs per lane
constexpr int kGemvMaxK = 16384;      // A rows staged in LDS: MR * K * 2 bytes
// Largest M * K * N the Int4 GEMV takes for 5..8 rows (above it the tiled
// kernel is faster): with K > 4096 (the whole-tile GEMV, passes over K), and
// with K <= 4096 (the half-tile GEMV).
constexpr long long kGemvInt4MaxMKN = 3LL << 26;
constexpr long long kGemvInt4HalfMaxMKN = 1LL << 29;
// LDS a GEMV workgroup may use (gfx950 gives a workgroup up to 160 KiB).
constexpr size_t kGemvLds = 150 * 1024;

// ---------------------------------------------------------------------------
// Fused epilogue, as the kernels see it: C = act(P + bias + residual), fp32
// throughout, stored as fp32 or fp16 (see qgemm_epilogue in qgemm.h).
// `plain` (no bias, no residual, no activation, fp32 C) keeps each kernel's
// plain store path.
// ---------------------------------------------------------------------------
struct Epilogue {
    const float *bias;
    const void *residual;
    int act;
    int f16;
    bool plain;
};

// ---------------------------------------------------------------------------
// Kernel launchers (defined in the .hip files). They assume validated
// arguments and return hipGetLastError() of their launches. C is float or
// fp16 per the epilogue.
// ---------------------------------------------------------------------------
// pair_g: pair entries per 64-element block, pair_groups(block) (1; 2 per
// 32-element half; 4 per 16-element quarter).
// nsplit > 1: K split over nsplit workgroups per tile, partial tiles in
// `part` ([nsplit][M][N] fp32) added by the fixed-order reduce.
hipError_t launch_gemv_int4b64(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, void *C, const Epilogue &epi, int pair_g,
                               int nsplit, float *part, hipStream_t s);
hipError_t launch_gemv_int8b0(int M, int K, int N, const void *A, const void *Wp,
                              const void *Sp, void *C, const Epilogue &epi, hipStream_t s);
// Blocked Int8: channel rows [Np][K] of codes and pairs [Np][K/64][pair_g],
// K % 64 == 0.
hipError_t launch_gemv_int8blk(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, void *C, const Epilogue &epi, int pair_g,
                               hipStream_t s);
hipError_t launch_gemm_int8blk(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, void *C, const Epilogue &epi, int pair_g,
                               int nsplit, float *part, hipStream_t s);
// Tiled kernels with split-K: nsplit > 1 writes partial tiles to `part`
// ([nsplit][M][N] fp32) and adds them into C with a fixed-order reduce that
// applies the epilogue.
hipError_t launch_gemm_int4b64(int M, int K, int N, const void *A, const void *Wp,
                               const void *Sp, void *C, const Epilogue &epi, int pair_g,
                               int nsplit, float *part, hipStream_t s);
hipError_t launch_splitk_reduce_f32(const float *part, int nsplit, int M, int N, void *C,
                                    const Epilogue &epi, hipStream_t s);
hipError_t launch_gemm_int8b0(int M, int K, int N, const void *A, const void *Wp,
                              const void *Sp, void *C, const Epilogue &epi, int nsplit,
                              float *part, hipStream_t s);
// fp16 weights as channel rows [Np][Kp] (Kp = roundup(K, 64)).
hipError_t launch_gemv_f16(int M, int K, int N, const void *A, const void *Wp, void *C,
                           const Epilogue &epi, hipStream_t s);
hipError_t launch_gemm_f16(int M, int K, int N, const void *A, const void *Wp, void *C,
                           const Epilogue &epi, int nsplit, float *part, hipStream_t s);
hipError_t launch_gemm_f32(int M, int K, int N, const float *A, const float *B, void *C,
                           const Epilogue &epi, int nsplit, float *part, hipStream_t s);
// W4A8: qa [M][Kq] int8 (Kq = roundup(K, 128)), sa [M] float, S [M] int32
// live in the workspace.
hipError_t launch_w4a8_actquant(int M, int K, int Kq, const void *A, int8_t *qa,
                                float *sa, int32_t *S, hipStream_t s);
// nsplit > 1: int32 partial tiles in `part` ([nsplit][M][N]), added exactly
// by a reduce kernel that applies the rescale and epilogue.
hipError_t launch_w4a8_gemm(int M, int K, int N, int Kq, const int8_t *qa, const float *sa,
                            const int32_t *S, const void *Wp, const void *Sp,
                            void *C, const Epilogue &epi, int32_t *D_debug, int nsplit,
                            int32_t *part, hipStream_t s);
// M <= 8 (the GEMV limit), K <= kGemvMaxK: quantises A itself (one launch);
// qa [M][Kq], sa and S are written only with D_debug.
// nsplit > 1 (shapes with few 32-channel tiles): the standalone quantiser,
// int32 partial tiles in `part` and the W4A8 reduce.
hipError_t launch_w4a8_gemv(int M, int K, int N, int Kq, const void *A, int8_t *qa, float *sa,
                            int32_t *S, const void *Wp, const void *Sp, void *C,
                            const Epilogue &epi, int32_t *D_debug, int nsplit, int32_t *part,
                            hipStream_t s);

// Device quantiser (float W [N][K] -> codes and pairs): canonical layout, or
// with `packed` the format's packed layout including its zero padding.
hipError_t launch_quantize(int K, int N, qgemm_format f, bool packed, const float *W, void *q,
                           float *pairs, const Geometry &g, hipStream_t s);

// W4A8 scratch: qa [M][qa_stride] int8 (qa_stride = roundup(K, 128), zero
// past K), sa [M] float, S [M] int32.
struct W4A8Workspace {
    int qa_stride;
    size_t qa_off, sa_off, S_off, bytes;
};
W4A8Workspace w4a8_workspace(int M, int K);

// Split-K for the tiled (prefill) kernels. When a shape has too few output
// tiles to occupy the chip, nsplit workgroups share each tile, each over a
// contiguous range of K, and write partial tiles (fp32; int32 for W4A8) that a
// reduce kernel adds in a fixed order, so results stay bit-reproducible. The
// plan is a pure function of the shape (sized for a 256-CU part), so the
// workspace size never depends on the device.
// Output tile of the Int4-Block64 prefill GEMM (rows x columns), shared by
// the kernel and the split-K planner: 128 x 64 once M reaches 128 (each
// dequantised weight serves 128 rows) or 128 x 128 where that takes fewer
// rounds of the CUs, else 64 x 128, or the skinny kernel's 32- or 64-row
// tiles of 32 channels (below).
struct Int4Tile {
    int bm, bn;
};
// CUs a launch should cover (split-K plans, the skinny kernel's choice).
constexpr int kSplitTargetCUs = 256;
// Up to kSkinnyMaxM rows, while the 32-channel tiles are fewer than the CUs,
// the skinny kernel runs: a 32-channel tile of all rows (32 or 64, M padded)
// per workgroup. (With more tiles than CUs it re-reads A once per tile and
// takes a second round of workgroups; the 64 x 128 tiles do better there.)
constexpr int kSkinnyMaxM = 64;
inline Int4Tile int4_tile(int M, int N) {
    if (M >= 128) {
        // 128 x 128 tiles (each A element serves twice the columns per byte
        // brought into the CU) take 1.73x the time of a 128 x 64 tile per
        // round of 256 CUs (1024 x 4096 x 4096: 41.6 us in one round against
        // 48.0 in two); they run where their rounds cost less, which needs
        // more than 128 of them (so they never split K)
        const int tm = div_up(M, 128);
        const long long r128 = ((long long)tm * div_up(N, 128) + kSplitTargetCUs - 1) / kSplitTargetCUs;
        const long long r64 = ((long long)tm * div_up(N, 64) + kSplitTargetCUs - 1) / kSplitTargetCUs;
        return 7 * r128 < 4 * r64 ? Int4Tile{128, 128} : Int4Tile{128, 64};
    }
    return M > kSkinnyMaxM || (N + 31) / 32 >= kSplitTargetCUs ? Int4Tile{64, 128}
         : M > 32 ? Int4Tile{64, 32} : Int4Tile{32, 32};
}
// Output tile of the channel-row (Int8-Block0, fp16-weight) prefill GEMM.
constexpr int kRowsTileM = 128, kRowsTileN = 64;
// Output tile of the W4A8 prefill GEMM and its K stage (qa bytes per row).
constexpr int kW4A8TileM = 128, kW4A8TileN = 256, kW4A8StageK = 128;
// Columns of a W4A8 tile for a shape: 128 while 128-column tiles fit one
// round of the CUs (twice the workgroups for shapes with few tiles, so less
// K splitting), else 256. Measured on the benchmark page's shapes at M = 32
// to 1024 (us, 256 -> 128 columns): 512 x 2560 x 4096 24.5 -> 20.3, 1024 x
// 4096 x 2560 36.3 -> 29.0, 128 x 2560 x 9728 23.5 -> 19.8; with more tiles
// than that 256 columns stay faster (1024 x 3072 x 8192: 36.6 against 43.6).
inline int w4a8_tile_n(int M, int N) {
    return (long long)div_up(M, kW4A8TileM) * div_up(N, kW4A8TileN / 2) <= kSplitTargetCUs ? kW4A8TileN / 2
                                                                                          : kW4A8TileN;
}
// Output tiles of the fp32 GEMM: 16 x 64 for M <= 16, else 64 x 64; K in
// chunks of 64.
constexpr int kF32TileN = 64, kF32TileMSmall = 16, kF32TileM = 64, kF32ChunkK = 64;
// K-groups (256 threads each) inside an fp32 workgroup when the shape has
// fewer output tiles than CUs; 1 otherwise.
constexpr int kF32KGroups = 2;
int f32_kgroups(int M, int N);
constexpr int kMaxSplit = 8;
int splitk_plan(qgemm_format f, int M, int K, int N);      // 1 = no split
// The same for the Int4 GEMV (M up to the GEMV limit): shapes with few
// 32-channel tiles split K over the workgroups of a tile.
int gemv_split_plan(qgemm_format f, int M, int K, int N);

// Full scratch layout of one call: the W4A8 part (if any) first, then the
// split-K partials [S][M][N] (4 bytes each), sized for the larger of the
// tiled GEMM's plan (nsplit) and the GEMV's (gemv_nsplit), so that the size
// is a function of the shape alone whichever kernel a call takes.
struct RunWorkspace {
    W4A8Workspace w4a8;       // bytes == 0 unless W4A8
    int nsplit, gemv_nsplit;
    size_t part_off, part_bytes, bytes;
};
RunWorkspace run_workspace(qgemm_format f, int M, int K, int N);

}  // namespace qg
