// host_pack.cpp -- host side of libqgemm that never touches the GPU:
// geometry of the formats, the quantiser, the packer and its inverse.
//
// Formats follow the MNN GemmSpeed benchmark page, section "Why Conv1x1 is
// used to measure GEMM" (Int8-Block0: 8-bit codes, blockSize = K; Int4-Block64:
// 4-bit codes, blockSize 64, K % 64 == 0 or the shape is skipped; pairs laid
// out as oc x blockNum groups of [offset, scale]) and section "Test cases and
// registration" (W4A8: per-channel 4-bit weights).
#include <cmath>
#include <cstring>
#include <vector>

#include "qgemm_internal.h"

namespace qg {

static bool valid_format(int f) {
    return f == QGEMM_F32 || f == QGEMM_INT4_B64 || f == QGEMM_INT8_B0 || f == QGEMM_W4A8 ||
           f == QGEMM_F16 || f == QGEMM_INT4_B0 || is_int4_blocked(f) || is_int8_blocked(f);
}

// Shapes are capped so that every element count and byte offset the kernels
// form stays far inside 64-bit and every per-dimension index inside int32.
constexpr int kMaxDim = 1 << 24;
// W4A8 keeps D = sum_k qa * q in int32: |D| <= K * 127 * 15 must stay < 2^31.
constexpr long long kW4A8MaxK = ((1LL << 31) - 1) / (127 * 15);

// The quantised formats carry [offset, scale] pairs; float weights do not.
static bool has_pairs(qgemm_format f) { return f != QGEMM_F32 && f != QGEMM_F16; }

qgemm_status geometry(int K, int N, qgemm_format f, Geometry *g) {
    if (!valid_format(f)) return QGEMM_ERR_FORMAT;
    if (K < 0 || N < 0 || K > kMaxDim || N > kMaxDim) return QGEMM_ERR_SHAPE;
    Geometry r;
    r.K = K;
    r.N = N;
    if (is_int4_blocked(f)) {
        // Int4 with one pair per b K-elements (b a multiple of 16), packed as
        // Int4-Block64 with each pair repeated in the 64-blocks it covers;
        // pair records hold pair_groups(b) entries per channel and 64-block
        // (256, 512 or 1024 bytes)
        const int b = f - QGEMM_INT4_BLOCK_BASE;
        if (b % 16 != 0) return QGEMM_ERR_FORMAT;
        if (K == 0 || K % b != 0 || K % 64 != 0) return QGEMM_ERR_SHAPE;
        r.Kp = K; r.Np = (int)round_up(N, 32); r.nblk = K / b; r.block = b;
        r.w_bytes = round_up((size_t)(r.Np / 32) * (K / 64) * 1024, kPackAlign);
        r.s_bytes = round_up((size_t)(r.Np / 32) * (K / 64) * 256 * pair_groups(b), kPackAlign);
        *g = r;
        return QGEMM_OK;
    }
    if (is_int8_blocked(f)) {
        // Int8 with one pair per b K-elements (b a multiple of 16): channel
        // rows of codes [Np][K] (as Int8-Block0) and the pairs channel-major
        // with pair_groups(b) entries per 64-block (one per 64-block, 32-half
        // or 16-quarter), repeated over the entries a block covers
        const int b = f - QGEMM_INT8_BLOCK_BASE;
        if (b % 16 != 0) return QGEMM_ERR_FORMAT;
        if (K == 0 || K % b != 0 || K % 64 != 0) return QGEMM_ERR_SHAPE;
        r.Kp = K; r.Np = (int)round_up(N, 4); r.nblk = K / b; r.block = b;
        r.w_bytes = round_up((size_t)r.Np * K, kPackAlign);
        r.s_bytes = round_up((size_t)r.Np * (K / 64) * pair_groups(b) * 2 * sizeof(float),
                             kPackAlign);
        *g = r;
        return QGEMM_OK;
    }
    switch (f) {
    case QGEMM_F32:
        r.Kp = K; r.Np = N; r.nblk = 0;
        r.w_bytes = round_up((size_t)K * N * sizeof(float), kPackAlign);
        r.s_bytes = 0;
        break;
    case QGEMM_F16:
        // channel rows [Np][Kp] of fp16 weights, zero padded
        if (K == 0) return QGEMM_ERR_SHAPE;
        r.Kp = (int)round_up(K, 64); r.Np = (int)round_up(N, 4); r.nblk = 0;
        r.w_bytes = round_up((size_t)r.Np * r.Kp * 2, kPackAlign);
        r.s_bytes = 0;
        break;
    case QGEMM_INT4_B64:
    case QGEMM_INT4_B0:
        // Int4-Block0 is packed as Int4-Block64 with the channel's one pair
        // repeated in every 64-block: the same weights, the same kernels
        if (K == 0 || K % 64 != 0) return QGEMM_ERR_SHAPE;
        r.Kp = K; r.Np = (int)round_up(N, 32); r.nblk = f == QGEMM_INT4_B0 ? 1 : K / 64;
        r.block = f == QGEMM_INT4_B0 ? K : 64;
        r.w_bytes = round_up((size_t)(r.Np / 32) * (K / 64) * 1024, kPackAlign);
        r.s_bytes = round_up((size_t)(r.Np / 32) * (K / 64) * 256, kPackAlign);
        break;
    case QGEMM_INT8_B0:
        if (K == 0) return QGEMM_ERR_SHAPE;
        r.Kp = (int)round_up(K, 64); r.Np = (int)round_up(N, 4); r.nblk = 1; r.block = K;
        r.w_bytes = round_up((size_t)r.Np * r.Kp, kPackAlign);
        r.s_bytes = round_up((size_t)r.Np * 2 * sizeof(float), kPackAlign);
        break;
    case QGEMM_W4A8:
        if (K == 0 || K % 2 != 0 || K > kW4A8MaxK) return QGEMM_ERR_SHAPE;
        r.Kp = (int)round_up(K, 64); r.Np = (int)round_up(N, 32); r.nblk = 1; r.block = K;
        r.w_bytes = round_up((size_t)r.Np * (r.Kp / 2), kPackAlign);
        r.s_bytes = round_up((size_t)r.Np * 2 * sizeof(float), kPackAlign);
        break;
    }
    *g = r;
    return QGEMM_OK;
}

W4A8Workspace w4a8_workspace(int M, int K) {
    W4A8Workspace w;
    w.qa_stride = (int)round_up((size_t)K, 128);
    w.qa_off = 0;
    w.sa_off = round_up((size_t)M * w.qa_stride, kPackAlign);
    w.S_off = w.sa_off + round_up((size_t)M * sizeof(float), kPackAlign);
    w.bytes = w.S_off + round_up((size_t)M * sizeof(int32_t), kPackAlign);
    return w;
}

int f32_kgroups(int M, int N) {
    const long long tiles = (long long)div_up(M, M <= kF32TileMSmall ? kF32TileMSmall : kF32TileM) *
                            div_up(N, kF32TileN);
    return tiles < kSplitTargetCUs ? kF32KGroups : 1;
}

int splitk_plan(qgemm_format f, int M, int K, int N) {
    if (M <= 0 || N <= 0 || K <= 0) return 1;
    f = kernel_format(f);
    long long tiles = 0;
    int kunits = 0;                  // K granules: the most slices a split may have
    switch (f) {
    case QGEMM_INT4_B64:
    case QGEMM_INT4_B0:
        if (int4_tile(M, N).bn == 32) {
            // the skinny kernel: one workgroup per 32-channel tile and slice
            // streams its weights; it splits as far as the tiles and slices
            // still fit the CUs in one round (its LDS holds one workgroup per
            // CU), eight waves with one or more 64-blocks each
            const long long nt = div_up(N, 32);
            long long sp = kSplitTargetCUs / nt;
            if (sp > kMaxSplit) sp = kMaxSplit;
            if (sp > K / 64 / 8) sp = K / 64 / 8;
            return sp < 2 ? 1 : (int)sp;
        }
        tiles = (long long)div_up(M, int4_tile(M, N).bm) * div_up(N, int4_tile(M, N).bn);
        kunits = K / 64 / 8;         // four waves, two or more 64-blocks each
        break;
    case QGEMM_F32: {
        // the K-groups of a workgroup share its CU, so only the split spreads
        // a tile over more CUs; a split costs a second launch, so each group
        // of each slice keeps four or more chunks
        const int kg = f32_kgroups(M, N);
        tiles = (long long)div_up(M, M <= kF32TileMSmall ? kF32TileMSmall : kF32TileM) *
                div_up(N, kF32TileN);
        kunits = div_up(K, kF32ChunkK) / (kg * 4);
        break;
    }
    case QGEMM_INT8_B0:
    case QGEMM_F16:
    case QGEMM_INT8_BLOCK_BASE:
        // four waves, two or more 64-blocks each
        tiles = (long long)div_up(M, kRowsTileM) * div_up(N, kRowsTileN);
        kunits = (int)(round_up((size_t)K, 64) / 64) / 8;
        break;
    case QGEMM_W4A8:
        // each slice keeps four or more K stages (one turn of the load ring)
        tiles = (long long)div_up(M, kW4A8TileM) * div_up(N, w4a8_tile_n(M, N));
        kunits = (int)(round_up((size_t)K, kW4A8StageK) / kW4A8StageK) / 4;
        {
            // The slices' int32 partial tiles and their reduce cost time in
            // proportion to (slices + 1) x M x N, which outweighs the shorter
            // K of each slice where M x N is large and K short (512 x 2560 x
            // 4096: 24.5 us unsplit, 31.6 in four slices). Estimated time,
            // fitted to the benchmark page's shapes at M = 128 and 512 (us):
            // 4 per 1000 K-elements of a slice, plus for a split 4 and 0.2
            // per MB of (slices + 1) x M x N x 4 bytes.
            tiles = (long long)div_up(M, kW4A8TileM) * div_up(N, w4a8_tile_n(M, N));
            if (tiles >= kSplitTargetCUs / 2) return 1;
            long long cap = kSplitTargetCUs / tiles;
            if (cap > kMaxSplit) cap = kMaxSplit;
            if (cap > kunits) cap = kunits;
            const double mn_mb = (double)M * N * 4 / 1e6;
            int best = 1;
            double best_t = 0.004 * K;
            for (int sp = 2; sp <= cap; ++sp) {
                const double t = 0.004 * K / sp + 4.0 + 0.2 * (sp + 1) * mn_mb;
                if (t < best_t) { best = sp; best_t = t; }
            }
            return best;
        }
    default:
        return 1;
    }
    if (tiles >= kSplitTargetCUs / 2) return 1;
    long long sp = kSplitTargetCUs / tiles;
    if (sp > kMaxSplit) sp = kMaxSplit;
    if (sp > kunits) sp = kunits;
    return sp < 2 ? 1 : (int)sp;
}

int gemv_split_plan(qgemm_format f, int M, int K, int N) {
    f = kernel_format(f);
    if ((f != QGEMM_INT4_B64 && f != QGEMM_W4A8) || M <= 0 || M > kGemvMaxM || N <= 0 || K <= 0)
        return 1;
    K = (int)round_up((size_t)K, 64);   // W4A8 records cover K rounded up to 64
    // A split W4A8 GEMV reads the standalone quantiser's codes: not worth it
    // where the unsplit one quantises inside the kernel (one row, or two rows
    // up to K = 8192); measured at M = 1, K = 9728, N = 2560: 9.6 us fused,
    // 13.2 us as quantiser + three slices + reduce.
    if (f == QGEMM_W4A8 && (M == 1 || (M == 2 && K <= 8192))) return 1;
    // one pass over the rows (M <= 8); each slice keeps three or more
    // 64-blocks per wave (16 waves per tile), since a split costs a second
    // launch (measured: two per wave lose at K = 4096)
    const long long tiles = div_up(N, 32);
    if (tiles >= kSplitTargetCUs / 2) return 1;
    long long sp = kSplitTargetCUs / tiles;
    if (sp > kMaxSplit) sp = kMaxSplit;
    if (sp > K / 64 / 48) sp = K / 64 / 48;
    // the unsplit Int4 GEMV runs half tiles (twice the workgroups), which a
    // two-way split does not beat (measured: 16384 x 3072 11.1 us unsplit
    // against 11.6 split in two, 6144 x 2560 5.7 against 7.0); three or more
    // slices still win (9728 x 2560: 7.6 us in three, 9.4 in two)
    if (f == QGEMM_INT4_B64 && sp < 3) return 1;
    return sp < 2 ? 1 : (int)sp;
}

RunWorkspace run_workspace(qgemm_format f, int M, int K, int N) {
    RunWorkspace r;
    r.w4a8 = f == QGEMM_W4A8 ? w4a8_workspace(M, K) : W4A8Workspace{0, 0, 0, 0, 0};
    r.nsplit = splitk_plan(f, M, K, N);
    r.gemv_nsplit = gemv_split_plan(f, M, K, N);
    const int most = r.nsplit > r.gemv_nsplit ? r.nsplit : r.gemv_nsplit;
    r.part_off = round_up(r.w4a8.bytes, kPackAlign);
    r.part_bytes = most > 1 ? round_up((size_t)most * M * N * 4, kPackAlign) : 0;
    r.bytes = r.part_off + r.part_bytes;
    return r;
}

static size_t canonical_q_bytes(const Geometry &g, qgemm_format f) {
    switch (kernel_format(f)) {
    case QGEMM_F32: return (size_t)g.K * g.N * sizeof(float);
    case QGEMM_F16: return (size_t)g.K * g.N * 2;
    case QGEMM_INT8_B0:
    case QGEMM_INT8_BLOCK_BASE: return (size_t)g.N * g.K;
    default: return (size_t)g.N * (g.K / 2);
    }
}

static size_t canonical_pair_floats(const Geometry &g, qgemm_format f) {
    return has_pairs(f) ? (size_t)g.N * g.nblk * 2 : 0;
}

// Canonical code of channel n at k (INT4 / W4A8: low nibble first).
static inline uint8_t nib(const uint8_t *row, int k) {
    uint8_t b = row[k >> 1];
    return (k & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
}

}  // namespace qg

using namespace qg;

extern "C" {

const char *qgemm_status_string(int s) {
    switch (s) {
    case QGEMM_OK: return "QGEMM_OK";
    case QGEMM_ERR_NULL: return "QGEMM_ERR_NULL: a required pointer is NULL";
    case QGEMM_ERR_SHAPE: return "QGEMM_ERR_SHAPE: invalid shape for this format";
    case QGEMM_ERR_FORMAT: return "QGEMM_ERR_FORMAT: unknown or unsupported format";
    case QGEMM_ERR_ALIGN: return "QGEMM_ERR_ALIGN: device pointer not 16-byte aligned";
    case QGEMM_ERR_NOMEM: return "QGEMM_ERR_NOMEM: scratch allocation failed";
    case QGEMM_ERR_DEVICE: return "QGEMM_ERR_DEVICE: no usable gfx950 HIP device";
    case QGEMM_ERR_LAUNCH: return "QGEMM_ERR_LAUNCH: kernel launch failed";
    case QGEMM_ERR_SIZE: return "QGEMM_ERR_SIZE: buffer smaller than required";
    case QGEMM_ERR_VALUE: return "QGEMM_ERR_VALUE: non-finite weight";
    default: return "QGEMM_ERR_UNKNOWN";
    }
}

int qgemm_abi_version(void) { return QGEMM_ABI_VERSION; }

qgemm_status qgemm_canonical_size(int K, int N, qgemm_format f, size_t *q_bytes,
                                  size_t *pair_floats) {
    Geometry g;
    qgemm_status st = geometry(K, N, f, &g);
    if (st != QGEMM_OK) return st;
    if (!q_bytes || !pair_floats) return QGEMM_ERR_NULL;
    *q_bytes = canonical_q_bytes(g, f);
    *pair_floats = canonical_pair_floats(g, f);
    return QGEMM_OK;
}

qgemm_status qgemm_packed_size(int K, int N, qgemm_format f, size_t *w_bytes,
                               size_t *s_bytes) {
    Geometry g;
    qgemm_status st = geometry(K, N, f, &g);
    if (st != QGEMM_OK) return st;
    if (!w_bytes || !s_bytes) return QGEMM_ERR_NULL;
    *w_bytes = g.w_bytes;
    *s_bytes = g.s_bytes;
    return QGEMM_OK;
}

qgemm_status qgemm_workspace_size(int M, int K, int N, qgemm_format f, size_t *bytes) {
    Geometry g;
    qgemm_status st = geometry(K, N, f, &g);
    if (st != QGEMM_OK) return st;
    if (M < 0 || M > (1 << 24)) return QGEMM_ERR_SHAPE;
    if (!bytes) return QGEMM_ERR_NULL;
    *bytes = (M > 0 && N > 0) ? run_workspace(f, M, K, N).bytes : 0;
    return QGEMM_OK;
}

qgemm_status qgemm_quantize_weights(int K, int N, qgemm_format f, const float *W,
                                    void *q_out, size_t q_bytes, float *pairs,
                                    size_t pair_floats) {
    if (!has_pairs(f)) return QGEMM_ERR_FORMAT;   // float weights are not quantised
    Geometry g;
    qgemm_status st = geometry(K, N, f, &g);
    if (st != QGEMM_OK) return st;
    if (N == 0) return QGEMM_OK;
    if (!W || !q_out || !pairs) return QGEMM_ERR_NULL;
    if (q_bytes < canonical_q_bytes(g, f) || pair_floats < canonical_pair_floats(g, f))
        return QGEMM_ERR_SIZE;
    const size_t total = (size_t)N * K;
    for (size_t i = 0; i < total; ++i)
        if (!std::isfinite(W[i])) return QGEMM_ERR_VALUE;

    const int bits = (f == QGEMM_INT8_B0 || is_int8_blocked(f)) ? 8 : 4;
    const int block = g.block;
    const int nblk = K / block;
    const int qmax = (1 << bits) - 1;
    uint8_t *q = static_cast<uint8_t *>(q_out);
    if (bits == 4) std::memset(q, 0, (size_t)N * (K / 2));

    for (int n = 0; n < N; ++n) {
        const float *wrow = W + (size_t)n * K;
        for (int b = 0; b < nblk; ++b) {
            const float *wb = wrow + (size_t)b * block;
            double lo = wb[0], hi = wb[0];
            for (int i = 1; i < block; ++i) {
                double v = wb[i];
                lo = v < lo ? v : lo;
                hi = v > hi ? v : hi;
            }
            const float offset = (float)lo;
            const float scale = (float)((hi - lo) / (double)qmax);
            pairs[((size_t)n * nblk + b) * 2 + 0] = offset;
            pairs[((size_t)n * nblk + b) * 2 + 1] = scale;
            const double off_d = offset, scale_d = scale;
            for (int i = 0; i < block; ++i) {
                int code = 0;
                if (scale != 0.0f) {
                    double r = std::nearbyint(((double)wb[i] - off_d) / scale_d);
                    r = r < 0.0 ? 0.0 : (r > qmax ? (double)qmax : r);
                    code = (int)r;
                }
                const int k = b * block + i;
                if (bits == 8)
                    q[(size_t)n * K + k] = (uint8_t)code;
                else
                    q[(size_t)n * (K / 2) + (k >> 1)] |= (uint8_t)(code << ((k & 1) * 4));
            }
        }
    }
    return QGEMM_OK;
}

qgemm_status qgemm_pack_weights(int K, int N, qgemm_format f, const void *w_canonical,
                                const float *pairs_canonical, void *w_packed,
                                size_t w_bytes, void *s_packed, size_t s_bytes) {
    Geometry g;
    qgemm_status st = geometry(K, N, f, &g);
    if (st != QGEMM_OK) return st;
    if (!w_packed || (g.s_bytes && !s_packed)) return QGEMM_ERR_NULL;
    if (w_bytes < g.w_bytes || s_bytes < g.s_bytes) return QGEMM_ERR_SIZE;
    if ((size_t)N * K > 0 && !w_canonical) return QGEMM_ERR_NULL;
    if (has_pairs(f) && N > 0 && !pairs_canonical) return QGEMM_ERR_NULL;

    uint8_t *wp = static_cast<uint8_t *>(w_packed);
    uint8_t *sp = static_cast<uint8_t *>(s_packed);
    float *spf = reinterpret_cast<float *>(s_packed);
    std::memset(wp, 0, g.w_bytes);
    if (g.s_bytes) std::memset(sp, 0, g.s_bytes);
    const uint8_t *wc = static_cast<const uint8_t *>(w_canonical);

    switch (kernel_format(f)) {
    case QGEMM_F32:
        if ((size_t)K * N) std::memcpy(wp, wc, (size_t)K * N * sizeof(float));
        break;
    case QGEMM_F16: {
        // [K][N] -> channel rows [Np][Kp]
        const uint16_t *src = reinterpret_cast<const uint16_t *>(wc);
        uint16_t *dst = reinterpret_cast<uint16_t *>(wp);
        for (int k = 0; k < K; ++k)
            for (int n = 0; n < N; ++n) dst[(size_t)n * g.Kp + k] = src[(size_t)k * N + n];
        break;
    }
    case QGEMM_INT4_B64:
    case QGEMM_INT4_B0: {
        const int nblk = K / 64;
        const size_t row = (size_t)K / 2;
        const int G = pair_groups(g.block);
        for (int n = 0; n < N; ++n) {
            const int t = n >> 5, c = n & 31;
            for (int b = 0; b < nblk; ++b) {
                const size_t rec = (size_t)t * nblk + b;
                for (int half = 0; half < 2; ++half)
                    std::memcpy(wp + rec * 1024 + (size_t)(32 * half + c) * 16,
                                wc + (size_t)n * row + (size_t)b * 32 + half * 16, 16);
                // entry sub of the record: the pair of the block holding
                // K-elements 64 b + sub * 64 / G (Block0: the channel's one pair)
                for (int sub = 0; sub < G; ++sub) {
                    const size_t pi = ((size_t)n * g.nblk + ((size_t)b * 64 + sub * (64 / G)) / g.block) * 2;
                    const size_t so = int4_pair_entry(rec, c, sub, G);
                    spf[so + 0] = pairs_canonical[pi + 0];
                    spf[so + 1] = pairs_canonical[pi + 1];
                }
            }
        }
        break;
    }
    case QGEMM_INT8_B0:
        for (int n = 0; n < N; ++n) {
            std::memcpy(wp + (size_t)n * g.Kp, wc + (size_t)n * K, (size_t)K);
            spf[(size_t)n * 2 + 0] = pairs_canonical[(size_t)n * 2 + 0];
            spf[(size_t)n * 2 + 1] = pairs_canonical[(size_t)n * 2 + 1];
        }
        break;
    case QGEMM_INT8_BLOCK_BASE: {
        // entry (n, 64-block b, sub-block h) = pair of the block holding
        // k = 64 b + h * 64 / H
        const int H = pair_groups(g.block), nb = K / 64;
        for (int n = 0; n < N; ++n) {
            std::memcpy(wp + (size_t)n * K, wc + (size_t)n * K, (size_t)K);
            for (int b = 0; b < nb; ++b)
                for (int h = 0; h < H; ++h) {
                    const size_t pi = ((size_t)n * g.nblk + ((size_t)b * 64 + h * (64 / H)) / g.block) * 2;
                    const size_t so = (((size_t)n * nb + b) * H + h) * 2;
                    spf[so + 0] = pairs_canonical[pi + 0];
                    spf[so + 1] = pairs_canonical[pi + 1];
                }
        }
        break;
    }
    case QGEMM_W4A8: {
        // 1 KiB records (g, kc) of 32 channels x 64 codes; piece 32 h + c
        // (16 bytes) holds channel 32 g + c's codes of k = 64 kc + 32 s +
        // 16 h + [0, 16) for s = 0, 1 (8 bytes each); in word w (k0 = 64 kc +
        // 32 s + 16 h + 8 w) byte i holds q[k0 + i] | q[k0 + 4 + i] << 4.
        const int nkc = g.Kp / 64;
        const size_t row = (size_t)K / 2;
        for (int n = 0; n < N; ++n) {
            const uint8_t *src = wc + (size_t)n * row;
            const int grp = n >> 5, c = n & 31;
            for (int kc = 0; kc < nkc; ++kc) {
                uint8_t *rec = wp + ((size_t)grp * nkc + kc) * 1024;
                for (int h = 0; h < 2; ++h)
                    for (int sv = 0; sv < 2; ++sv)
                        for (int w = 0; w < 2; ++w) {
                            const int k0 = 64 * kc + 32 * sv + 16 * h + 8 * w;
                            for (int i = 0; i < 4; ++i) {
                                const uint8_t lo = (k0 + i < K) ? nib(src, k0 + i) : 0;
                                const uint8_t hi = (k0 + 4 + i < K) ? nib(src, k0 + 4 + i) : 0;
                                rec[(32 * h + c) * 16 + 8 * sv + 4 * w + i] = (uint8_t)(lo | (hi << 4));
                            }
                        }
            }
            spf[(size_t)n * 2 + 0] = pairs_canonical[(size_t)n * 2 + 0];
            spf[(size_t)n * 2 + 1] = pairs_canonical[(size_t)n * 2 + 1];
        }
        break;
    }
    }
    return QGEMM_OK;
}

qgemm_status qgemm_unpack_weights(int K, int N, qgemm_format f, const void *w_packed,
                                  size_t w_bytes, const void *s_packed, size_t s_bytes,
                                  void *w_canonical, float *pairs_canonical) {
    Geometry g;
    qgemm_status st = geometry(K, N, f, &g);
    if (st != QGEMM_OK) return st;
    if (!w_packed || (g.s_bytes && !s_packed)) return QGEMM_ERR_NULL;
    if (w_bytes < g.w_bytes || s_bytes < g.s_bytes) return QGEMM_ERR_SIZE;
    if ((size_t)N * K > 0 && !w_canonical) return QGEMM_ERR_NULL;
    if (has_pairs(f) && N > 0 && !pairs_canonical) return QGEMM_ERR_NULL;

    const uint8_t *wp = static_cast<const uint8_t *>(w_packed);
    const float *spf = reinterpret_cast<const float *>(s_packed);
    uint8_t *wc = static_cast<uint8_t *>(w_canonical);

    switch (kernel_format(f)) {
    case QGEMM_F32:
        if ((size_t)K * N) std::memcpy(wc, wp, (size_t)K * N * sizeof(float));
        break;
    case QGEMM_F16: {
        const uint16_t *src = reinterpret_cast<const uint16_t *>(wp);
        uint16_t *dst = reinterpret_cast<uint16_t *>(wc);
        for (int k = 0; k < K; ++k)
            for (int n = 0; n < N; ++n) dst[(size_t)k * N + n] = src[(size_t)n * g.Kp + k];
        break;
    }
    case QGEMM_INT4_B64:
    case QGEMM_INT4_B0: {
        const int nblk = K / 64;
        const int G = pair_groups(g.block);
        const size_t row = (size_t)K / 2;
        for (int n = 0; n < N; ++n) {
            const int t = n >> 5, c = n & 31;
            for (int b = 0; b < nblk; ++b) {
                const size_t rec = (size_t)t * nblk + b;
                for (int half = 0; half < 2; ++half)
                    std::memcpy(wc + (size_t)n * row + (size_t)b * 32 + half * 16,
                                wp + rec * 1024 + (size_t)(32 * half + c) * 16, 16);
                // every entry a block covers holds its pair
                for (int sub = 0; sub < G; ++sub) {
                    const size_t pi = ((size_t)n * g.nblk + ((size_t)b * 64 + sub * (64 / G)) / g.block) * 2;
                    const size_t so = int4_pair_entry(rec, c, sub, G);
                    pairs_canonical[pi + 0] = spf[so + 0];
                    pairs_canonical[pi + 1] = spf[so + 1];
                }
            }
        }
        break;
    }
    case QGEMM_INT8_B0:
        for (int n = 0; n < N; ++n) {
            std::memcpy(wc + (size_t)n * K, wp + (size_t)n * g.Kp, (size_t)K);
            pairs_canonical[(size_t)n * 2 + 0] = spf[(size_t)n * 2 + 0];
            pairs_canonical[(size_t)n * 2 + 1] = spf[(size_t)n * 2 + 1];
        }
        break;
    case QGEMM_INT8_BLOCK_BASE: {
        // each block's pair from the first entry it covers
        const int H = pair_groups(g.block), nb = K / 64;
        for (int n = 0; n < N; ++n) {
            std::memcpy(wc + (size_t)n * K, wp + (size_t)n * K, (size_t)K);
            for (int j = 0; j < g.nblk; ++j) {
                const size_t k = (size_t)j * g.block;
                const size_t so = (((size_t)n * nb + k / 64) * H + (k % 64) / (64 / H)) * 2;
                pairs_canonical[((size_t)n * g.nblk + j) * 2 + 0] = spf[so + 0];
                pairs_canonical[((size_t)n * g.nblk + j) * 2 + 1] = spf[so + 1];
            }
        }
        break;
    }
    case QGEMM_W4A8: {
        const int nkc = g.Kp / 64;
        const size_t row = (size_t)K / 2;
        for (int n = 0; n < N; ++n) {
            uint8_t *dst = wc + (size_t)n * row;
            std::memset(dst, 0, row);
            const int grp = n >> 5, c = n & 31;
            for (int kc = 0; kc < nkc; ++kc) {
                const uint8_t *rec = wp + ((size_t)grp * nkc + kc) * 1024;
                for (int h = 0; h < 2; ++h)
                    for (int sv = 0; sv < 2; ++sv)
                        for (int w = 0; w < 2; ++w) {
                            const int k0 = 64 * kc + 32 * sv + 16 * h + 8 * w;
                            for (int i = 0; i < 4; ++i) {
                                const uint8_t byte = rec[(32 * h + c) * 16 + 8 * sv + 4 * w + i];
                                const int ka = k0 + i, kb = k0 + 4 + i;
                                if (ka < K) dst[ka >> 1] |= (uint8_t)((byte & 15) << ((ka & 1) * 4));
                                if (kb < K) dst[kb >> 1] |= (uint8_t)((byte >> 4) << ((kb & 1) * 4));
                            }
                        }
            }
            pairs_canonical[(size_t)n * 2 + 0] = spf[(size_t)n * 2 + 0];
            pairs_canonical[(size_t)n * 2 + 1] = spf[(size_t)n * 2 + 1];
        }
        break;
    }
    }
    return QGEMM_OK;
}

}  // extern "C"
