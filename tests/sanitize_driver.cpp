// Host-side driver for the AddressSanitizer / UndefinedBehaviorSanitizer build
// of the library's host code (csrc/host_pack.cpp: sizes, quantiser, packer,
// unpacker, plans) and of the CPU oracle (oracle/oracle.c). Every buffer is a
// heap allocation of exactly the size the call is entitled to, so a read or
// write one byte past it is reported. Exits non-zero on the first mismatch;
// the sanitizers abort on the first error they find.
//
// Checks, over every weight format and a spread of shapes (ragged N, K tails
// of each format, blocks of 32 up to K):
//   - canonical / packed / workspace sizes are consistent;
//   - quantise -> pack -> unpack returns the canonical buffers byte for byte;
//   - the library's quantiser equals the oracle's (codes and pairs);
//   - short buffers give QGEMM_ERR_SIZE, NULL pointers QGEMM_ERR_NULL;
//   - the oracle's GEMMs, W4A8 steps and epilogue run on small inputs, and
//     the W4A8 regrouping agrees with the dequantise-then-multiply product.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "qgemm.h"

extern "C" {
double orc_half_to_double(uint16_t h);
int orc_quantize(int N, int K, int bits, int block, const float *W, uint8_t *q, float *pairs);
int orc_gemm_f32(int M, int K, int N, const float *A, const float *B, double *C);
int orc_gemm_blockq(int M, int K, int N, int bits, int block, const uint16_t *A,
                    const uint8_t *q, const float *pairs, double *C);
int orc_w4a8_actquant(int M, int K, const uint16_t *A, int8_t *qa, float *sa, int32_t *S);
int orc_w4a8_dot(int M, int K, int N, const int8_t *qa, const uint8_t *q, int64_t *D);
int orc_w4a8_rescale(int M, int N, const int64_t *D, const float *sa, const int32_t *S,
                     const float *pairs, double *C);
int orc_w4a8_dequant_product(int M, int K, int N, const int8_t *qa, const float *sa,
                             const uint8_t *q, const float *pairs, double *C);
int orc_epilogue(int M, int N, const double *P, const float *bias, const float *res_f32,
                 const uint16_t *res_f16, int act, double *out);
}

static int g_cases = 0;

#define CHECK(cond, ...)                                               \
    do {                                                               \
        if (!(cond)) {                                                 \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);  \
            std::fprintf(stderr, __VA_ARGS__);                         \
            std::fprintf(stderr, "\n");                                \
            std::exit(1);                                              \
        }                                                              \
    } while (0)

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {       // xorshift64*, a seeded stream for the inputs
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float rndf() { return ((int)(rnd() % 20001) - 10000) / 4000.0f; }

// a random finite fp16 bit pattern of magnitude in [1/8, 4)
static uint16_t rnd_half() {
    return (uint16_t)((rnd() & 0x8000u) | ((12u + rnd() % 4u) << 10) | (rnd() & 0x3FFu));
}

struct Fmt {
    qgemm_format f;
    int bits;       // 0: float format
    int block;      // 0: one pair per channel (block = K)
    int k_mult;     // K must be a multiple of this
};

static void pack_roundtrip(const Fmt &F, int K, int N) {
    size_t qb = 0, pf = 0, wb = 0, sb = 0;
    CHECK(qgemm_canonical_size(K, N, F.f, &qb, &pf) == QGEMM_OK, "canonical_size %d %d fmt %d", K, N, (int)F.f);
    CHECK(qgemm_packed_size(K, N, F.f, &wb, &sb) == QGEMM_OK, "packed_size %d %d", K, N);
    std::vector<uint8_t> q(qb);
    std::vector<float> pairs(pf);
    if (F.bits) {
        std::vector<float> W((size_t)N * K);
        for (auto &w : W) w = rndf();
        // a constant block in channel 0 (scale 0, codes 0)
        const int blk = F.block ? F.block : K;
        for (int k = 0; k < blk; ++k) W[k] = 0.75f;
        CHECK(qgemm_quantize_weights(K, N, F.f, W.data(), q.data(), qb, pairs.data(), pf) ==
                  QGEMM_OK, "quantize %d %d", K, N);
        // the oracle's quantiser gives the same codes and pairs
        std::vector<uint8_t> oq(qb);
        std::vector<float> op(pf);
        CHECK(orc_quantize(N, K, F.bits, blk, W.data(), oq.data(), op.data()) == 0, "orc_quantize");
        CHECK(std::memcmp(oq.data(), q.data(), qb) == 0, "codes differ from the oracle's %d %d", K, N);
        CHECK(std::memcmp(op.data(), pairs.data(), pf * sizeof(float)) == 0, "pairs differ %d %d", K, N);
        // too-short canonical buffers
        CHECK(qgemm_quantize_weights(K, N, F.f, W.data(), q.data(), qb - 1, pairs.data(), pf) ==
                  QGEMM_ERR_SIZE, "short q accepted");
        if (pf)
            CHECK(qgemm_quantize_weights(K, N, F.f, W.data(), q.data(), qb, pairs.data(), pf - 1) ==
                      QGEMM_ERR_SIZE, "short pairs accepted");
        CHECK(qgemm_quantize_weights(K, N, F.f, nullptr, q.data(), qb, pairs.data(), pf) ==
                  QGEMM_ERR_NULL, "NULL W accepted");
    } else {
        for (auto &b : q) b = (uint8_t)rnd();
        if (F.f == QGEMM_F16)     // keep the fp16 weights finite
            for (size_t i = 1; i < qb; i += 2) q[i] &= 0x3B;
    }
    std::vector<uint8_t> wp(wb);
    std::vector<uint8_t> sp(sb);
    CHECK(qgemm_pack_weights(K, N, F.f, q.data(), pf ? pairs.data() : nullptr, wp.data(), wb,
                             sb ? sp.data() : nullptr, sb) == QGEMM_OK, "pack %d %d", K, N);
    if (wb)
        CHECK(qgemm_pack_weights(K, N, F.f, q.data(), pf ? pairs.data() : nullptr, wp.data(),
                                 wb - 1, sb ? sp.data() : nullptr, sb) == QGEMM_ERR_SIZE,
              "short packed buffer accepted");
    std::vector<uint8_t> q2(qb);
    std::vector<float> p2(pf);
    CHECK(qgemm_unpack_weights(K, N, F.f, wp.data(), wb, sb ? sp.data() : nullptr, sb, q2.data(),
                               pf ? p2.data() : nullptr) == QGEMM_OK, "unpack %d %d", K, N);
    CHECK(std::memcmp(q.data(), q2.data(), qb) == 0, "codes did not round-trip %d %d", K, N);
    if (pf)
        CHECK(std::memcmp(pairs.data(), p2.data(), pf * sizeof(float)) == 0,
              "pairs did not round-trip %d %d", K, N);
    for (int M : {0, 1, 3, 8, 64, 513}) {
        size_t ws = 1;
        CHECK(qgemm_workspace_size(M, K, N, F.f, &ws) == QGEMM_OK, "workspace_size");
        CHECK(M > 0 || ws == 0, "workspace for an empty shape");
    }
    ++g_cases;
}

static void oracle_small() {
    const int M = 3, K = 128, N = 5;
    std::vector<uint16_t> A((size_t)M * K);
    std::vector<float> Af((size_t)M * K), Bf((size_t)K * N);
    for (size_t i = 0; i < A.size(); ++i) {
        A[i] = rnd_half();
        Af[i] = (float)orc_half_to_double(A[i]);
    }
    for (auto &b : Bf) b = rndf();
    std::vector<double> C((size_t)M * N), C2((size_t)M * N);
    CHECK(orc_gemm_f32(M, K, N, Af.data(), Bf.data(), C.data()) == 0, "orc_gemm_f32");

    std::vector<float> W((size_t)N * K);
    for (auto &w : W) w = rndf();
    for (int bits : {4, 8})
        for (int block : {16, 32, 64, K}) {
            std::vector<uint8_t> q((size_t)N * K * bits / 8);
            std::vector<float> pairs((size_t)N * (K / block) * 2);
            CHECK(orc_quantize(N, K, bits, block, W.data(), q.data(), pairs.data()) == 0, "quantize");
            CHECK(orc_gemm_blockq(M, K, N, bits, block, A.data(), q.data(), pairs.data(), C.data()) == 0,
                  "orc_gemm_blockq");
            ++g_cases;
        }

    // W4A8: the regrouped product equals the dequantise-then-multiply one
    std::vector<uint8_t> q4((size_t)N * K / 2);
    std::vector<float> pch((size_t)N * 2);
    CHECK(orc_quantize(N, K, 4, K, W.data(), q4.data(), pch.data()) == 0, "quantize b0");
    std::vector<int8_t> qa((size_t)M * K);
    std::vector<float> sa(M);
    std::vector<int32_t> S(M);
    std::vector<int64_t> D((size_t)M * N);
    CHECK(orc_w4a8_actquant(M, K, A.data(), qa.data(), sa.data(), S.data()) == 0, "actquant");
    CHECK(orc_w4a8_dot(M, K, N, qa.data(), q4.data(), D.data()) == 0, "dot");
    CHECK(orc_w4a8_rescale(M, N, D.data(), sa.data(), S.data(), pch.data(), C.data()) == 0, "rescale");
    CHECK(orc_w4a8_dequant_product(M, K, N, qa.data(), sa.data(), q4.data(), pch.data(), C2.data()) == 0,
          "dequant_product");
    for (size_t i = 0; i < C.size(); ++i)
        CHECK(std::fabs(C[i] - C2[i]) <= 1e-9 * (1.0 + std::fabs(C2[i])), "W4A8 regrouping %zu", i);

    // epilogue: every activation, fp32 and fp16 residuals
    std::vector<float> bias(N), rf((size_t)M * N);
    std::vector<uint16_t> rh((size_t)M * N);
    for (auto &b : bias) b = rndf();
    for (size_t i = 0; i < rf.size(); ++i) {
        rh[i] = rnd_half();
        rf[i] = (float)orc_half_to_double(rh[i]);
    }
    std::vector<double> out((size_t)M * N);
    for (int act = 0; act <= 3; ++act) {
        CHECK(orc_epilogue(M, N, C.data(), bias.data(), rf.data(), nullptr, act, out.data()) == 0, "epi");
        CHECK(orc_epilogue(M, N, C.data(), nullptr, nullptr, rh.data(), act, out.data()) == 0, "epi16");
        ++g_cases;
    }
}

int main() {
    const Fmt fmts[] = {
        {QGEMM_F32, 0, 0, 1},
        {QGEMM_F16, 0, 0, 2},
        {QGEMM_INT4_B64, 4, 64, 64},
        {QGEMM_INT8_B0, 8, 0, 1},
        {QGEMM_W4A8, 4, 0, 2},
        {QGEMM_INT4_B0, 4, 0, 64},
        {QGEMM_INT4_BLOCK(16), 4, 16, 16},
        {QGEMM_INT4_BLOCK(32), 4, 32, 32},
        {QGEMM_INT4_BLOCK(48), 4, 48, 48},
        {QGEMM_INT4_BLOCK(128), 4, 128, 128},
        {QGEMM_INT8_BLOCK(16), 8, 16, 16},
        {QGEMM_INT8_BLOCK(32), 8, 32, 32},
        {QGEMM_INT8_BLOCK(80), 8, 80, 80},
        {QGEMM_INT8_BLOCK(192), 8, 192, 192},
    };
    const int Ks[] = {2, 30, 64, 66, 128, 130, 192, 320, 384, 1024};
    const int Ns[] = {1, 7, 31, 32, 33, 70, 100};
    for (const Fmt &F : fmts)
        for (int K : Ks) {
            if (K % F.k_mult) continue;
            for (int N : Ns) pack_roundtrip(F, K, N);
        }
    // a shape each format rejects is an error, not an access
    size_t a = 0, b = 0;
    CHECK(qgemm_packed_size(63, 4, QGEMM_INT4_B64, &a, &b) == QGEMM_ERR_SHAPE, "K %% 64 accepted");
    CHECK(qgemm_packed_size(64, 4, (qgemm_format)77, &a, &b) == QGEMM_ERR_FORMAT, "format 77 accepted");
    CHECK(qgemm_packed_size(64, 4, QGEMM_INT4_B64, nullptr, &b) == QGEMM_ERR_NULL, "NULL size accepted");
    oracle_small();
    std::printf("ok %d cases\n", g_cases);
    return 0;
}
