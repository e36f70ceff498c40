// api.hip -- qgemm_run / qgemm_run_ws / qgemm_run_ex / qgemm_w4a8_debug:
// argument checks, kernel choice and launches on the caller's stream.
//
// Kernel choice follows the MNN GemmSpeed benchmark page, section "Default
// test sizes and the meaning of M": M = 8 is the narrow, near-decode GEMM
// (bounded by the GEMV bandwidth floor, section "Sample data"), M = 512 a
// dense prefill GEMM. Small M therefore streams the weights once through a
// GEMV kernel; larger M goes to the MFMA tile kernels.
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "qgemm_internal.h"

namespace qg {

static std::atomic<int> g_gemv_max_m{-1};

static int gemv_max_m() {
    int v = g_gemv_max_m.load(std::memory_order_relaxed);
    if (v >= 0) return v;
    int init = kGemvMaxM;
    if (const char *e = std::getenv("QGEMM_GEMV_MAX_M")) {
        char *end = nullptr;
        long x = std::strtol(e, &end, 10);
        if (end != e && x >= 0 && x <= kGemvMaxM) init = (int)x;
    }
    int expected = -1;
    g_gemv_max_m.compare_exchange_strong(expected, init);
    return g_gemv_max_m.load(std::memory_order_relaxed);
}

// 0 unknown, 1 usable gfx950, 2 not usable; indexed by HIP device ordinal.
static std::atomic<int> g_dev_state[64];

static qgemm_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return QGEMM_ERR_DEVICE;
    }
    if (dev >= 64) return QGEMM_ERR_DEVICE;
    int st = g_dev_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        st = 2;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
            std::strncmp(prop.gcnArchName, "gfx950", 6) == 0)
            st = 1;
        (void)hipGetLastError();
        g_dev_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? QGEMM_OK : QGEMM_ERR_DEVICE;
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by every run entry point; *empty is set for M == 0 or N == 0.
static qgemm_status check_run(int M, int K, int N, qgemm_format f, const void *A,
                              const void *Bq, const void *scales, const void *C,
                              Geometry *g, bool *empty) {
    qgemm_status st = geometry(K, N, f, g);
    if (st != QGEMM_OK) return st;
    if (M < 0 || M > (1 << 24)) return QGEMM_ERR_SHAPE;
    *empty = (M == 0 || N == 0);
    if (*empty) return QGEMM_OK;
    if (!C) return QGEMM_ERR_NULL;
    if (K > 0 && (!A || !Bq)) return QGEMM_ERR_NULL;
    if (f == QGEMM_F32 || f == QGEMM_F16) {   // float weights: no pairs
        if (scales) return QGEMM_ERR_FORMAT;
    } else if (!scales) {
        return QGEMM_ERR_NULL;
    }
    if (!aligned16(C) || (A && !aligned16(A)) || (Bq && !aligned16(Bq)) ||
        (scales && !aligned16(scales)))
        return QGEMM_ERR_ALIGN;
    return QGEMM_OK;
}

// The caller's epilogue (NULL: none, fp32 C) as the kernels take it.
static qgemm_status make_epilogue(const qgemm_epilogue *e, Epilogue *out) {
    *out = Epilogue{nullptr, nullptr, QGEMM_ACT_NONE, 0, true};
    if (!e) return QGEMM_OK;
    if (e->activation < QGEMM_ACT_NONE || e->activation > QGEMM_ACT_GELU) return QGEMM_ERR_FORMAT;
    if (e->out_type != QGEMM_OUT_F32 && e->out_type != QGEMM_OUT_F16) return QGEMM_ERR_FORMAT;
    if ((e->bias && !aligned16(e->bias)) || (e->residual && !aligned16(e->residual)))
        return QGEMM_ERR_ALIGN;
    out->bias = e->bias;
    out->residual = e->residual;
    out->act = e->activation;
    out->f16 = e->out_type == QGEMM_OUT_F16 ? 1 : 0;
    out->plain = !e->bias && !e->residual && e->activation == QGEMM_ACT_NONE && !out->f16;
    return QGEMM_OK;
}

static qgemm_status launched(hipError_t e) {
    return e == hipSuccess ? QGEMM_OK : QGEMM_ERR_LAUNCH;
}

// The Int4 (every block size), Int8 (Block0 and blocked), W4A8 and
// fp16-weight GEMV kernels serve M <= the current GEMV limit (and K within
// their register budgets), within each format's own crossover with the tiled
// MFMA kernels, measured on the benchmark page's shapes: the Int8 GEMV does
// all its arithmetic on the vector ALUs and loses past 4 rows; the Int4 GEMV
// loses past 4 rows once M * K * N exceeds about 2^27.6 for K > 4096, or 2^29
// for K <= 4096 (the half-tile kernel; 8 x 4096 x 16384 is a tie), where the
// weights are large enough for the split-K GEMM to fill the chip; the fp16
// and W4A8 GEMVs win up to 8 rows.
// Everything else takes a tiled GEMM. A function of the shape alone.
static bool use_gemv(qgemm_format f, int M, int K, int N) {
    if (M > gemv_max_m()) return false;
    f = kernel_format(f);
    if (f == QGEMM_INT8_B0) return M <= 4 && K <= kGemvMaxK;
    if (f == QGEMM_INT8_BLOCK_BASE) return M <= 4 && K <= kGemvI8BlkMaxK;
    if (f == QGEMM_INT4_B64)
        return K <= kGemvMaxK &&
               (M <= 4 || (long long)M * K * N <= (K <= 4096 ? kGemvInt4HalfMaxMKN : kGemvInt4MaxMKN));
    if (f == QGEMM_W4A8) return K <= kGemvMaxK;
    if (f == QGEMM_F16) return K <= kGemvF16MaxK;
    return false;
}

// What one call does, decided once from the shape and the GEMV limit in force
// when the call starts: the kernel family and the scratch layout the caller's
// workspace was checked against. Every later step of the call reads this
// plan, so a concurrent qgemm_set_gemv_max_m cannot make one call size its
// scratch for one kernel and launch another.
struct CallPlan {
    bool gemv;
    RunWorkspace r;
    int nsplit() const { return gemv ? r.gemv_nsplit : r.nsplit; }
    // Scratch bytes the call touches: the W4A8 activation codes first, then
    // (when the kernel splits K) the partial tiles. The size reported to
    // callers (run_workspace().bytes) is a function of the shape alone and
    // never smaller than this.
    size_t used_bytes() const { return nsplit() <= 1 ? r.w4a8.bytes : r.bytes; }
};

static CallPlan plan_call(qgemm_format f, int M, int K, int N) {
    return CallPlan{use_gemv(f, M, K, N), run_workspace(f, M, K, N)};
}

static qgemm_status run_w4a8(int M, int K, int N, const CallPlan &p, const void *A,
                             const void *Bq, const void *scales, void *C, const Epilogue &epi,
                             void *ws, hipStream_t s, int32_t *D_debug) {
    const W4A8Workspace &w = p.r.w4a8;
    uint8_t *base = static_cast<uint8_t *>(ws);
    int8_t *qa = reinterpret_cast<int8_t *>(base + w.qa_off);
    float *sa = reinterpret_cast<float *>(base + w.sa_off);
    int32_t *S = reinterpret_cast<int32_t *>(base + w.S_off);
    int32_t *part = p.nsplit() > 1 ? reinterpret_cast<int32_t *>(base + p.r.part_off) : nullptr;
    if (p.gemv)   // quantises the activations itself unless split
        return launched(launch_w4a8_gemv(M, K, N, w.qa_stride, A, qa, sa, S, Bq, scales, C, epi,
                                         D_debug, p.nsplit(), part, s));
    hipError_t e = launch_w4a8_actquant(M, K, w.qa_stride, A, qa, sa, S, s);
    if (e != hipSuccess) return QGEMM_ERR_LAUNCH;
    return launched(launch_w4a8_gemm(M, K, N, w.qa_stride, qa, sa, S, Bq, scales, C, epi, D_debug,
                                     p.nsplit(), part, s));
}


static qgemm_status dispatch(int M, int K, int N, qgemm_format f, const Geometry &g,
                             const CallPlan &p, const void *A, const void *Bq, const void *scales,
                             void *C, const Epilogue &epi, void *ws, hipStream_t s) {
    (void)hipGetLastError();   // start from a clean per-thread error state
    const bool gemv = p.gemv;
    const int nsplit = p.nsplit();
    float *part = nsplit > 1 ? reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + p.r.part_off)
                             : nullptr;
    switch (kernel_format(f)) {
    case QGEMM_F32:
        return launched(launch_gemm_f32(M, K, N, static_cast<const float *>(A),
                                        static_cast<const float *>(Bq), C, epi, nsplit, part, s));
    case QGEMM_INT4_B64:   // every Int4 format without A8 packs as Int4-Block64
        return launched(gemv ? launch_gemv_int4b64(M, K, N, A, Bq, scales, C, epi, pair_groups(g.block),
                                                   nsplit, part, s)
                             : launch_gemm_int4b64(M, K, N, A, Bq, scales, C, epi, pair_groups(g.block),
                                                   nsplit, part, s));
    case QGEMM_INT8_B0:
        return launched(gemv ? launch_gemv_int8b0(M, K, N, A, Bq, scales, C, epi, s)
                             : launch_gemm_int8b0(M, K, N, A, Bq, scales, C, epi, nsplit, part, s));
    case QGEMM_INT8_BLOCK_BASE:   // Int8 with a pair per block of K
        return launched(gemv ? launch_gemv_int8blk(M, K, N, A, Bq, scales, C, epi, pair_groups(g.block), s)
                             : launch_gemm_int8blk(M, K, N, A, Bq, scales, C, epi, pair_groups(g.block),
                                                   nsplit, part, s));
    case QGEMM_W4A8:
        return run_w4a8(M, K, N, p, A, Bq, scales, C, epi, ws, s, nullptr);
    case QGEMM_F16:
        return launched(gemv ? launch_gemv_f16(M, K, N, A, Bq, C, epi, s)
                             : launch_gemm_f16(M, K, N, A, Bq, C, epi, nsplit, part, s));
    default:
        break;
    }
    return QGEMM_ERR_FORMAT;
}

// Scratch of qgemm_run_noalloc: one array in each GPU's memory, reserved
// when this code object is loaded on the device. In host code the array's
// name is only a stand-in: its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[QGEMM_NOALLOC_SCRATCH_BYTES];
static std::atomic<void *> g_scratch_ptr[64];
static std::mutex g_scratch_mutex;

static qgemm_status scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return QGEMM_ERR_DEVICE;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return QGEMM_ERR_DEVICE;
            }
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return QGEMM_OK;
}

}  // namespace qg

using namespace qg;

extern "C" {

int qgemm_set_gemv_max_m(int max_m) {
    int prev = gemv_max_m();
    if (max_m >= 0 && max_m <= kGemvMaxM) g_gemv_max_m.store(max_m);
    return prev;
}

qgemm_status qgemm_run_ex(int M, int K, int N, qgemm_format f, const void *A,
                          const void *Bq, const void *scales, void *C,
                          const qgemm_epilogue *epilogue, void *workspace, size_t ws_bytes,
                          void *stream) {
    Geometry g;
    bool empty = false;
    qgemm_status st = check_run(M, K, N, f, A, Bq, scales, C, &g, &empty);
    if (st != QGEMM_OK || empty) return st;
    Epilogue epi;
    st = make_epilogue(epilogue, &epi);
    if (st != QGEMM_OK) return st;
    const CallPlan plan = plan_call(f, M, K, N);
    const size_t need = plan.used_bytes();
    const bool own = !workspace && ws_bytes == 0;   // scratch, if any, is ours to allocate
    if (need > 0 && !own) {
        if (!workspace) return QGEMM_ERR_NULL;
        if (!aligned16(workspace)) return QGEMM_ERR_ALIGN;
        if (ws_bytes < need) return QGEMM_ERR_SIZE;
    }
    st = check_device();
    if (st != QGEMM_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (need == 0 || !own) return dispatch(M, K, N, f, g, plan, A, Bq, scales, C, epi, workspace, s);
    // Scratch (W4A8 codes, split-K partials), allocated and released in stream order.
    void *ws = nullptr;
    if (hipMallocAsync(&ws, need, s) != hipSuccess || !ws) {
        (void)hipGetLastError();
        return QGEMM_ERR_NOMEM;
    }
    st = dispatch(M, K, N, f, g, plan, A, Bq, scales, C, epi, ws, s);
    if (hipFreeAsync(ws, s) != hipSuccess) {
        (void)hipGetLastError();
        if (st == QGEMM_OK) st = QGEMM_ERR_LAUNCH;
    }
    return st;
}

qgemm_status qgemm_run_noalloc(int M, int K, int N, qgemm_format f, const void *A,
                               const void *Bq, const void *scales, void *C,
                               const qgemm_epilogue *epilogue, void *stream) {
    Geometry g;
    bool empty = false;
    qgemm_status st = check_run(M, K, N, f, A, Bq, scales, C, &g, &empty);
    if (st != QGEMM_OK || empty) return st;
    Epilogue epi;
    st = make_epilogue(epilogue, &epi);
    if (st != QGEMM_OK) return st;
    const CallPlan plan = plan_call(f, M, K, N);
    const size_t need = plan.used_bytes();
    if (need > QGEMM_NOALLOC_SCRATCH_BYTES) return QGEMM_ERR_SIZE;
    st = check_device();
    if (st != QGEMM_OK) return st;
    void *ws = nullptr;
    if (need > 0) {
        st = scratch_address(&ws);
        if (st != QGEMM_OK) return st;
    }
    return dispatch(M, K, N, f, g, plan, A, Bq, scales, C, epi, ws, static_cast<hipStream_t>(stream));
}

qgemm_status qgemm_run_ws(int M, int K, int N, qgemm_format f, const void *A,
                          const void *Bq, const void *scales, float *C, void *workspace,
                          size_t ws_bytes, void *stream) {
    // a caller workspace, never a library allocation (NULL with size 0 is
    // only accepted when the shape needs none)
    if (!workspace && ws_bytes == 0 && M > 0 && N > 0) {
        Geometry g;
        bool empty = false;
        qgemm_status st = check_run(M, K, N, f, A, Bq, scales, C, &g, &empty);
        if (st != QGEMM_OK) return st;
        if (plan_call(f, M, K, N).used_bytes() > 0) return QGEMM_ERR_NULL;
    }
    return qgemm_run_ex(M, K, N, f, A, Bq, scales, C, nullptr, workspace, ws_bytes, stream);
}

qgemm_status qgemm_run(int M, int K, int N, qgemm_format f, const void *A, const void *Bq,
                       const void *scales, float *C, void *stream) {
    return qgemm_run_ex(M, K, N, f, A, Bq, scales, C, nullptr, nullptr, 0, stream);
}

qgemm_status qgemm_w4a8_debug(int M, int K, int N, const void *A, const void *Bq,
                              const void *scales, float *C, int8_t *qa, float *sa,
                              int32_t *S, int32_t *D, void *workspace, size_t ws_bytes,
                              void *stream) {
    Geometry g;
    bool empty = false;
    qgemm_status st = check_run(M, K, N, QGEMM_W4A8, A, Bq, scales, C, &g, &empty);
    if (st != QGEMM_OK || empty) return st;
    if (!qa || !sa || !S || !D || !workspace) return QGEMM_ERR_NULL;
    if (!aligned16(workspace) || !aligned16(D)) return QGEMM_ERR_ALIGN;
    const CallPlan plan = plan_call(QGEMM_W4A8, M, K, N);
    const W4A8Workspace &w = plan.r.w4a8;
    if (ws_bytes < plan.used_bytes()) return QGEMM_ERR_SIZE;
    st = check_device();
    if (st != QGEMM_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const Epilogue plain{nullptr, nullptr, QGEMM_ACT_NONE, 0, true};
    st = run_w4a8(M, K, N, plan, A, Bq, scales, C, plain, workspace, s, D);
    if (st != QGEMM_OK) return st;
    const uint8_t *base = static_cast<const uint8_t *>(workspace);
    if (hipMemcpy2DAsync(qa, (size_t)K, base + w.qa_off, (size_t)w.qa_stride, (size_t)K, (size_t)M,
                         hipMemcpyDeviceToDevice, s) != hipSuccess ||
        hipMemcpyAsync(sa, base + w.sa_off, (size_t)M * sizeof(float),
                       hipMemcpyDeviceToDevice, s) != hipSuccess ||
        hipMemcpyAsync(S, base + w.S_off, (size_t)M * sizeof(int32_t),
                       hipMemcpyDeviceToDevice, s) != hipSuccess) {
        (void)hipGetLastError();
        return QGEMM_ERR_LAUNCH;
    }
    return QGEMM_OK;
}

// Checks shared by the device quantisers; *empty is set for N == 0.
static qgemm_status check_quantize(int K, int N, qgemm_format f, const float *W, const void *q,
                                   const void *pairs, Geometry *g, bool *empty) {
    if (f == QGEMM_F32 || f == QGEMM_F16) return QGEMM_ERR_FORMAT;   // float weights are not quantised
    qgemm_status st = geometry(K, N, f, g);
    if (st != QGEMM_OK) return st;
    // blocked formats: blocks of 16, 32 or a multiple of 64 (other multiples
    // of 16 straddle the kernel's 64-element chunks; quantise them on the host)
    if ((is_int4_blocked(f) || is_int8_blocked(f)) && g->block != 16 && g->block != 32 &&
        g->block % 64 != 0)
        return QGEMM_ERR_FORMAT;
    *empty = N == 0;
    if (*empty) return QGEMM_OK;
    if (!W || !q || !pairs) return QGEMM_ERR_NULL;
    if (!aligned16(W) || !aligned16(q) || !aligned16(pairs)) return QGEMM_ERR_ALIGN;
    return check_device();
}

qgemm_status qgemm_quantize_weights_device(int K, int N, qgemm_format f, const float *W,
                                           void *q, float *pairs, void *stream) {
    Geometry g;
    bool empty = false;
    qgemm_status st = check_quantize(K, N, f, W, q, pairs, &g, &empty);
    if (st != QGEMM_OK || empty) return st;
    (void)hipGetLastError();
    return launched(launch_quantize(K, N, f, false, W, q, pairs, g, static_cast<hipStream_t>(stream)));
}

qgemm_status qgemm_quantize_pack_device(int K, int N, qgemm_format f, const float *W, void *Bq,
                                        void *scales, void *stream) {
    Geometry g;
    bool empty = false;
    qgemm_status st = check_quantize(K, N, f, W, Bq, scales, &g, &empty);
    if (st != QGEMM_OK || empty) return st;
    (void)hipGetLastError();
    return launched(launch_quantize(K, N, f, true, W, Bq, static_cast<float *>(scales), g,
                                    static_cast<hipStream_t>(stream)));
}

}  // extern "C"
