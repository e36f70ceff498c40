// probe.hip -- measured-peak probes of this chip (a separate library,
// libqgemm_probe.so, used by the bench's peak mode; never by the GEMM path).
//
// The roofline fractions the bench reports are against MI355X's published
// peaks. These probes measure what the same chip delivers to plain kernels
// of the same shape, so a kernel's gap to the published peak can be split
// into the part any kernel pays and the part that is its own:
//  - an HBM read stream and a read+write copy over a buffer of the decode
//    GEMV's size (and larger), rotated past the Infinity Cache by the caller;
//  - a loop of independent fp16 MFMAs (32 x 32 x 16), optionally interleaved
//    with fp32->fp16 fused multiply-adds from the same wave (the dequantising
//    instruction of the Int4 GEMM), with the shader clock read in-kernel;
//  - an L2-resident read in the access patterns of the prefill GEMM's
//    operands, in bytes per clock per CU.
// Every index stays inside the caller's buffer: the stream probes cover
// exactly `bytes` (a multiple of 16), and the L2 probe wraps its offsets
// modulo a power-of-two window no larger than the buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemm_probe.h"

namespace {

typedef unsigned u4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f16_t __attribute__((ext_vector_type(16)));

constexpr int kUnroll = 8;   // independent 16-byte loads per thread per turn

// Read-only stream: thread t of T reads 16-byte items t, t + T, ... of n,
// eight at a time, and folds them into one word per thread (stored, so the
// loads cannot be dropped).
__global__ __launch_bounds__(256) void read_stream_kernel(const u4_t *__restrict__ src, size_t n,
                                                          unsigned *__restrict__ sink) {
    const size_t T = (size_t)gridDim.x * blockDim.x;
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u4_t acc = {0u, 0u, 0u, 0u};
    size_t i = t;
    for (; i + (kUnroll - 1) * T < n; i += kUnroll * T) {
        u4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * T);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n; i += T) acc ^= src[i];
    sink[t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Copy: the same walk, each item stored to dst.
__global__ __launch_bounds__(256) void copy_stream_kernel(const u4_t *__restrict__ src,
                                                          u4_t *__restrict__ dst, size_t n) {
    const size_t T = (size_t)gridDim.x * blockDim.x;
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t i = t;
    for (; i + (kUnroll - 1) * T < n; i += kUnroll * T) {
        u4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * T);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * T);
    }
    for (; i < n; i += T) dst[i] = src[i];
}

// MFMA loop: each wave runs `iters` turns of four independent
// v_mfma_f32_32x32x16_f16 (four accumulator tiles), and, with VALU > 0,
// VALU fp32 fused multiply-adds rounded to fp16 per MFMA on registers the
// MFMAs do not touch. Wave 0 of each workgroup records the shader clock and
// the 100 MHz reference clock at its start and end in clk[4 * block ..].
template <int VALU>
__global__ __launch_bounds__(1024) void mfma_loop_kernel(int iters, float seed,
                                                         unsigned long long *__restrict__ clk,
                                                         float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    h8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (_Float16)(seed * (float)(lane + e));
        b[e] = (_Float16)(seed * (float)(lane - e));
    }
    f16_t acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
    float x[8];
    h8_t hv = {};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = seed + (float)e;
    const bool w0 = threadIdx.x == 0;
    unsigned long long c0 = 0, r0 = 0;
    if (w0) {
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int it = 0; it < iters; ++it) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc0, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < VALU; ++v) hv[v & 7] = (_Float16)fmaf((float)hv[v & 7], seed, x[v & 7]);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc1, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < VALU; ++v) hv[v & 7] = (_Float16)fmaf((float)hv[v & 7], seed, x[v & 7]);
        acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc2, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < VALU; ++v) hv[v & 7] = (_Float16)fmaf((float)hv[v & 7], seed, x[v & 7]);
        acc3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc3, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < VALU; ++v) hv[v & 7] = (_Float16)fmaf((float)hv[v & 7], seed, x[v & 7]);
    }
    if (w0) {
        const unsigned long long c1 = __builtin_amdgcn_s_memtime();
        const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
        clk[4 * blockIdx.x + 0] = c0;
        clk[4 * blockIdx.x + 1] = c1;
        clk[4 * blockIdx.x + 2] = r0;
        clk[4 * blockIdx.x + 3] = r1;
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc0[e] + acc1[e] + acc2[e] + acc3[e];
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)hv[e];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// L2-resident read. Every wave of the grid reads, `iters` times, 16-byte
// pieces of a window of 2^wbits bytes (offsets wrap modulo the window) in
// one of three patterns, per load instruction of a wave:
//   0: 1 KiB contiguous (a packed weight record);
//   1: 8 rows x 128 bytes, rows `stride` bytes apart (an A block fetched with
//      128-byte row runs);
//   2: 16 rows x 64 bytes, rows `stride` bytes apart (A read in the MFMA's
//      lane layout).
// Eight loads are in flight per thread. Wave 0 of each workgroup records
// the shader clock at start and end in clk[2 * block ..].
__global__ __launch_bounds__(512) void l2_read_kernel(const unsigned char *__restrict__ buf,
                                                      int wbits, int pattern, int stride, int iters,
                                                      unsigned long long *__restrict__ clk,
                                                      unsigned *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const unsigned mask = (1u << wbits) - 1u;
    unsigned lane_off;
    if (pattern == 0) lane_off = 16u * lane;
    else if (pattern == 1) lane_off = (unsigned)(lane >> 3) * stride + 16u * (lane & 7);
    else lane_off = (unsigned)(lane >> 2) * stride + 16u * (lane & 3);
    // each wave starts at its own place in the window
    unsigned base = (unsigned)(blockIdx.x * 16 + wave) * 4096u;
    const unsigned step = pattern == 0 ? 1024u : (pattern == 1 ? 128u : 64u);
    u4_t acc = {0u, 0u, 0u, 0u};
    const bool w0 = threadIdx.x == 0;
    unsigned long long c0 = 0;
    __syncthreads();
    if (w0) c0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
        u4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            // patterns 1 and 2 walk along the row (the K direction) and then
            // to the next row band
            const unsigned o = (base + (unsigned)(it * kUnroll + u) * step + lane_off) & mask & ~15u;
            v[u] = *reinterpret_cast<const u4_t *>(buf + o);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    __syncthreads();
    if (w0) {
        clk[2 * blockIdx.x + 0] = c0;
        clk[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memtime();
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" {

int qgemm_probe_read(const void *src, size_t bytes, unsigned *sink, int grid, void *stream) {
    if (!src || !sink || grid <= 0 || (bytes & 15)) return 1;
    hipLaunchKernelGGL(read_stream_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u4_t *>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

int qgemm_probe_copy(const void *src, void *dst, size_t bytes, int grid, void *stream) {
    if (!src || !dst || grid <= 0 || (bytes & 15)) return 1;
    hipLaunchKernelGGL(copy_stream_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u4_t *>(src), static_cast<u4_t *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

int qgemm_probe_mfma(int iters, int valu_per_mfma, int waves, int grid, unsigned long long *clk,
                     float *sink, void *stream) {
    if (!clk || !sink || iters <= 0 || grid <= 0 || waves < 1 || waves > 16) return 1;
    auto s = static_cast<hipStream_t>(stream);
    const dim3 g(grid), b(64 * waves);
    switch (valu_per_mfma) {
    case 0: hipLaunchKernelGGL(mfma_loop_kernel<0>, g, b, 0, s, iters, 0.001f, clk, sink); break;
    case 4: hipLaunchKernelGGL(mfma_loop_kernel<4>, g, b, 0, s, iters, 0.001f, clk, sink); break;
    case 8: hipLaunchKernelGGL(mfma_loop_kernel<8>, g, b, 0, s, iters, 0.001f, clk, sink); break;
    case 16: hipLaunchKernelGGL(mfma_loop_kernel<16>, g, b, 0, s, iters, 0.001f, clk, sink); break;
    default: return 3;
    }
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

int qgemm_probe_l2(const void *buf, size_t bytes, int wbits, int pattern, int stride, int iters,
                   int waves, int grid, unsigned long long *clk, unsigned *sink, void *stream) {
    if (!buf || !clk || !sink || iters <= 0 || grid <= 0 || waves < 1 || waves > 8) return 1;
    if (wbits < 12 || wbits > 30 || ((size_t)1 << wbits) > bytes) return 2;
    if (pattern < 0 || pattern > 2 || stride < 0 || (stride & 15)) return 3;
    hipLaunchKernelGGL(l2_read_kernel, dim3(grid), dim3(64 * waves), 0, static_cast<hipStream_t>(stream),
                       static_cast<const unsigned char *>(buf), wbits, pattern, stride, iters, clk, sink);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
