// kernels_common.h -- vector types and small device helpers of the HIP
// kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemm_internal.h"

namespace qg {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f16_t __attribute__((ext_vector_type(16)));
typedef unsigned u2_t __attribute__((ext_vector_type(2)));
typedef unsigned u4_t __attribute__((ext_vector_type(4)));
typedef int i4_t __attribute__((ext_vector_type(4)));
typedef int i16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ h2_t as_h2(unsigned x) { return __builtin_bit_cast(h2_t, x); }
__device__ __forceinline__ unsigned as_u(h2_t x) { return __builtin_bit_cast(unsigned, x); }

// fp32 pair -> packed fp16 pair (round to nearest even).
__device__ __forceinline__ unsigned pack_h2(float lo, float hi) {
    h2_t r = {(_Float16)lo, (_Float16)hi};
    return as_u(r);
}

// a.x*b.x + a.y*b.y + c with fp32 accumulation (v_dot2_f32_f16).
__device__ __forceinline__ float dot2(h2_t a, h2_t b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

// First item of slice z when n items are dealt to Z contiguous slices of
// near-equal length (z = Z gives n); the split-K kernels' K ranges. 32-bit
// arithmetic (z <= Z <= 16 and n < 2^27 keep the product exact; a 64-bit
// division would put hundreds of instructions before a kernel's first
// load), and none at all for a single slice.
__device__ __forceinline__ int slice_begin(unsigned z, int n, unsigned Z) {
    return Z == 1 ? (z == 0 ? 0 : n) : (int)(z * (unsigned)n / Z);
}

// Wave-uniform value as a scalar (lets the compiler use scalar loads).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Buffer resource of a raw byte range (gfx9 format word: 32-bit data,
// no swizzle); loads through it take a per-lane and a scalar byte offset, so
// a per-block advance is one scalar add.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS, lane l's at lds + 16 l
// (the gfx950 16-byte form of the LDS DMA: no registers, no LDS write
// instruction). The compiler does not order these LDS writes against later
// LDS reads: a reader waits for them with an explicit vm_wait.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void *lds, unsigned voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             (int)voff, 0, 0, 0);
#endif
}

// s_waitcnt operand that waits until at most n vector memory loads are
// outstanding and nothing else (vmcnt split over bits 3:0 and 15:14).
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// ---------------------------------------------------------------------------
// Fused epilogue (SimdPaddleOCR pull request: fp32 accumulators are never
// narrowed before bias, residual and activation): for output (m, n) at
// mn = m * N + n, v = act((p + bias[n]) + residual[mn]) in fp32, then stored
// as fp32 or rounded once to fp16 (nearest even). The activations use the
// device math library's expf / erff.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float epi_act(float v, int act) {
    switch (act) {
    case 1: return v > 0.f ? v : 0.f;                                     // ReLU
    case 2: return v / (1.0f + expf(-v));                                 // SiLU
    case 3: return 0.5f * v * (1.0f + erff(v * 0.7071067811865476f));     // GELU (erf)
    default: return v;
    }
}

__device__ __forceinline__ float epi_value(const Epilogue &e, float p, size_t mn, int n) {
    float v = p;
    if (e.bias) v += e.bias[n];
    if (e.residual)
        v += e.f16 ? (float)static_cast<const _Float16 *>(e.residual)[mn]
                   : static_cast<const float *>(e.residual)[mn];
    return epi_act(v, e.act);
}

__device__ __forceinline__ void epi_store(const Epilogue &e, void *C, size_t mn, float v) {
    if (e.f16) static_cast<_Float16 *>(C)[mn] = (_Float16)v;
    else static_cast<float *>(C)[mn] = v;
}

// One output through the epilogue.
__device__ __forceinline__ void epi_put(const Epilogue &e, void *C, int m, int n, int N, float p) {
    const size_t mn = (size_t)m * N + n;
    epi_store(e, C, mn, epi_value(e, p, mn, n));
}

// Four consecutive outputs (m, n .. n + 3), the same arithmetic as epi_put
// per element, with 16-byte (fp32) or 8-byte (fp16) accesses. Requires
// n + 3 < N, n % 4 == 0 and N % 4 == 0 (so every access is aligned).
__device__ __forceinline__ void epi_put4(const Epilogue &e, void *C, int m, int n, int N, f4_t p) {
    const size_t mn = (size_t)m * N + n;
    f4_t v = p;
    if (e.bias) v += *reinterpret_cast<const f4_t *>(e.bias + n);
    if (e.residual) {
        if (e.f16) {
            const h4_t r = *reinterpret_cast<const h4_t *>(static_cast<const _Float16 *>(e.residual) + mn);
            v += f4_t{(float)r[0], (float)r[1], (float)r[2], (float)r[3]};
        } else {
            v += *reinterpret_cast<const f4_t *>(static_cast<const float *>(e.residual) + mn);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = epi_act(v[i], e.act);
    if (e.f16)
        *reinterpret_cast<h4_t *>(static_cast<_Float16 *>(C) + mn) =
            h4_t{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    else
        *reinterpret_cast<f4_t *>(static_cast<float *>(C) + mn) = v;
}

}  // namespace qg
