// kernels_common.h -- vector types and small device helpers of the HIP
// kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
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

// Wave-uniform value as a scalar (lets the compiler use scalar loads).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace qg
