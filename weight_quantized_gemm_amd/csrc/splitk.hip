// splitk.hip -- the fixed-order reduction behind split-K: C = sum over s of
// part[s] (s = 0, 1, ..., nsplit - 1, always in that order, so a result does
// not depend on which workgroup finished first). The partial tiles are
// contiguous [nsplit][M][N] fp32 arrays; four outputs per thread, 16-byte
// accesses when M * N is a multiple of 4.
#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

__global__ __launch_bounds__(256) void splitk_reduce_f32_kernel(const float *__restrict__ part,
                                                                int nsplit, size_t mn,
                                                                float *__restrict__ C) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= mn) return;
    if ((mn & 3) == 0) {
        f4_t acc = *reinterpret_cast<const f4_t *>(part + i);
        for (int sp = 1; sp < nsplit; ++sp) acc += *reinterpret_cast<const f4_t *>(part + (size_t)sp * mn + i);
        *reinterpret_cast<f4_t *>(C + i) = acc;
    } else {
        for (size_t j = i; j < i + 4 && j < mn; ++j) {
            float acc = part[j];
            for (int sp = 1; sp < nsplit; ++sp) acc += part[(size_t)sp * mn + j];
            C[j] = acc;
        }
    }
}

hipError_t launch_splitk_reduce_f32(const float *part, int nsplit, int M, int N, float *C,
                                    hipStream_t s) {
    const size_t mn = (size_t)M * N;
    const size_t blocks = (mn + 1023) / 1024;
    hipLaunchKernelGGL(splitk_reduce_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, part,
                       nsplit, mn, C);
    return hipGetLastError();
}

}  // namespace qg
