// splitk.hip -- the fixed-order reduction behind split-K: C = sum over s of
// part[s] (s = 0, 1, ..., nsplit - 1, always in that order, so a result does
// not depend on which workgroup finished first), then the fused epilogue
// once per output. The partial tiles are contiguous [nsplit][M][N] fp32
// arrays; four outputs per thread, 16-byte accesses when M * N is a multiple
// of 4 and C is plain fp32.
#include "kernels_common.h"
#include "qgemm_internal.h"

namespace qg {

__global__ __launch_bounds__(256) void splitk_reduce_f32_kernel(const float *__restrict__ part,
                                                                int nsplit, size_t mn, int N,
                                                                void *__restrict__ C,
                                                                Epilogue epi) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= mn) return;
    if ((N & 3) == 0) {        // four outputs of one row (mn is a multiple of 4 too)
        f4_t acc = *reinterpret_cast<const f4_t *>(part + i);
        for (int sp = 1; sp < nsplit; ++sp) acc += *reinterpret_cast<const f4_t *>(part + (size_t)sp * mn + i);
        if (epi.plain) *reinterpret_cast<f4_t *>(static_cast<float *>(C) + i) = acc;
        else epi_put4(epi, C, (int)(i / (size_t)N), (int)(i % (size_t)N), N, acc);
    } else {
        for (size_t j = i; j < i + 4 && j < mn; ++j) {
            float acc = part[j];
            for (int sp = 1; sp < nsplit; ++sp) acc += part[(size_t)sp * mn + j];
            if (epi.plain) static_cast<float *>(C)[j] = acc;
            else epi_store(epi, C, j, epi_value(epi, acc, j, (int)(j % (size_t)N)));
        }
    }
}

hipError_t launch_splitk_reduce_f32(const float *part, int nsplit, int M, int N, void *C,
                                    const Epilogue &epi, hipStream_t s) {
    const size_t mn = (size_t)M * N;
    const size_t blocks = (mn + 1023) / 1024;
    hipLaunchKernelGGL(splitk_reduce_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, part,
                       nsplit, mn, N, C, epi);
    return hipGetLastError();
}

}  // namespace qg
