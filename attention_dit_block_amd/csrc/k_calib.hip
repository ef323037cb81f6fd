// Calibration kernel for measurements: a loop of independent fp16 MFMAs with no memory traffic,
// whose rate is the matrix cores' sustained throughput on this device at its present clock (the
// dense 2.5 PFLOP/s figure assumes the 2.4 GHz peak clock; under a full MFMA load the clock is
// usually lower).  Measurements of the other kernels are read against it.
#include "dev_common.h"
#include "launch.h"

namespace dit {

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* out) {
    const int t = threadIdx.x;
    // operands from the thread index, so the compiler cannot fold the products
    f16x8_v a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)((t + i) & 7);
        b[i] = (_Float16)((t * 3 + i) & 7);
    }
    f32x16_v c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) c[j][q] = 0.0f;
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
    out[(size_t)blockIdx.x * 256 + t] = c[0][0] + c[1][1] + c[2][2] + c[3][3];
}

hipError_t launch_mfma_loop(int workgroups, int iters, float* out, hipStream_t s) {
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0, s, iters, out);
    return hipGetLastError();
}

}  // namespace dit
