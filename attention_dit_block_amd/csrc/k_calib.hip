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

namespace dit {

// Streaming probes: every thread moves 64 B per iteration (four 16-byte accesses, unrolled, all
// loads issued before any use), grid-stride over the buffer.  mode 0 reads src and writes one
// float per thread (the HBM read ceiling); mode 1 copies src to dst (read + write).
__global__ __launch_bounds__(256) void stream_probe_kernel(const u32x4_v* __restrict__ src, u32x4_v* __restrict__ dst,
                                                           size_t n16, int mode, float* sink) {
    const size_t stride = (size_t)gridDim.x * 256 * 4;
    size_t i = ((size_t)blockIdx.x * 256) * 4 + threadIdx.x;
    u32x4_v acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * 256 < n16; i += stride) {
        u32x4_v v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(src + i + j * 256);
        if (mode == 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(v[j], dst + i + j * 256);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc ^= v[j];
        }
    }
    if (mode == 0) sink[(size_t)blockIdx.x * 256 + threadIdx.x] = __uint_as_float(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

hipError_t launch_stream_probe(const void* src, void* dst, size_t bytes, int mode, int workgroups, float* sink,
                               hipStream_t s) {
    hipLaunchKernelGGL(stream_probe_kernel, dim3(workgroups), dim3(256), 0, s, reinterpret_cast<const u32x4_v*>(src),
                       reinterpret_cast<u32x4_v*>(dst), bytes / 16, mode, sink);
    return hipGetLastError();
}

}  // namespace dit
