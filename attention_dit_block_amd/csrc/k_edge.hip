// Kernels of the layers either side of the DiT block stack on gfx950: the conditioning vector
// from the timestep (and guidance) value, and the final layer's LayerNorm modulation.  The pages
// name the denoising step of a FLUX-style model (the "CUDA codepath !" thread, antirez/iris.c
// issue #15) but print none of these layers; they follow the FLUX model's conventions.  The
// linear layers (patch / text embedding, the final projection) run on the block's GEMM kernel.
//
// All of it is small next to the blocks (a GEMV over a d x d matrix, one pass over the image
// rows), so the kernels are plain: one wave per output row, 16-byte loads, fp32 arithmetic.
#include <algorithm>

#include "dev_common.h"
#include "launch.h"

namespace dit {

// emb[j] = cos(s f_j), emb[half + j] = sin(s f_j), s = time_factor * t[0],
// f_j = exp(-log(max_period) * j / half).  In double: s f_j reaches 1e3 radians.
__global__ __launch_bounds__(256) void freq_embed_kernel(const float* t, double time_factor, double log_max_period,
                                                         int half, float* emb) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= half) return;
    const double s = time_factor * (double)t[0];
    const double a = s * exp(-log_max_period * (double)j / (double)half);
    emb[j] = (float)cos(a);
    emb[half + j] = (float)sin(a);
}

// out[r] (+)= sum_k W[r, k] act(v[k]), act = SiLU or identity; v fp32 [K] staged in LDS.
// One wave per row, 4 rows per workgroup; K % 8 == 0 (bf16) or K % 4 == 0 (fp32).
template <int WT, bool SILU_IN>
__global__ __launch_bounds__(256) void vec_gemv_kernel(const void* w, int rows, int K, const float* v, float* out,
                                                       int accumulate) {
    extern __shared__ float sv[];
    for (int k = threadIdx.x; k < K; k += 256) {
        const float x = v[k];
        sv[k] = SILU_IN ? x / (1.0f + expf(-x)) : x;
    }
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + wave;
    if (r >= rows) return;
    float acc = 0.0f;
    if constexpr (WT == BF16) {
        const bf16_t* wr = reinterpret_cast<const bf16_t*>(w) + (size_t)r * K;
        for (int k0 = lane * 8; k0 < K; k0 += 512) {
            const u32x4_v q = ld16(wr + k0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc = fmaf(bf_lo(q[j]), sv[k0 + 2 * j], fmaf(bf_hi(q[j]), sv[k0 + 2 * j + 1], acc));
        }
    } else {
        const float* wr = reinterpret_cast<const float*>(w) + (size_t)r * K;
        for (int k0 = lane * 4; k0 < K; k0 += 256) {
            const f32x4_v q = ldf4(wr + k0);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = fmaf(q[j], sv[k0 + j], acc);
        }
    }
    acc = wave_sum(acc);
    if (lane == 0) out[r] = accumulate ? out[r] + acc : acc;
}

// out (dtype) = in (fp32), n elements, rounded to nearest even.
__global__ __launch_bounds__(256) void cast_kernel(const float* in, void* out, int n, int dtype) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float x = in[i];
    if (dtype == F32) reinterpret_cast<float*>(out)[i] = x;
    else if (dtype == F16) reinterpret_cast<_Float16*>(out)[i] = (_Float16)x;
    else reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)(pack_bf16x2(x, 0.0f) & 0xffffu);
}

// out = (1 + scale) * LayerNorm(x) + shift per row, LayerNorm(x) = (x - mean) / sqrt(var + eps)
// with the population variance.  One wave per row, three passes over the row (mean, variance,
// write); d % 8 == 0.
template <int XT, int OT>
__global__ __launch_bounds__(256) void layernorm_modulate_kernel(const void* x, long ld_x, void* out, long ld_out,
                                                                 const float* shift, const float* scale, int rows,
                                                                 int d, float eps) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + wave;
    if (r >= rows) return;
    constexpr int XS = XT == F32 ? 4 : 2, OS = OT == F32 ? 4 : 2;
    const char* xr = reinterpret_cast<const char*>(x) + (size_t)r * ld_x * XS;
    char* orow = reinterpret_cast<char*>(out) + (size_t)r * ld_out * OS;
    float f[8];
    float s = 0.0f;
    for (int k0 = lane * 8; k0 < d; k0 += 512) {
        load8<XT>(xr + (size_t)k0 * XS, f);
#pragma unroll
        for (int j = 0; j < 8; ++j) s += f[j];
    }
    const float mean = wave_sum(s) / (float)d;
    float q = 0.0f;
    for (int k0 = lane * 8; k0 < d; k0 += 512) {
        load8<XT>(xr + (size_t)k0 * XS, f);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float c = f[j] - mean;
            q = fmaf(c, c, q);
        }
    }
    const float inv = 1.0f / sqrtf(wave_sum(q) / (float)d + eps);
    for (int k0 = lane * 8; k0 < d; k0 += 512) {
        load8<XT>(xr + (size_t)k0 * XS, f);
        const f32x4_v s0 = ldf4(shift + k0), s1 = ldf4(shift + k0 + 4);
        const f32x4_v c0 = ldf4(scale + k0), c1 = ldf4(scale + k0 + 4);
        float o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[j] = fmaf(1.0f + c0[j], (f[j] - mean) * inv, s0[j]);
            o[4 + j] = fmaf(1.0f + c1[j], (f[4 + j] - mean) * inv, s1[j]);
        }
        store8<OT>(orow + (size_t)k0 * OS, o);
    }
}

hipError_t launch_freq_embed(const float* t, double time_factor, double max_period, int dim, float* emb,
                             hipStream_t s) {
    const int half = dim / 2;
    hipLaunchKernelGGL(freq_embed_kernel, dim3((half + 255) / 256), dim3(256), 0, s, t, time_factor,
                       std::log(max_period), half, emb);
    return hipGetLastError();
}

hipError_t launch_vec_gemv(const void* w, int w_dtype, int rows, int K, const float* v, bool silu_in, float* out,
                           bool accumulate, hipStream_t s) {
    const dim3 grid((rows + 3) / 4), block(256);
    const size_t lds = (size_t)K * 4;
    const int acc = accumulate ? 1 : 0;
    if (w_dtype == BF16) {
        if (silu_in) hipLaunchKernelGGL((vec_gemv_kernel<BF16, true>), grid, block, lds, s, w, rows, K, v, out, acc);
        else hipLaunchKernelGGL((vec_gemv_kernel<BF16, false>), grid, block, lds, s, w, rows, K, v, out, acc);
    } else {
        if (silu_in) hipLaunchKernelGGL((vec_gemv_kernel<F32, true>), grid, block, lds, s, w, rows, K, v, out, acc);
        else hipLaunchKernelGGL((vec_gemv_kernel<F32, false>), grid, block, lds, s, w, rows, K, v, out, acc);
    }
    return hipGetLastError();
}

// bf16 -> fp16, 8 elements per thread per step (16-byte loads and stores), grid-stride; the same
// rounding as the GEMM's staging conversion (exact for |x| >= 2^-14, nearest even below).
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const uint16_t* in, uint16_t* out, size_t n) {
    const size_t n8 = n / 8;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n8; i += (size_t)gridDim.x * blockDim.x) {
        const u32x4_v w = ld16(in + i * 8);
        u32x4_v o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = bf16x2_to_f16x2(w[j]);
        *reinterpret_cast<u32x4_v*>(out + i * 8) = o;
    }
    if (blockIdx.x == 0 && threadIdx.x < n - n8 * 8) {
        const size_t i = n8 * 8 + threadIdx.x;
        out[i] = (uint16_t)(bf16x2_to_f16x2(in[i]) & 0xffffu);
    }
}

hipError_t launch_bf16_to_f16(const void* in, void* out, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t blocks = std::min<size_t>((n / 8 + 255) / 256 + 1, 8192);
    hipLaunchKernelGGL(bf16_to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(in), reinterpret_cast<uint16_t*>(out), n);
    return hipGetLastError();
}

hipError_t launch_cast(const float* in, void* out, int n, int dtype, hipStream_t s) {
    hipLaunchKernelGGL(cast_kernel, dim3((n + 255) / 256), dim3(256), 0, s, in, out, n, dtype);
    return hipGetLastError();
}

hipError_t launch_layernorm_modulate(const void* x, int x_dtype, long ld_x, void* out, int out_dtype, long ld_out,
                                     const float* shift, const float* scale, int rows, int d, float eps,
                                     hipStream_t s) {
    const dim3 grid((rows + 3) / 4), block(256);
#define DIT_LN(XT, OT)                                                                                      \
    hipLaunchKernelGGL((layernorm_modulate_kernel<XT, OT>), grid, block, 0, s, x, ld_x, out, ld_out, shift, \
                       scale, rows, d, eps)
    if (x_dtype == F32) {
        if (out_dtype == F32) DIT_LN(F32, F32);
        else if (out_dtype == F16) DIT_LN(F32, F16);
        else DIT_LN(F32, BF16);
    } else {
        if (out_dtype == F32) DIT_LN(BF16, F32);
        else if (out_dtype == F16) DIT_LN(BF16, F16);
        else DIT_LN(BF16, BF16);
    }
#undef DIT_LN
    return hipGetLastError();
}

}  // namespace dit
