// Device helpers shared by the gfx950 kernels of the DiT block library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef uint16_t bf16_t;  // bf16 storage: the raw 16-bit pattern

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));
typedef float f32x16_v __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_v __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_v f = {lo, hi};
    bf16x2_v b = __builtin_convertvector(f, bf16x2_v);
    return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ bf16_t f2bf(float f) {
    return bf16_t(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// Unpack 8 bf16 (one 16-byte load) into fp32.
__device__ __forceinline__ void unpack8(const u32x4_v& w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf_lo(w[i]);
        f[2 * i + 1] = bf_hi(w[i]);
    }
}
__device__ __forceinline__ u32x4_v pack8(const float* f) {
    u32x4_v w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return w;
}

// Wave-wide reductions (64 lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}
// Reduction over aligned groups of `G` lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// 16-byte global loads / stores.
__device__ __forceinline__ u32x4_v ld16(const void* p) { return *reinterpret_cast<const u32x4_v*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4_v& v) { *reinterpret_cast<u32x4_v*>(p) = v; }
__device__ __forceinline__ f32x4_v ldf4(const void* p) { return *reinterpret_cast<const f32x4_v*>(p); }
__device__ __forceinline__ void stf4(void* p, const f32x4_v& v) { *reinterpret_cast<f32x4_v*>(p) = v; }

}  // namespace dit
