// Pieces shared by the gfx950 attention kernels (joint attention and windowed attention): the
// K / V tile geometry in LDS, the MFMA fragment types and the cross-half-wave reductions.
#pragma once

#include "dev_common.h"

namespace dit {

constexpr int AK = 64;       // keys per tile
constexpr int HD = 128;      // head dim
constexpr int kTile = AK * HD * 2;          // bytes of one K (or V) tile: 64 rows of 256 B
constexpr float kLazyMax = 8.0f;            // log2 of the largest unnormalised probability
constexpr float kLazyP = 256.0f;             // 2^kLazyMax


typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4_v __attribute__((ext_vector_type(4)));
typedef short s16x8_v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_v lds_s16x4;

// Key held by S^T fragment row r of a 32-key block: bits 2 and 3 of r exchanged.
__device__ __forceinline__ int key_of_row(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
// K and V tiles are four slabs of 64 rows x 64 B (4 chunks of 16 B), slab b holding features
// 32 b .. 32 b + 31 of each key.  K: chunk c of row r sits at position c ^ ((r >> 2) & 3), so the
// 16 lanes of a ds_read_b128 (16 keys, one chunk) hit 16 different bank groups.  V is not
// swizzled: the rows addressed by each half-wave of a transposing read are 4 consecutive
// 64-byte rows of one slab, 256 contiguous bytes.
__device__ __forceinline__ int kpos(int r, int c) { return c ^ ((r >> 2) & 3); }

template <int DT> struct AFrag;
template <> struct AFrag<BF16> { typedef bf16x8_v T; };
template <> struct AFrag<F16> { typedef f16x8_v T; };

template <int DT>
__device__ __forceinline__ f32x16_v amfma(const typename AFrag<DT>::T& a, const typename AFrag<DT>::T& b,
                                          const f32x16_v& c) {
    if constexpr (DT == F16) return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max of x over lanes l and l ^ 32
__device__ __forceinline__ float half_swap_max(float x) {
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace dit
