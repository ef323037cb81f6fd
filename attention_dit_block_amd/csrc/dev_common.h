// Device helpers shared by the gfx950 kernels of the DiT block library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace dit {

typedef uint16_t bf16_t;  // 16-bit storage: the raw bit pattern (bf16 or fp16)

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));
typedef float f32x16_v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_v __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

template <int DT> struct ESize { static constexpr int v = DT == F32 ? 4 : (DT == 3 ? 1 : 2); };   // 3: fp8 codes

// ---- 16-bit formats <-> fp32.  Widening is exact; narrowing rounds to nearest even
// (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float h_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_v, w)[0]; }
__device__ __forceinline__ float h_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_v, w)[1]; }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_v f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f32x2_v f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_v));
}
// Two bf16 values -> the same two values as fp16 (exact for normal fp16 magnitudes; values
// below 2^-14 become fp16 subnormals, rounded to nearest even).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) { return pack_f16x2(bf_lo(w), bf_hi(w)); }

template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return DT == F16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}
template <int DT>
__device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi) {
    if (DT == F16) { lo = h_lo(w); hi = h_hi(w); }
    else { lo = bf_lo(w); hi = bf_hi(w); }
}

// 16-byte global loads / stores.
__device__ __forceinline__ u32x4_v ld16(const void* p) { return *reinterpret_cast<const u32x4_v*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4_v& v) { *reinterpret_cast<u32x4_v*>(p) = v; }
__device__ __forceinline__ f32x4_v ldf4(const void* p) { return *reinterpret_cast<const f32x4_v*>(p); }
__device__ __forceinline__ void stf4(void* p, const f32x4_v& v) { *reinterpret_cast<f32x4_v*>(p) = v; }

// 8 consecutive elements of type DT <-> fp32 (one 16-byte access for 16-bit types, two for fp32).
template <int DT>
__device__ __forceinline__ void load8(const char* p, float* f) {
    if (DT == F32) {
        const f32x4_v a = ldf4(p), b = ldf4(p + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[i] = a[i]; f[4 + i] = b[i]; }
    } else {
        const u32x4_v w = ld16(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) unpack2<DT>(w[i], f[2 * i], f[2 * i + 1]);
    }
}
template <int DT>
__device__ __forceinline__ void store8(char* p, const float* f) {
    if (DT == F32) {
        f32x4_v a = {f[0], f[1], f[2], f[3]}, b = {f[4], f[5], f[6], f[7]};
        stf4(p, a);
        stf4(p + 16, b);
    } else {
        u32x4_v w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack2<DT>(f[2 * i], f[2 * i + 1]);
        st16(p, w);
    }
}
// 4 consecutive elements (8 bytes for 16-bit types, 16 for fp32).
template <int DT>
__device__ __forceinline__ void load4(const char* p, float* f) {
    if (DT == F32) {
        const f32x4_v a = ldf4(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = a[i];
    } else {
        const u32x2_v w = *reinterpret_cast<const u32x2_v*>(p);
        unpack2<DT>(w[0], f[0], f[1]);
        unpack2<DT>(w[1], f[2], f[3]);
    }
}
template <int DT>
__device__ __forceinline__ void store4(char* p, const float* f) {
    if (DT == F32) {
        f32x4_v a = {f[0], f[1], f[2], f[3]};
        stf4(p, a);
    } else {
        u32x2_v w = {pack2<DT>(f[0], f[1]), pack2<DT>(f[2], f[3])};
        *reinterpret_cast<u32x2_v*>(p) = w;
    }
}

// One element (RNE for 16-bit types).
template <int DT>
__device__ __forceinline__ void store1(char* p, float f) {
    if (DT == F32) *reinterpret_cast<float*>(p) = f;
    else *reinterpret_cast<unsigned short*>(p) = (unsigned short)(pack2<DT>(f, 0.0f) & 0xffffu);
}

// fp16 range check of an fp32 result about to be rounded to fp16: true when it is NaN or
// |x| > 65504 (it would not stay a finite fp16 value).
__device__ __forceinline__ bool f16_out_of_range(float x) { return !(fabsf(x) <= 65504.0f); }
__device__ __forceinline__ bool f16_out_of_range4(const float* x) {
    return (int)f16_out_of_range(x[0]) + (int)f16_out_of_range(x[1]) + (int)f16_out_of_range(x[2]) +
           (int)f16_out_of_range(x[3]) != 0;
}
// OR kRangeF16 into the range-flag word (vector atomic; only lanes that saw a bad value write).
__device__ __forceinline__ void raise_range_flag(unsigned* flag, bool bad) {
    if (bad && flag) __hip_atomic_fetch_or(flag, kRangeF16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Reductions over aligned groups of 16 lanes by DPP moves (no LDS round trip).  Every lane of a
// group ends with the same bits: after the quad steps each lane holds its quad's value S_q, then
// row_mirror adds quad 3 - q and row_half_mirror the neighbouring quad's pair, so each lane forms
// (S_0 + S_3) + (S_1 + S_2) up to the order of two commutative operands.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f32<0xB1>(v);      // quad_perm [1, 0, 3, 2]
    v += dpp_f32<0x4E>(v);      // quad_perm [2, 3, 0, 1]
    v += dpp_f32<0x140>(v);     // row_mirror: lane 15 - j of the row of 16
    v += dpp_f32<0x141>(v);     // row_half_mirror: lane 7 - j of the half row
    return v;
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    return v;
}

// XCD-aware remap: consecutive workgroup ids go round-robin over the 8 XCDs; give each XCD a
// contiguous range of work indices instead (workgroups sharing operands then share one L2).
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
    const int x = bid & 7, idx = bid >> 3;
    const int q = nwg >> 3, r = nwg & 7;
    return x * q + min(x, r) + idx;
}

// ---- stream-K plumbing.  A persistent grid of G workgroups splits S work steps evenly; a piece
// of a work unit that some workgroup does not finish itself is handed over through a partial
// result and a 32-bit flag.  Partials move as 16-byte sc1 buffer loads and stores and flags as
// relaxed device-scope atomics (sc1 accesses as well): on gfx950 these go to the coherence point
// past the XCD-private L2s, so no cache-wide writeback or invalidate (which a release / acquire
// fence would issue, for the whole XCD's L2) is needed.  Ordering comes from waiting for the
// partial's stores to be acknowledged before the flag is raised.
//
// Hand-over protocol.  A flag holding anything but this launch's tag or tag | kSkAbandoned means
// "not published" (the workspace is never zeroed: a fresh one holds arbitrary bits, a reused one
// whatever earlier launches left):
//   producer: partial stored, then the flag swapped from its current value to tag -- unless it
//             reads tag | kSkAbandoned, i.e. the owner has given up on the piece: then it resets the
//             flag to 0.
//   owner:    waits (bounded) for flag == tag, then takes the partial and resets the flag to 0.  When
//             the wait expires it swaps the flag from its current value to tag | kSkAbandoned and
//             computes the piece itself -- unless it reads tag, i.e. the partial arrived meanwhile:
//             then it takes it as usual.
// Both swaps are compare-and-swaps on the value just read; apart from the owner's final reset, each
// side writes the flag at most once, so a failed swap means the other side's swap came first.
// Exactly one side wins: a piece is never dropped nor counted twice, a late producer never leaves a raised flag behind (a replay
// of a captured launch reuses its tag), and the result does not depend on every workgroup of the
// grid being resident at once.
// A wait bound of 0 turns the hand-over off: producers do not publish and owners compute every
// piece themselves, touching no flag (a host-side test setting that exercises the owners' path).
// First step of workgroup g's share.
__device__ __forceinline__ long sk_begin(long S, int g, int G) { return S * g / G; }

constexpr unsigned kSkAbandoned = 1u << 31;   // launch tags stay below 2^31
constexpr int kCachePolicySc1 = 16;      // cache-policy operand of the buffer builtins: sc1
// A partial slot (workgroup-uniform base) as a raw buffer; offsets in bytes: a per-lane part `off`
// and a uniform part `soff` (a constant in a scalar register; per-lane offsets are then one VGPR for
// a whole tile's accesses).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_slot(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void sk_store(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff, float a, float b,
                                         float c, float d) {
    const u32x4_v v = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, soff, kCachePolicySc1);
}
__device__ __forceinline__ float4 sk_load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    const u32x4_v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kCachePolicySc1);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}
// Publish: every thread's partial stores acknowledged, then thread 0 raises the flag (or, if the
// owner has given up on the piece, resets it).
__device__ __forceinline__ void sk_raise(unsigned* flag, unsigned tag, int spins) {
    if (spins == 0) return;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v == (tag | kSkAbandoned) ||
            !__hip_atomic_compare_exchange_strong(flag, &v, tag, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT))
            __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);     // the owner gave up
    }
}
// Take (every thread of the workgroup calls it): true = the piece's partial is published and may be
// read (the flag is reset already: the partial stays in place until this launch ends); false = the
// owner claimed the piece and computes it itself.  `spins` bounds the wait (0: give up at once).
// Thread 0 decides; the rest of the workgroup reads the decision from the flag itself between two
// barriers (tag: taken; anything else: claimed -- after a claim only the producer writes the flag,
// and only from tag | kSkAbandoned to 0).  The kernels avoid plain LDS stores (an LDS broadcast here
// would make the compiler wait for every in-flight global -> LDS load before any LDS read).
__device__ __forceinline__ bool sk_take(unsigned* flag, unsigned tag, int spins) {
    if (spins == 0) return false;
    if (threadIdx.x == 0) {
        bool got = false;
        for (int spin = 0;; ++spin) {
            if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag) { got = true; break; }
            if (spin >= spins) break;
            __builtin_amdgcn_s_sleep(2);
        }
        if (!got) {
            // claim the piece, unless the producer published in between (the swap then fails)
            unsigned v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (v != tag)
                __hip_atomic_compare_exchange_strong(flag, &v, tag | kSkAbandoned, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    // workgroup-uniform; readfirstlane tells the compiler so (a branch on it stays scalar)
    const bool ok = __builtin_amdgcn_readfirstlane(
                        (int)(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag)) != 0;
    __syncthreads();
    if (ok && threadIdx.x == 0) __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return ok;
}

}  // namespace dit
