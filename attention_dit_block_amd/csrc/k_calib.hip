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


// ------------------------------------------------------------------------------------------
// Schedule probes: the inner loops of the GEMM and attention kernels on LDS-resident operands,
// so that their rates separate what the instruction schedule reaches from what the global loads
// and the epilogues cost.  Every staged fp16 element is 2^-6 (0x2400), which makes the results
// closed forms the tests check.
// ------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void calib_lds_void;
constexpr uint32_t kHalf2Pow6 = 0x24002400u;      // two fp16 2^-6

// 16 bytes of staged operand number i: eight fp16 2^-6, or (rnd) eight hashed fp16 values of random
// sign, magnitude in [2^-6, 2^-2), so that the matrix cores switch realistic bit patterns (constant
// operands let the chip hold a higher clock)
__device__ __forceinline__ u32x4_v calib_fill(int i, int rnd) {
    if (!rnd) return u32x4_v{kHalf2Pow6, kHalf2Pow6, kHalf2Pow6, kHalf2Pow6};
    u32x4_v w;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t h = (uint32_t)(4 * i + t) * 2654435761u;
        h ^= h >> 13;
        h *= 0x5bd1e995u;
        h ^= h >> 15;
        const uint32_t a = ((h & 1u) << 15) | ((9u + ((h >> 1) & 3u)) << 10) | ((h >> 3) & 0x3ffu);
        const uint32_t b = (((h >> 13) & 1u) << 15) | ((9u + ((h >> 14) & 3u)) << 10) | ((h >> 16) & 0x3ffu);
        w[t] = a | (b << 16);
    }
    return w;
}

__device__ __forceinline__ void calib_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// The GEMM's 256 x 256 x 64 k-step: 8 waves of 128 x 64 sub-tiles (2 along M, 4 along N), fragments
// read from two 64 KB stages laid out as the GEMM lays them out (rows of 128 B, 16-byte chunk XOR
// (row >> 1) & 7), v_mfma_f32_32x32x16_f16.  MODE bit 0: ping-pong schedule (the two waves of a SIMD
// alternate 32-deep fragment-read phases and 16-MFMA phases a phase apart, a barrier per phase, the
// MFMA phase at raised wave priority) instead of the kernel's interleaved one (each k16 sub-step's
// MFMAs beside the next sub-step's reads, a barrier per k-step).  Bit 1: also load each k-step's
// 64 KB global -> LDS (8 KB per wave) from a 4 MiB window of 2^-6 values, as the GEMM does.  Bit 3:
// the fragments are read once before the loop and the MFMAs run on them from registers (the
// matrix cores' rate in this layout, without LDS).
// out[w * 512 + t] = the sum of thread t's 128 accumulators = 2 * ksteps.
template <int MODE>
__global__ __launch_bounds__(512, 1) void gemm_kloop_kernel(int n, const char* win, float* out, int rnd) {
    __shared__ __attribute__((aligned(1024))) char smem[131072];
    constexpr bool PP = MODE & 1, GL = (MODE & 2) != 0, REGS = (MODE & 8) != 0;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / 4, wn = wave % 4, khalf = lane >> 5;
    for (int i = tid; i < 131072 / 16; i += 512) reinterpret_cast<u32x4_v*>(smem)[i] = calib_fill(i, rnd);
    __syncthreads();
    int a_row[4], b_row[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) a_row[j] = wm * 128 + j * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < 2; ++j) b_row[j] = wn * 64 + j * 32 + (lane & 31);
    f32x16_v acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    f16x8_v fa[2][4], fb[2][2];
    auto rd = [&](f16x8_v* a, f16x8_v* b, int base, int s) {
        const int c = 2 * s + khalf;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            a[j] = *reinterpret_cast<const f16x8_v*>(smem + base + a_row[j] * 128 + ((c ^ ((a_row[j] >> 1) & 7)) << 4));
#pragma unroll
        for (int j = 0; j < 2; ++j)
            b[j] = *reinterpret_cast<const f16x8_v*>(smem + base + 32768 + b_row[j] * 128 +
                                                      ((c ^ ((b_row[j] >> 1) & 7)) << 4));
    };
    // this wave's load i (of 8) of k-step t's stage: 1 KB from the window (offsets wrap at 4 MiB)
    auto gl = [&](int t, int i) {
        const size_t off = ((size_t)((t * 64 + wave * 8 + i) & 4095) << 10) + lane * 16;
        __builtin_amdgcn_global_load_lds(win + off, (calib_lds_void*)(smem + (t & 1) * 65536 + (wave * 8 + i) * 1024),
                                         16, 0, 0);
    };
    auto mfmas = [&](int s) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[s][nb], fa[s][mb], acc[nb][mb], 0, 0, 0);
    };
    if constexpr (REGS) {
        rd(fa[0], fb[0], 0, 0);
        rd(fa[1], fb[1], 0, 1);
    }
    if constexpr (!PP) {
        if constexpr (!REGS) rd(fa[0], fb[0], 0, 0);
        for (int t = 0; t < n; ++t) {
            const int base = (t & 1) * 65536;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int cur = s & 1;
                if (!REGS && s < 3) rd(fa[cur ^ 1], fb[cur ^ 1], base, s + 1);
                if (GL && s == 0 && t + 1 < n)
#pragma unroll
                    for (int i = 0; i < 8; ++i) gl(t + 1, i);
                mfmas(cur);
                if (s < 3) {
#pragma unroll
                    for (int i = 0; i < 6; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        if (GL && s == 0) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (!REGS) rd(fa[0], fb[0], ((t + 1) & 1) * 65536, 0);
        }
    } else {
        // group 0 (waves 0-3) reads half h while group 1 (waves 4-7, one per SIMD beside them)
        // runs the MFMAs of its previous half, then the other way round
        auto mph = [&](int t, int h) {
            if (!REGS) {
                rd(fa[0], fb[0], (t & 1) * 65536, 2 * h);
                rd(fa[1], fb[1], (t & 1) * 65536, 2 * h + 1);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0)
        };
        auto cph = [&]() {
            __builtin_amdgcn_s_setprio(1);
            mfmas(0);
            mfmas(1);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
        };
        if (wm == 1) calib_barrier();
        for (int t = 0; t < n; ++t) {
            mph(t, 0);
            if (GL && t + 1 < n)
#pragma unroll
                for (int i = 0; i < 8; ++i) gl(t + 1, i);
            calib_barrier();
            cph();
            calib_barrier();
            mph(t, 1);
            calib_barrier();
            cph();
            if (GL) __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): k-step t + 1 has landed
            if (wm == 0 || t < n - 1) calib_barrier();
        }
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) sum += acc[i][j][q];
    out[(size_t)blockIdx.x * 512 + tid] = sum;
}

// The 16-bit attention kernel's step on LDS-resident K and V: 8 waves of 32 queries, 64-key
// tiles, d = 128; per tile and wave 16 score MFMAs (S^T = K Q^T), 32 exponentials of
// fma(s, c2, -1) with their row sum and fp16 packing, a rarely taken branch (the lazy-max test), 16
// PV MFMAs.  MODE 0: the kernel's order (scores of tile j + 1, softmax of tile j, the branch, PV of
// tile j; a barrier per tile).  MODE 1: the two waves of a SIMD half a tile apart (an MFMA phase:
// scores j + 1 and PV j, at raised priority; a softmax phase), a barrier per phase.  With c2 = 0
// every probability is 1/2 and out[w * 512 + t] = 48 * tiles (+ 16 in MODE 1, one more softmax).
template <int MODE>
__global__ __launch_bounds__(512, 2) void attention_step_kernel(int n, float c2, float* out, int rnd) {
    // 96 KB so that, like the kernel it stands for, one workgroup holds a CU (64 KB are used)
    __shared__ __attribute__((aligned(1024))) char smem[98304];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i < 65536 / 16; i += 512) reinterpret_cast<u32x4_v*>(smem)[i] = calib_fill(i, rnd);
    __syncthreads();
    f16x8_v qf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const u32x4_v w = calib_fill(4096 + 64 * i + lane, rnd);
        qf[i] = __builtin_bit_cast(f16x8_v, w);
    }
    f32x16_v o[4], S[2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) o[i][q] = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) S[i][q] = 0.0f;
    uint32_t ph[16];
    float lsum = 0.0f;
    const float nm = -1.0f;
    auto scores = [&](int slot) {
        const char* kt = smem + slot * 16384;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int es = 0; es < 8; ++es) {
                const f16x8_v kf = *reinterpret_cast<const f16x8_v*>(kt + (es * 2 + kb) * 1024 + lane * 16);
                S[kb] = es == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[es], f32x16_v{}, 0, 0, 0)
                                : __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[es], S[kb], 0, 0, 0);
            }
    };
    auto softmax = [&]() {
        float ls = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 16; q += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(S[kb][q], c2, nm));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(S[kb][q + 1], c2, nm));
                ls += p0 + p1;
                ph[8 * kb + (q >> 1)] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p0, p1));
            }
        lsum += ls;
    };
    auto rare = [&]() {
        if (__builtin_amdgcn_ballot_w64(lsum > 1e30f)) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 16; ++q) o[i][q] *= 0.5f;
        }
    };
    auto pv = [&](int slot) {
        const char* vt = smem + 32768 + slot * 16384;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4_v hv = {ph[4 * ks], ph[4 * ks + 1], ph[4 * ks + 2], ph[4 * ks + 3]};
#pragma unroll
            for (int eb = 0; eb < 4; ++eb) {
                const f16x8_v vf = *reinterpret_cast<const f16x8_v*>(vt + (ks * 4 + eb) * 1024 + lane * 16);
                o[eb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, __builtin_bit_cast(f16x8_v, hv), o[eb], 0, 0, 0);
            }
        }
    };
    scores(0);
    if constexpr (MODE == 0) {
        for (int j = 0; j < n; ++j) {
            const f32x16_v c0 = S[0], c1 = S[1];
            scores((j + 1) & 1);
            const f32x16_v n0 = S[0], n1 = S[1];
            S[0] = c0;
            S[1] = c1;
            softmax();
            rare();
            S[0] = n0;
            S[1] = n1;
            pv(j & 1);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    } else {
        softmax();
        if (wave >= 4) calib_barrier();
        for (int j = 0; j < n; ++j) {
            __builtin_amdgcn_s_setprio(1);
            scores((j + 1) & 1);
            pv(j & 1);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
            calib_barrier();
            softmax();
            rare();
            if (wave < 4 || j < n - 1) calib_barrier();
        }
    }
    float sum = lsum;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) sum += o[i][q];
    out[(size_t)blockIdx.x * 512 + tid] = sum;
}

hipError_t launch_gemm_kloop_probe(int mode, int workgroups, int ksteps, const void* win, float* out, hipStream_t s) {
    const char* w = reinterpret_cast<const char*>(win);
    const int rnd = (mode >> 2) & 1;
    switch (mode & 11) {
    case 0: hipLaunchKernelGGL(gemm_kloop_kernel<0>, dim3(workgroups), dim3(512), 0, s, ksteps, w, out, rnd); break;
    case 1: hipLaunchKernelGGL(gemm_kloop_kernel<1>, dim3(workgroups), dim3(512), 0, s, ksteps, w, out, rnd); break;
    case 2: hipLaunchKernelGGL(gemm_kloop_kernel<2>, dim3(workgroups), dim3(512), 0, s, ksteps, w, out, rnd); break;
    case 3: hipLaunchKernelGGL(gemm_kloop_kernel<3>, dim3(workgroups), dim3(512), 0, s, ksteps, w, out, rnd); break;
    case 8: hipLaunchKernelGGL(gemm_kloop_kernel<8>, dim3(workgroups), dim3(512), 0, s, ksteps, w, out, rnd); break;
    default: hipLaunchKernelGGL(gemm_kloop_kernel<9>, dim3(workgroups), dim3(512), 0, s, ksteps, w, out, rnd); break;
    }
    return hipGetLastError();
}

hipError_t launch_attention_step_probe(int mode, int workgroups, int tiles, float c2, float* out, hipStream_t s) {
    const int rnd = (mode >> 1) & 1;
    if ((mode & 1) == 0) hipLaunchKernelGGL(attention_step_kernel<0>, dim3(workgroups), dim3(512), 0, s, tiles, c2, out, rnd);
    else hipLaunchKernelGGL(attention_step_kernel<1>, dim3(workgroups), dim3(512), 0, s, tiles, c2, out, rnd);
    return hipGetLastError();
}

}  // namespace dit
