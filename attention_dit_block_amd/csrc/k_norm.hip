// HBM-bound per-token kernels of the DiT block on gfx950:
//  * adaln_gemv   -- AdaLN modulation vectors m = W_mod . SiLU(c)
//  * modulate     -- (1 + scale) * RMSNorm(x) + shift, one wave per row
//  * qk_norm_rope -- per-head RMSNorm of q and k, then 4-axis RoPE, in place
// (the custom RMSNorm / RoPE / AdaLN-modulation / activation kernels of the
// "CUDA codepath !" thread, antirez/iris.c issue #15; RoPE axes from its GGML
// update, item 3).
#include "dev_common.h"
#include "launch.h"

namespace dit {

// ------------------------------------------------------------------------------------------
// AdaLN GEMV.  Each wave owns 4 consecutive output rows; each lane streams 16-byte slices of
// those rows and multiplies them with SiLU(cond), which the block stages in LDS as fp32.
// Bound: HBM bytes of W (rows * d_cond * sizeof(T)).
// ------------------------------------------------------------------------------------------
constexpr int kGemvRowsPerWave = 4;
constexpr int kGemvWaves = 4;

template <int DT>
__global__ __launch_bounds__(256) void adaln_gemv_kernel(GemvBatch b) {
    extern __shared__ float s_act[];
    constexpr int kES = ESize<DT>::v;
    if (b.clear_flag && blockIdx.x == 0 && threadIdx.x == 0) *b.clear_flag = 0u;
    constexpr int kElems = 16 / kES;                       // elements per 16-byte slice
    constexpr int kQ = kElems / 4;                         // float4s of SiLU(c) per slice
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int total = b.p[0].rows + (b.n > 1 ? b.p[1].rows : 0);
    const int row0 = (blockIdx.x * kGemvWaves + wave) * kGemvRowsPerWave;
    const char* wrow[kGemvRowsPerWave];
    float acc[kGemvRowsPerWave];
    bool ok[kGemvRowsPerWave];
#pragma unroll
    for (int r = 0; r < kGemvRowsPerWave; ++r) {
        const int g = row0 + r;
        ok[r] = g < total;
        int pi = (g >= b.p[0].rows) ? 1 : 0;
        int lr = g - (pi ? b.p[0].rows : 0);
        if (!ok[r]) { pi = 0; lr = 0; }
        wrow[r] = reinterpret_cast<const char*>(b.p[pi].w) + (size_t)lr * b.d_cond * kES;
        acc[r] = 0.0f;
    }
    // slices of 64 lanes x kElems elements; the next slice's weights load while this one is summed
    // (nontemporal: every weight is read once)
    const int iters = (b.d_cond + 64 * kElems - 1) / (64 * kElems);
    u32x4_v w[kGemvRowsPerWave], wn[kGemvRowsPerWave];
    // (loads clamped into the row, d_cond >= 8 and a multiple of 8; a lane past the row's end skips
    // the sums below.  Loaded under a per-lane branch or zeroed right after, each slice waited for
    // its loads at once, and the next slice's loads no longer overlapped this one's sums.)
    auto load = [&](u32x4_v* dst, int it) {
        const int kc = min((it * 64 + lane) * kElems, b.d_cond - kElems);
#pragma unroll
        for (int r = 0; r < kGemvRowsPerWave; ++r)
            dst[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_v*>(wrow[r] + (size_t)kc * kES));
    };
    load(w, 0);       // the first slice's HBM latency overlaps the SiLU(c) staging below
    // SiLU(c) in LDS, interleaved so that the float4s a lane needs for one slice sit 16 bytes
    // apart across lanes (bank-conflict-free reads): element e = (it * 64 + l) * kElems + 4 q + j
    // goes to ((it * kQ + q) * 64 + l) * 4 + j.  Staged 4 elements per thread per step, all of a
    // pass's loads issued before the first SiLU.
    for (int base = 0; base < b.d_cond; base += 4 * 1024) {
        float cv[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = base + (tid + 256 * r) * 4;
            if (e < b.d_cond) {
                if constexpr (DT == BF16) {
                    const u32x2_v w = *reinterpret_cast<const u32x2_v*>(reinterpret_cast<const bf16_t*>(b.cond) + e);
                    cv[r][0] = bf_lo(w[0]); cv[r][1] = bf_hi(w[0]); cv[r][2] = bf_lo(w[1]); cv[r][3] = bf_hi(w[1]);
                } else {
                    const f32x4_v w = ldf4(reinterpret_cast<const float*>(b.cond) + e);
#pragma unroll
                    for (int j = 0; j < 4; ++j) cv[r][j] = w[j];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = base + (tid + 256 * r) * 4;
            if (e < b.d_cond) {
                const int slice = e / kElems, q = (e - slice * kElems) >> 2;
                const int it = slice >> 6, l = slice & 63;
                f32x4_v o;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = cv[r][j] / (1.0f + expf(-cv[r][j]));
                stf4(s_act + ((it * kQ + q) * 64 + l) * 4, o);
            }
        }
    }
    __syncthreads();

    auto sums = [&](const u32x4_v* wv, int it) {
        const int k0 = (it * 64 + lane) * kElems;
        if (k0 < b.d_cond) {
            float sa[8];
#pragma unroll
            for (int q = 0; q < kQ; ++q) {
                const f32x4_v v = ldf4(s_act + ((it * kQ + q) * 64 + lane) * 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) sa[4 * q + j] = v[j];
            }
#pragma unroll
            for (int r = 0; r < kGemvRowsPerWave; ++r) {
                if (DT == BF16) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        acc[r] = fmaf(bf_lo(wv[r][t]), sa[2 * t], acc[r]);
                        acc[r] = fmaf(bf_hi(wv[r][t]), sa[2 * t + 1], acc[r]);
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) acc[r] = fmaf(__uint_as_float(wv[r][t]), sa[t], acc[r]);
                }
            }
        }
    };
    // Two buffers in alternating roles, and no load under a branch inside the loop: a copy from the
    // prefetch buffer into the working one at the end of each slice, or a conditional prefetch
    // (whose two paths leave different loads outstanding), made every slice wait for the next
    // slice's loads.
    int it = 0;
    for (; it + 2 < iters; it += 2) {
        load(wn, it + 1);
        sums(w, it);
        load(w, it + 2);
        sums(wn, it + 1);
    }
    if (it + 1 < iters) {
        load(wn, it + 1);
        sums(w, it);
        sums(wn, it + 1);
    } else {
        sums(w, it);
    }
#pragma unroll
    for (int r = 0; r < kGemvRowsPerWave; ++r) {
        const float s = wave_sum(acc[r]);
        const int g = row0 + r;
        if (lane == 0 && ok[r]) {
            const int pi = (g >= b.p[0].rows) ? 1 : 0;
            b.p[pi].out[g - (pi ? b.p[0].rows : 0)] = s;
        }
    }
}

hipError_t launch_adaln_gemv(const GemvBatch& b, hipStream_t s) {
    const int total = b.p[0].rows + (b.n > 1 ? b.p[1].rows : 0);
    const int per_block = kGemvWaves * kGemvRowsPerWave;
    const dim3 grid((total + per_block - 1) / per_block);
    // SiLU(c), rounded up to whole 64-lane slices (the interleaved layout spans them)
    const int slice = 64 * (b.dtype == BF16 ? 8 : 4);
    const size_t lds = (size_t)((b.d_cond + slice - 1) / slice) * slice * sizeof(float);
    if (b.dtype == BF16)
        hipLaunchKernelGGL(adaln_gemv_kernel<BF16>, grid, dim3(256), lds, s, b);
    else
        hipLaunchKernelGGL(adaln_gemv_kernel<F32>, grid, dim3(256), lds, s, b);
    return hipGetLastError();
}

// Entry i = token * 64 + pair of the rotation-angle table: the angle in revolutions reduced in double
// precision, then the hardware cosine and sine (the QK RMSNorm + RoPE pass's angle arithmetic).
__device__ __forceinline__ void rope_table_entry(const int32_t* pos, int n_axes, const RopeTable& tab, float* cs,
                                                 long i) {
    const int tok = (int)(i >> 6), p = (int)(i & 63);
    const double inv_two_pi = 0.15915494309189533576888376337251;
    const double rev = (double)pos[(size_t)tok * n_axes + tab.axis[p]] * tab.omega_d[p] * inv_two_pi;
    const float fr = (float)(rev - rint(rev));
    *reinterpret_cast<f32x2_v*>(cs + 2 * i) = f32x2_v{__builtin_amdgcn_cosf(fr), __builtin_amdgcn_sinf(fr)};
}

// ------------------------------------------------------------------------------------------
// Modulate: out = (1 + scale) * x * rstd + shift with rstd = 1/sqrt(mean(x^2) + eps).
// One wave per row, four rows per workgroup, the row kept in registers between the reduction and
// the write.  Workgroups are laid out per problem (text rows, then image rows), and each stages
// its problem's shift and scale vectors in LDS once for its four rows: read per row from L2 they
// would be twice the row's own HBM bytes, and kept in registers they would cap occupancy.  On
// request the grid also writes the RoPE angle table of the QKV product's fused QK RMSNorm + RoPE,
// one entry per thread.
// Bound: HBM bytes  rows * d * (sizeof(x) + sizeof(out)) (+ 512 per row with the table).
// ------------------------------------------------------------------------------------------
template <int XT, int OT, int NC>
__global__ __launch_bounds__(256) void modulate_kernel(ModBatch b) {
    extern __shared__ float s_mod[];               // shift [d], then scale [d]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (b.clear && blockIdx.x == 0)
        for (int i = threadIdx.x; i < b.clear_n; i += 256) b.clear[i] = 0u;
    if (b.rope_cs) {
        // the QKV product's rotation table, one entry per thread (its own launch cost as much as
        // computing it here)
        const long i = (long)blockIdx.x * 256 + threadIdx.x;
        if (i < (long)b.rope_n * 64) rope_table_entry(b.rope_pos, b.rope_n_axes, b.rope_tab, b.rope_cs, i);
    }
    const int nb0 = (b.p[0].rows + 3) / 4;         // workgroups of problem 0
    const int pi = (b.n > 1 && (int)blockIdx.x >= nb0) ? 1 : 0;
    const ModProblem& P = b.p[pi];
    const int r = ((int)blockIdx.x - (pi ? nb0 : 0)) * 4 + wave;
    const bool active = r < P.rows;                // wave-uniform
    const int d = b.d;
    const char* xrow = reinterpret_cast<const char*>(P.x) + (size_t)min(r, P.rows - 1) * P.ld_x * ESize<XT>::v;
    char* orow = reinterpret_cast<char*>(P.out) + (size_t)r * P.ld_out * ESize<OT>::v;

    // every chunk's load issued unconditionally (column clamped into the row, d >= 8 and a multiple
    // of 8; rows past the problem read its last row), chunks past d zeroed after the loads: a load
    // under a per-chunk branch waited at the branch's join, one round trip per chunk
    float v[NC][8];
#pragma unroll
    for (int i = 0; i < NC; ++i)
        load8<XT>(xrow + (size_t)min((lane + 64 * i) * 8, d - 8) * ESize<XT>::v, v[i]);
#pragma unroll
    for (int i = 0; i < NC; ++i)
        if ((lane + 64 * i) * 8 >= d) {
#pragma unroll
            for (int t = 0; t < 8; ++t) v[i][t] = 0.0f;
        }
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
        stf4(s_mod + c, ldf4(P.shift + c));
        stf4(s_mod + d + c, ldf4(P.scale + c));
    }
    __syncthreads();
    if (!active) return;
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
        for (int t = 0; t < 8; ++t) ss = fmaf(v[i][t], v[i][t], ss);
    ss = wave_sum(ss);
    const float rstd = 1.0f / sqrtf(ss / (float)d + b.eps);
    if constexpr (OT == FP8_ROWS) {
        // e4m3 output: the modulated row stays in registers for its max, then s = max / 448 and
        // codes of v / s (both divisions correctly rounded, round-to-nearest-even conversion)
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = min((lane + 64 * i) * 8, d - 8);
            const f32x4_v sh0 = ldf4(s_mod + c), sh1 = ldf4(s_mod + c + 4);
            const f32x4_v sc0 = ldf4(s_mod + d + c), sc1 = ldf4(s_mod + d + c + 4);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float shv = t < 4 ? sh0[t] : sh1[t - 4], scv = t < 4 ? sc0[t] : sc1[t - 4];
                v[i][t] = fmaf(1.0f + scv, v[i][t] * rstd, shv);
                if ((lane + 64 * i) * 8 < d) amax = fmaxf(amax, fabsf(v[i][t]));
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
        const float qs = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
        if (lane == 0) P.out_scale[r] = qs;
        // v / qs through the double reciprocal of qs: the double product is within 2^-52 of the
        // quotient, which lies more than 2^-49 from any fp32 rounding midpoint in the normal range,
        // so it rounds to the correctly rounded quotient (three instructions instead of ten)
        const double rq = 1.0 / (double)qs;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = (lane + 64 * i) * 8;
            if (c < d) {
                float y[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) y[t] = (float)((double)v[i][t] * rq);
                int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
                w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
                int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
                w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
                *reinterpret_cast<u32x2_v*>(orow + c) = u32x2_v{(uint32_t)w0, (uint32_t)w1};
            }
        }
        return;
    }
    bool bad = false;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = (lane + 64 * i) * 8;
        if (c < d) {
            const f32x4_v sh0 = ldf4(s_mod + c), sh1 = ldf4(s_mod + c + 4);
            const f32x4_v sc0 = ldf4(s_mod + d + c), sc1 = ldf4(s_mod + d + c + 4);
            float o[8];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                o[t] = fmaf(1.0f + sc0[t], v[i][t] * rstd, sh0[t]);
                o[4 + t] = fmaf(1.0f + sc1[t], v[i][4 + t] * rstd, sh1[t]);
            }
            if constexpr (OT == F16) {
#pragma unroll
                for (int t = 0; t < 8; ++t) bad |= f16_out_of_range(o[t]);
            }
            store8<OT>(orow + (size_t)c * ESize<OT>::v, o);
        }
    }
    if constexpr (OT == F16) raise_range_flag(b.range_flag, bad);
}

template <int XT, int OT>
static hipError_t launch_mod_nc(const ModBatch& b, hipStream_t s, dim3 grid) {
    const int nc = (b.d + 511) / 512;
    const size_t lds = (size_t)2 * b.d * sizeof(float);
    if (nc <= 2) hipLaunchKernelGGL((modulate_kernel<XT, OT, 2>), grid, dim3(256), lds, s, b);
    else if (nc <= 4) hipLaunchKernelGGL((modulate_kernel<XT, OT, 4>), grid, dim3(256), lds, s, b);
    else if (nc <= 6) hipLaunchKernelGGL((modulate_kernel<XT, OT, 6>), grid, dim3(256), lds, s, b);
    else if (nc <= 8) hipLaunchKernelGGL((modulate_kernel<XT, OT, 8>), grid, dim3(256), lds, s, b);
    else hipLaunchKernelGGL((modulate_kernel<XT, OT, 16>), grid, dim3(256), lds, s, b);
    return hipGetLastError();
}

template <int XT>
static hipError_t launch_mod_x(const ModBatch& b, hipStream_t s, dim3 grid) {
    if (b.out_dtype == FP8_ROWS) return launch_mod_nc<XT, FP8_ROWS>(b, s, grid);
    if (b.out_dtype == F16) return launch_mod_nc<XT, F16>(b, s, grid);
    if (b.out_dtype == BF16) return launch_mod_nc<XT, BF16>(b, s, grid);
    return launch_mod_nc<XT, F32>(b, s, grid);
}

hipError_t launch_modulate(const ModBatch& b, hipStream_t s) {
    // four rows per workgroup, each problem's rows in workgroups of their own
    const dim3 grid((b.p[0].rows + 3) / 4 + (b.n > 1 ? (b.p[1].rows + 3) / 4 : 0));
    if (grid.x == 0) return hipSuccess;
    // All problems of one batch share x_dtype (the caller builds them so).
    return b.p[0].x_dtype == BF16 ? launch_mod_x<BF16>(b, s, grid) : launch_mod_x<F32>(b, s, grid);
}

// ------------------------------------------------------------------------------------------
// QK RMSNorm + 4-axis RoPE, in place.  One 256-thread block per token: the first wave computes
// the token's 64 rotation angles once (double-precision angle reduced in revolutions, hardware sin/cos)
// into LDS; then groups of 16 lanes each take one 128-dim head vector of q or k (16 B per lane
// for 16-bit types), reduce its mean square across the 16 lanes, scale by the QK-norm weight
// and rotate the four interleaved pairs they hold.
// Bound: HBM bytes  n_tok * 2 * n_heads * 128 * sizeof(T) read + the same written.
// ------------------------------------------------------------------------------------------
template <int DT, int WT>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(QkRopeArgs a) {
    __shared__ float s_cos[64], s_sin[64];
    const int n = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid < 64) {
        // the angle in revolutions, reduced to [-1/2, 1/2] in double precision, then the hardware
        // sine and cosine (v_sin_f32 / v_cos_f32 take revolutions), whose small absolute error stays
        // far below a 16-bit result's rounding (the parity tests hold the results to 0.6 ulp)
        const int ax = a.tab.axis[tid];
        const double inv_two_pi = 0.15915494309189533576888376337251;
        const double rev = (double)a.pos[(size_t)n * a.n_axes + ax] * a.tab.omega_d[tid] * inv_two_pi;
        const float fr = (float)(rev - rint(rev));
        s_cos[tid] = __builtin_amdgcn_cosf(fr);
        s_sin[tid] = __builtin_amdgcn_sinf(fr);
    }
    __syncthreads();
    const int set = n < a.n_first ? 0 : 1;
    const int g = tid >> 4;           // 16 groups of 16 lanes
    const int t = tid & 15;           // dims 8t .. 8t+7 of the head
    constexpr int ES = ESize<DT>::v, WS = ESize<WT>::v;
    for (int vec = g; vec < 2 * a.n_heads; vec += 16) {
        const int which = vec >= a.n_heads ? 1 : 0;
        const int h = vec - which * a.n_heads;
        char* base = which ? reinterpret_cast<char*>(a.k) + (size_t)n * a.ld_k * ES
                           : reinterpret_cast<char*>(a.q) + (size_t)n * a.ld_q * ES;
        char* p = base + (size_t)(h * 128 + t * 8) * ES;
        const char* wp = reinterpret_cast<const char*>(set ? a.qk_w1 : a.qk_w0) + (size_t)(which * 128 + t * 8) * WS;
        float v[8], w[8];
        load8<DT>(p, v);
        load8<WT>(wp, w);
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
        ss = row16_sum(ss);
        const float rstd = __builtin_amdgcn_rsqf(ss * (1.0f / 128.0f) + a.eps);
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = v[i] * rstd * w[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float c = s_cos[4 * t + i], s = s_sin[4 * t + i];
            const float u0 = y[2 * i], u1 = y[2 * i + 1];
            y[2 * i] = u0 * c - u1 * s;
            y[2 * i + 1] = u0 * s + u1 * c;
        }
        store8<DT>(p, y);
    }
}

// e4m3 variant for the attention of the fp8 blocks: the same norm and rotation of q and k, then
// codes instead of the rotated values -- q per (token, head) with s = max|y| / 448 (1 for a zero
// row), k per head with the static scale max|w_k| * sqrt(128) / 448 (a normed, rotated element never
// exceeds sqrt(128) times the largest weight), v per head with s = max|v| / 448 from the maxima the
// QKV epilogue raised; codes e4m3(y / s) of the correctly rounded fp32 quotient, nearest-even
// conversion.
constexpr float kKBound = 0x1.9dc22cp-6f;   // sqrt(128) / 448 rounded to fp32

template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

// x / s correctly rounded to fp32, from r = 1 / (double)s (correctly rounded): the double product
// x * r is within 2^-52 (relative) of x / s, while a quotient of two fp32 values in the normal range
// lies more than 2^-49 (relative) from every midpoint between neighbouring fp32 values, so the
// product rounds to the same fp32 value as the quotient.  (Quotients below the normal range are far
// below e4m3's smallest step and give the same zero code either way.)  Three instructions instead of
// the division's ten.
__device__ __forceinline__ float div_by_rcp(float x, double r) { return (float)((double)x * r); }

template <int DT, int WT>
__global__ __launch_bounds__(256) void qk_norm_rope_fp8_kernel(QkRopeArgs a) {
    __shared__ float s_cos[64], s_sin[64], s_kw[4];
    __shared__ double s_rv[256];        // 1 / (double)(v scale) per head
    constexpr int ES = ESize<DT>::v, WS = ESize<WT>::v;
    const int n = blockIdx.x;
    const int tid = threadIdx.x;
    const int H = a.n_heads;
    const int set = n < a.n_first ? 0 : 1;
    const int g = tid >> 4;           // 16 groups of 16 lanes
    const int t = tid & 15;           // dims 8t .. 8t+7 of the head
    // this lane's dims of the q- and k-norm weights
    float wq[8], wk[8];
    {
        const char* wrow = reinterpret_cast<const char*>(set ? a.qk_w1 : a.qk_w0);
        load8<WT>(wrow + (size_t)(t * 8) * WS, wq);
        load8<WT>(wrow + (size_t)(128 + t * 8) * WS, wk);
    }
    if (tid < 64) {
        // the angle in revolutions reduced in double precision, hardware sine and cosine (as in
        // the 16-bit pass)
        const int ax = a.tab.axis[tid];
        const double inv_two_pi = 0.15915494309189533576888376337251;
        const double rev = (double)a.pos[(size_t)n * a.n_axes + ax] * a.tab.omega_d[tid] * inv_two_pi;
        const float fr = (float)(rev - rint(rev));
        s_cos[tid] = __builtin_amdgcn_cosf(fr);
        s_sin[tid] = __builtin_amdgcn_sinf(fr);
    }
    {
        // the largest |k weight| of both sets: thread tid reads dim tid % 128 of set tid / 128
        const char* wkp = reinterpret_cast<const char*>(tid < 128 ? a.qk_w0 : a.qk_w1);
        float wv = 0.0f;
        if (wkp) {
            float w8[8];
            load8<WT>(wkp + (size_t)(128 + (tid & 127 & ~7)) * WS, w8);
            wv = fabsf(w8[tid & 7]);
        }
        wv = group_max<64>(wv);
        if ((tid & 63) == 0) s_kw[tid >> 6] = wv;
    }
    if (tid < H) {
        const float m = __uint_as_float(a.vmax[tid]);
        const float sv = m > 0.0f ? m / 448.0f : 1.0f;
        s_rv[tid] = 1.0 / (double)sv;
        if (n == 0) a.sv[tid] = sv;
    }
    __syncthreads();
    const float s_k = fmaxf(fmaxf(s_kw[0], s_kw[1]), fmaxf(s_kw[2], s_kw[3])) * kKBound;
    const double r_k = 1.0 / (double)s_k;
    if (n == 0 && tid < H) a.sk[tid] = s_k;
    const char* rows[3] = {reinterpret_cast<const char*>(a.q) + (size_t)n * a.ld_q * ES,
                           reinterpret_cast<const char*>(a.k) + (size_t)n * a.ld_k * ES,
                           reinterpret_cast<const char*>(a.v) + (size_t)n * a.ld_v * ES};
    uint8_t* dst_row = a.qkv8 + (size_t)n * a.ld8;
    // vectors g, g + 16, ... of the token's 3H (q heads, then k heads, then v heads), as (which, h)
    int which = 0, h = g;
    while (which < 3 && h >= H) { h -= H; ++which; }
    while (which < 3) {
        float y[8];
        load8<DT>(rows[which] + (size_t)(h * 128 + t * 8) * ES, y);
        double r;
        if (which < 2) {
            float ss = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fmaf(y[i], y[i], ss);
            ss = row16_sum(ss);
            const float rstd = __builtin_amdgcn_rsqf(ss * (1.0f / 128.0f) + a.eps);
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = y[i] * rstd * (which == 0 ? wq[i] : wk[i]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float c = s_cos[4 * t + i], s = s_sin[4 * t + i];
                const float u0 = y[2 * i], u1 = y[2 * i + 1];
                y[2 * i] = u0 * c - u1 * s;
                y[2 * i + 1] = u0 * s + u1 * c;
            }
            if (which == 0) {
                float m = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(y[i]));
                m = row16_max(m);
                const float sc = m > 0.0f ? m / 448.0f : 1.0f;
                if (t == 0) a.sq[(size_t)n * H + h] = sc;
                r = 1.0 / (double)sc;
            } else {
                r = r_k;
            }
        } else {
            r = s_rv[h];
        }
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_rcp(y[0], r), div_by_rcp(y[1], r), 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_rcp(y[2], r), div_by_rcp(y[3], r), w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_rcp(y[4], r), div_by_rcp(y[5], r), 0, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_rcp(y[6], r), div_by_rcp(y[7], r), w1, true);
        *reinterpret_cast<u32x2_v*>(dst_row + (which * H + h) * 128 + t * 8) = u32x2_v{(uint32_t)w0, (uint32_t)w1};
        h += 16;
        while (which < 3 && h >= H) { h -= H; ++which; }
    }
}

template <int DT>
static hipError_t launch_rope_fp8_w(const QkRopeArgs& a, hipStream_t s) {
    const dim3 grid(a.n_tok), block(256);
    if (a.w_dtype == F16) hipLaunchKernelGGL((qk_norm_rope_fp8_kernel<DT, F16>), grid, block, 0, s, a);
    else if (a.w_dtype == BF16) hipLaunchKernelGGL((qk_norm_rope_fp8_kernel<DT, BF16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((qk_norm_rope_fp8_kernel<DT, F32>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_rope_w(const QkRopeArgs& a, hipStream_t s) {
    const dim3 grid(a.n_tok), block(256);
    if (a.w_dtype == F16) hipLaunchKernelGGL((qk_norm_rope_kernel<DT, F16>), grid, block, 0, s, a);
    else if (a.w_dtype == BF16) hipLaunchKernelGGL((qk_norm_rope_kernel<DT, BF16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((qk_norm_rope_kernel<DT, F32>), grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_qk_rmsnorm_rope(const QkRopeArgs& a, hipStream_t s) {
    if (a.qkv8) {
        if (a.n_heads > 256) return hipErrorInvalidValue;
        if (a.dtype == F16) return launch_rope_fp8_w<F16>(a, s);
        if (a.dtype == BF16) return launch_rope_fp8_w<BF16>(a, s);
        return hipErrorInvalidValue;
    }
    if (a.dtype == F16) return launch_rope_w<F16>(a, s);
    if (a.dtype == BF16) return launch_rope_w<BF16>(a, s);
    return launch_rope_w<F32>(a, s);
}

}  // namespace dit
