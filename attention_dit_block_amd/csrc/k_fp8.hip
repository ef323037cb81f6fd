// fp8 (OCP e4m3) variant of the block's matrix products on gfx950: per-row quantisation and a GEMM
// on v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 operands, unit block scales), whose dense peak is
// twice bf16's.  The pages weigh speed against accuracy (a "slight (invisible) loss of accuracy"
// in the reply that follows the cuBLAS split of the "CUDA codepath !" thread, antirez/iris.c issue
// #15); this is that trade on MI355X.
//
// Quantisation: one wave per row; s = max|x| / 448 and q = e4m3(x / s) with correctly rounded
// fp32 divisions and the hardware's round-to-nearest-even conversion (v_cvt_pk_fp8_f32); the
// scaling keeps every value inside e4m3's finite range.
//
// GEMM: the bf16 kernel's geometry with bytes for elements -- a 256 x 256 tile, K steps of 128
// codes (rows of 128 B, the same XOR swizzle), both operands global -> LDS with
// global_load_lds_dwordx4 into two stages, 8 waves of 128 x 64.  A 32x32x64 MFMA takes 32 codes
// of one row per lane: lanes 0-31 codes 0-31 of the 64-code k-slice, lanes 32-63 codes 32-63, the
// same split on both operands.  Epilogue: acc * sa[m] * sb[n], four consecutive columns per lane,
// then the block's epilogues as in the 16-bit GEMM: plain store, gated residual R + gate[n] * (.),
// or SwiGLU (a tile's B rows are 128 gate rows and the 128 matching up rows).  One launch covers
// up to two problems (text and image streams).
#include "dev_common.h"
#include "launch.h"

namespace dit {

constexpr float kE4M3Max = 448.0f;

// One wave per row.  x / s goes through the double reciprocal of s: the double product is within
// 2^-52 (relative) of the quotient, and a quotient of two fp32 values in the normal range lies more
// than 2^-49 from every midpoint between neighbouring fp32 values, so the product rounds to the
// correctly rounded quotient (results below the normal range are e4m3 zeros of the same sign either
// way) -- three instructions instead of a division's ten.
__device__ __forceinline__ float div_by_rcp8(float x, double r) { return (float)((double)x * r); }

template <int XT>
__device__ __forceinline__ void quant_store8(uint8_t* dst, const float* f, double r) {
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_rcp8(f[0], r), div_by_rcp8(f[1], r), 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_rcp8(f[2], r), div_by_rcp8(f[3], r), w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_rcp8(f[4], r), div_by_rcp8(f[5], r), 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(div_by_rcp8(f[6], r), div_by_rcp8(f[7], r), w1, true);
    *reinterpret_cast<u32x2_v*>(dst) = u32x2_v{(uint32_t)w0, (uint32_t)w1};
}

// 16-bit rows of up to 512 * NC columns: the row is loaded once, all its chunks in flight together
// (columns clamped into the row, cols >= 8 and a multiple of 8), and kept packed in registers
// between the max and the codes.
template <int XT, int NC>
__global__ __launch_bounds__(256) void quantize_fp8_rows_kernel(const void* x, long ld_x, int rows, int cols,
                                                                uint8_t* q, long ld_q, float* scales) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + wave;
    if (r >= rows) return;
    const char* xr = reinterpret_cast<const char*>(x) + (size_t)r * ld_x * 2;
    u32x4_v raw[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i)
        raw[i] = *reinterpret_cast<const u32x4_v*>(xr + (size_t)min((lane + 64 * i) * 8, cols - 8) * 2);
    auto unpack = [&](const u32x4_v& w, float* f) {
#pragma unroll
        for (int t = 0; t < 4; ++t) unpack2<XT>(w[t], f[2 * t], f[2 * t + 1]);
    };
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        if ((lane + 64 * i) * 8 < cols) {
            float f[8];
            unpack(raw[i], f);
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    const float s = amax > 0.0f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
    if (lane == 0) scales[r] = s;
    const double rs = 1.0 / (double)s;
    uint8_t* qr = q + (size_t)r * ld_q;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int k0 = (lane + 64 * i) * 8;
        if (k0 < cols) {
            float f[8];
            unpack(raw[i], f);
            quant_store8<XT>(qr + k0, f, rs);
        }
    }
}

// Any row length and fp32 rows: two passes over the row, four chunks in flight per pass step.
template <int XT>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const void* x, long ld_x, int rows, int cols, uint8_t* q,
                                                           long ld_q, float* scales) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + wave;
    if (r >= rows) return;
    constexpr int XS = XT == F32 ? 4 : 2;
    const char* xr = reinterpret_cast<const char*>(x) + (size_t)r * ld_x * XS;
    float amax = 0.0f;
    for (int k0 = lane * 8; k0 < cols; k0 += 4 * 512) {
        float f[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) load8<XT>(xr + (size_t)min(k0 + 512 * u, cols - 8) * XS, f[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (k0 + 512 * u < cols) {
#pragma unroll
                for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[u][j]));
            }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    const float s = amax > 0.0f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
    if (lane == 0) scales[r] = s;
    const double rs = 1.0 / (double)s;
    uint8_t* qr = q + (size_t)r * ld_q;
    for (int k0 = lane * 8; k0 < cols; k0 += 4 * 512) {
        float f[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) load8<XT>(xr + (size_t)min(k0 + 512 * u, cols - 8) * XS, f[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (k0 + 512 * u < cols) quant_store8<XT>(qr + k0 + 512 * u, f[u], rs);
    }
}

template <int XT>
static void launch_quant_rows(const void* x, long ld_x, int rows, int cols, uint8_t* q, long ld_q, float* scales,
                              hipStream_t s, dim3 grid) {
    const int nc = (cols + 511) / 512;
    if (nc <= 2) hipLaunchKernelGGL((quantize_fp8_rows_kernel<XT, 2>), grid, dim3(256), 0, s, x, ld_x, rows, cols, q, ld_q, scales);
    else if (nc <= 6) hipLaunchKernelGGL((quantize_fp8_rows_kernel<XT, 6>), grid, dim3(256), 0, s, x, ld_x, rows, cols, q, ld_q, scales);
    else if (nc <= 12) hipLaunchKernelGGL((quantize_fp8_rows_kernel<XT, 12>), grid, dim3(256), 0, s, x, ld_x, rows, cols, q, ld_q, scales);
    else if (nc <= 18) hipLaunchKernelGGL((quantize_fp8_rows_kernel<XT, 18>), grid, dim3(256), 0, s, x, ld_x, rows, cols, q, ld_q, scales);
    else hipLaunchKernelGGL((quantize_fp8_rows_kernel<XT, 24>), grid, dim3(256), 0, s, x, ld_x, rows, cols, q, ld_q, scales);
}

hipError_t launch_quantize_fp8(const void* x, int x_dtype, long ld_x, int rows, int cols, uint8_t* q, long ld_q,
                               float* scales, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const dim3 grid((rows + 3) / 4), block(256);
    const bool in_regs = cols <= 512 * 24;
    if (x_dtype == F32) hipLaunchKernelGGL((quantize_fp8_kernel<F32>), grid, block, 0, s, x, ld_x, rows, cols, q, ld_q, scales);
    else if (x_dtype == F16 && in_regs) launch_quant_rows<F16>(x, ld_x, rows, cols, q, ld_q, scales, s, grid);
    else if (x_dtype == F16) hipLaunchKernelGGL((quantize_fp8_kernel<F16>), grid, block, 0, s, x, ld_x, rows, cols, q, ld_q, scales);
    else if (in_regs) launch_quant_rows<BF16>(x, ld_x, rows, cols, q, ld_q, scales, s, grid);
    else hipLaunchKernelGGL((quantize_fp8_kernel<BF16>), grid, block, 0, s, x, ld_x, rows, cols, q, ld_q, scales);
    return hipGetLastError();
}

// ---- GEMM ----------------------------------------------------------------------------------
typedef int i32x8_v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int QBM = 256, QBN = 256, QBK = 128;          // codes (= bytes) per k-step
constexpr int kQStage = (QBM + QBN) * QBK;              // 64 KB: A then B
constexpr int kQLds = 2 * kQStage;

__device__ __forceinline__ int qswz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ f32x16_v mfma_f8(const i32x8_v& a, const i32x8_v& b, const f32x16_v& c) {
    // e4m3 operands (format 0), block scales 2^(127 - 127) = 1
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// SiLU of an fp32 accumulator whose product is rounded to 16 bits or fewer: the reciprocal instruction
// (within 1 ulp) in place of a correctly rounded division, whose fix-up sequence is ~10 instructions
__device__ __forceinline__ float silu_f8(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Four consecutive columns of one output row, output type chosen at run time.
__device__ __forceinline__ void store4_any(void* base, size_t off, int dt, const float* o) {
    char* p = reinterpret_cast<char*>(base);
    if (dt == F32) store4<F32>(p + off * 4, o);
    else if (dt == F16) store4<F16>(p + off * 2, o);
    else store4<BF16>(p + off * 2, o);
}

// MODE: EPI_STORE, EPI_GATED_RES or EPI_SWIGLU for every problem of the batch.
template <int MODE>
__global__ __launch_bounds__(512, 1) void gemm_fp8_kernel(Fp8GemmBatch bt) {
    constexpr int NW = 8, WN = 4, NB = 2, LPW = 32 / NW;   // waves, along N, 32-col blocks, loads
    constexpr bool kSwiglu = MODE == EPI_SWIGLU;
    __shared__ __attribute__((aligned(1024))) char smem[kQLds];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    // tile: XCD-contiguous; per problem, groups of 8 M-tiles walked N-major
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int pi = (bt.n > 1 && L >= bt.p[1].tile_begin) ? 1 : 0;
    const Fp8GemmProblem& g = bt.p[pi];
    const int t = L - g.tile_begin;
    const int per_group = 8 * g.tiles_n;
    const int grp = t / per_group, first_m = grp * 8;
    const int gsize = min(g.tiles_m - first_m, 8);
    const int rr = t - grp * per_group;
    const int tm = first_m + rr % gsize, tn = rr / gsize;
    const int m0 = tm * QBM;
    const int n0 = kSwiglu ? tn * (QBN / 2) : tn * QBN;     // first output column

    // load plan: wave w, instruction i covers tile rows (w*LPW+i)*8 .. +7; lane l writes LDS bytes
    // l*16 .. +15 of the 1 KB block = row l/8, position l%8, holding chunk (l%8) ^ swz(row).
    // SwiGLU tiles stage the gate rows of their 128 output columns in B rows 0-127 and the
    // matching up rows in 128-255.
    auto b_src = [&](int row) -> long {
        if (kSwiglu) {
            const bool up = row >= QBN / 2;
            const long n = min((long)n0 + (up ? row - QBN / 2 : row), (long)g.N - 1);
            return up ? n + g.up_off : n;
        }
        return min((long)n0 + row, (long)g.N - 1);
    };
    const uint8_t* gA[LPW];
    const uint8_t* gB[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int row = (wave * LPW + i) * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ qswz(row);
        gA[i] = g.a + (size_t)min(m0 + row, g.M - 1) * g.lda + chunk * 16;
        gB[i] = g.b + (size_t)b_src(row) * g.ldb + chunk * 16;
    }
    auto issue = [&](int buf, int k0) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            __builtin_amdgcn_global_load_lds(gA[i] + k0, (lds_void*)(smem + buf * kQStage + (wave * LPW + i) * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(gB[i] + k0, (lds_void*)(smem + buf * kQStage + QBM * QBK + (wave * LPW + i) * 1024),
                                             16, 0, 0);
        }
    };
    const int h = lane >> 5;
    int a_row[4], b_row[NB];
#pragma unroll
    for (int j = 0; j < 4; ++j) a_row[j] = wm * 128 + j * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < NB; ++j)
        b_row[j] = (kSwiglu ? j * (QBN / 2) + wn * 32 : wn * 64 + j * 32) + (lane & 31);
    // fragment of sub-step s (codes 64 s .. 64 s + 63 of the k-step): chunks 4 s + 2 h, + 1
    auto frag = [&](const char* base, int row, int s) -> i32x8_v {
        const int c = 4 * s + 2 * h;
        const u32x4_v lo = *reinterpret_cast<const u32x4_v*>(base + row * 128 + ((c ^ qswz(row)) << 4));
        const u32x4_v hi = *reinterpret_cast<const u32x4_v*>(base + row * 128 + (((c + 1) ^ qswz(row)) << 4));
        return i32x8_v{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };

    f32x16_v acc[NB][4];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    const int nk = g.K / QBK;
    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
        const int buf = it & 1;
        if (it + 1 < nk) issue(buf ^ 1, (it + 1) * QBK);
        const char* la = smem + buf * kQStage;
        const char* lb = la + QBM * QBK;
#pragma unroll
        for (int s = 0; s < QBK / 64; ++s) {
            i32x8_v fa[4], fb[NB];
#pragma unroll
            for (int j = 0; j < 4; ++j) fa[j] = frag(la, a_row[j], s);
#pragma unroll
            for (int j = 0; j < NB; ++j) fb[j] = frag(lb, b_row[j], s);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = mfma_f8(fb[nb], fa[mb], acc[nb][mb]);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // epilogue: acc[nb][mb][q] -> row m0 + wm*128 + mb*32 + (lane & 31); B row b_row[nb] - (lane & 31)
    // + 8 (q >> 2) + 4 h + (q & 3) of the tile
    bool bad = false;              // an fp16 output out of fp16's range
    float vm = 0.0f;               // EPI_STORE with vmax: largest |stored value| of this lane
    // Output type CT and residual type RT dispatched once per tile; each 32-column block's scale,
    // gate and residual loads issue together before its stores, rows and columns clamped into the
    // problem (N is a multiple of 8) and the stores tested -- under a type switch or a bounds test
    // each load waited at the branch's join, one round trip per 4 outputs.
    auto tile_out = [&]<int CT, int RT>() {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int m = m0 + wm * 128 + mb * 32 + (lane & 31);
            const int mc = min(m, g.M - 1);
            const float sa = g.sa[mc];
            char* crow = reinterpret_cast<char*>(g.c) + (size_t)m * g.ldc * ESize<CT>::v;
            if constexpr (kSwiglu) {
                f32x4_v sg[4], su[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int cc = min(n0 + wn * 32 + 8 * i + 4 * h, g.N - 4);
                    sg[i] = ldf4(g.sb + cc);
                    su[i] = ldf4(g.sb + g.up_off + cc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int col = n0 + wn * 32 + 8 * i + 4 * h;
                    float o[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        o[j] = silu_f8(acc[0][mb][4 * i + j] * sa * sg[i][j]) * (acc[1][mb][4 * i + j] * sa * su[i][j]);
                    if (m < g.M && col < g.N) {
                        if constexpr (CT == F16) bad |= f16_out_of_range4(o);
                        store4<CT>(crow + (size_t)col * ESize<CT>::v, o);
                    }
                }
            } else {
                const char* rrow = MODE == EPI_GATED_RES
                                       ? reinterpret_cast<const char*>(g.r) + (size_t)mc * g.ldr * ESize<RT>::v
                                       : nullptr;
#pragma unroll
                for (int hb = 0; hb < 2 * NB; ++hb) {      // 16-column halves of the 32-column blocks
                    const int nb = hb >> 1, i0 = 2 * (hb & 1);
                    f32x4_v sb[4], gt[4];
                    float r[4][4];
#pragma unroll
                    for (int i = i0; i < i0 + 2; ++i) {
                        const int cc = min(n0 + wn * 64 + nb * 32 + 8 * i + 4 * h, g.N - 4);
                        sb[i] = ldf4(g.sb + cc);
                        if constexpr (MODE == EPI_GATED_RES) {
                            gt[i] = ldf4(g.gate + cc);
                            load4<RT>(rrow + (size_t)cc * ESize<RT>::v, r[i]);
                        }
                    }
#pragma unroll
                    for (int i = i0; i < i0 + 2; ++i) {
                        const int col = n0 + wn * 64 + nb * 32 + 8 * i + 4 * h;
                        float o[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) o[j] = acc[nb][mb][4 * i + j] * sa * sb[i][j];
                        if constexpr (MODE == EPI_GATED_RES) {
#pragma unroll
                            for (int j = 0; j < 4; ++j) o[j] = fmaf(gt[i][j], o[j], r[i][j]);
                        }
                        if (m < g.M && col < g.N) {
                            if constexpr (CT == F16) bad |= f16_out_of_range4(o);
                            if constexpr (MODE == EPI_STORE) {
                                if (bt.vmax) {
#pragma unroll
                                    for (int j = 0; j < 4; ++j) {
                                        // the value as stored (the QK-norm + RoPE pass quantises that)
                                        const float st = CT == F16 ? (float)(_Float16)o[j]
                                                       : CT == BF16 ? bf_lo(pack_bf16x2(o[j], 0.0f)) : o[j];
                                        vm = fmaxf(vm, fabsf(st));
                                    }
                                }
                            }
                            store4<CT>(crow + (size_t)col * ESize<CT>::v, o);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };
    if constexpr (MODE == EPI_GATED_RES) {
        // gated-residual outputs are F32 or BF16 over BF16 or F32 residuals (checked on the host)
        if (g.r_dtype == BF16) {
            if (g.c_dtype == BF16) tile_out.template operator()<BF16, BF16>();
            else tile_out.template operator()<F32, BF16>();
        } else {
            if (g.c_dtype == BF16) tile_out.template operator()<BF16, F32>();
            else tile_out.template operator()<F32, F32>();
        }
    } else {
        if (g.c_dtype == F32) tile_out.template operator()<F32, F32>();
        else if (g.c_dtype == F16) tile_out.template operator()<F16, F32>();
        else tile_out.template operator()<BF16, F32>();
    }
    raise_range_flag(bt.range_flag, bad);
    if constexpr (MODE == EPI_STORE) {
        // a wave's 64 columns lie inside one 128-column head: one atomic max per wave
        const int cb = n0 + wn * 64;
        if (bt.vmax && cb >= bt.vmax_col0 && cb < g.N) {
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) vm = fmaxf(vm, __shfl_xor(vm, off, 64));
            if (lane == 0)
                __hip_atomic_fetch_max(bt.vmax + (cb - bt.vmax_col0) / 128, __float_as_uint(vm), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

hipError_t launch_gemm_fp8(Fp8GemmBatch& bt, hipStream_t s) {
    int total = 0;
    for (int i = 0; i < bt.n; ++i) {
        Fp8GemmProblem& g = bt.p[i];
        const bool sw = g.epi == EPI_SWIGLU;
        if (g.M > 0 && g.epi == EPI_GATED_RES &&
            ((g.c_dtype != F32 && g.c_dtype != BF16) || (g.r_dtype != F32 && g.r_dtype != BF16)))
            return hipErrorInvalidValue;
        g.tiles_m = g.M > 0 ? (g.M + QBM - 1) / QBM : 0;
        g.tiles_n = sw ? (g.N + QBN / 2 - 1) / (QBN / 2) : (g.N + QBN - 1) / QBN;
        g.tile_begin = total;
        total += g.tiles_m * g.tiles_n;
    }
    bt.total_tiles = total;
    if (total == 0) return hipSuccess;
    const dim3 grid(total), block(512);
    // every problem of a batch has the first one's epilogue (the callers build them so)
    if (bt.p[0].epi == EPI_SWIGLU) hipLaunchKernelGGL((gemm_fp8_kernel<EPI_SWIGLU>), grid, block, 0, s, bt);
    else if (bt.p[0].epi == EPI_GATED_RES) hipLaunchKernelGGL((gemm_fp8_kernel<EPI_GATED_RES>), grid, block, 0, s, bt);
    else hipLaunchKernelGGL((gemm_fp8_kernel<EPI_STORE>), grid, block, 0, s, bt);
    return hipGetLastError();
}

}  // namespace dit
