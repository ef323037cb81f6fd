// 2-D and causal 3-D convolutions of the diffusion-VAE decoder (the second stage of the pipeline;
// the decoder page measures its convolutions at length, those of a video VAE with causal 3-D
// kernels) on gfx950 as an implicit GEMM: no column buffer is materialised -- the page's point
// against im2col -- each k-step stages 64 input channels of one kernel tap for 256 output pixels
// straight from the channels-last input (the last block of a tap zero-filled where Cin is not a
// multiple of 64: the 96-channel layers of the decoder's last stage).
//
//   y[b, t, h, w, co] = bias[co] + sum_{s, i, j, ci} x[b, t + s - (KT-1), h + i - KH/2, w + j - KW/2, ci]
//                                                  W[co, s, i, j, ci]
//
// with zeros before the first frame and outside the image (stride 1, "same" spatial padding,
// causal in time; KT = T = 1 is the 2-D convolution).  GEMM view: M = B*T*H*W output pixels,
// N = Cout, K = KT*KH*KW*Cin in tap-major order, W read as a [Cout, K] row-major matrix.  The bf16
// GEMM's geometry: 256-row tiles, 64-channel k-steps (rows of 128 B, XOR-swizzled chunks), both
// operands global -> LDS with global_load_lds_dwordx4 into two stages, 8 waves on
// v_mfma_f32_32x32x16_bf16; 256-, 128- or 32-wide output-channel tiles by the layer's width.  A
// row whose tap falls outside the image writes zeros to its LDS bytes (ds_write) instead of
// loading them, and so do the A and B chunks past Cin.  Outputs go out four channels per store
// when Cout is a multiple of 4, one by one otherwise (the 96 -> 3 head).
#include "dev_common.h"
#include "launch.h"

namespace dit {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int CBM = 256, CBK = 64;

// Output-channel tile width by wave layout: WM waves along M (of 8), each a (256 / WM) x (NB * 32)
// sub-tile.  WM = 2: 256-wide tiles (wave tiles 128 x 64); WM = 4: 128-wide (64 x 64) for layers
// of up to 128 channels; WM = 8: 32-wide (32 x 32) for the narrow head.
template <int WM> struct ConvGeom {
    static constexpr int WN = 8 / WM;                 // waves along N
    static constexpr int MB = CBM / (WM * 32);        // 32-row m-blocks per wave
    static constexpr int NB = WM == 8 ? 1 : 2;        // 32-column n-blocks per wave
    static constexpr int BN = WN * NB * 32;           // tile columns
    static constexpr int kStage = (CBM + BN) * CBK * 2;
    static constexpr int kBLoads = BN / 8;            // 1 KB B-load instructions per stage
    static constexpr int BPW = kBLoads >= 8 ? kBLoads / 8 : 1;   // per wave (waves past kBLoads idle)
};

__device__ __forceinline__ int cswz(int row) { return (row >> 1) & 7; }

template <int DT>
__device__ __forceinline__ f32x16_v cmfma(const u32x4_v& a, const u32x4_v& b, const f32x16_v& c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_v, a), __builtin_bit_cast(f16x8_v, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_v, a), __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
}

template <int DT, int OT, int WM>
__device__ __forceinline__ void conv_body(const ConvArgs& a, char* smem) {
    typedef ConvGeom<WM> G;
    constexpr int LPW = 32 / 8;                       // A-load instructions per wave (256 rows)
    constexpr int WN = G::WN, MB = G::MB, NB = G::NB, BPW = G::BPW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int per_group = 8 * a.tiles_n;
    const int grp = L / per_group, first_m = grp * 8;
    const int gsize = min(a.tiles_m - first_m, 8);
    const int rr = L - grp * per_group;
    const int tm = first_m + rr % gsize, tn = rr / gsize;
    const int HW = a.H * a.W;
    const int M = a.B * a.T * HW;
    const int m0 = tm * CBM, n0 = tn * G::BN;
    const int KHW = a.KH * a.KW;
    const int K = a.KT * KHW * a.Cin;
    const int ncb = (a.Cin + CBK - 1) / CBK;     // channel blocks per tap (the last one zero-padded)
    const int nk = a.KT * KHW * ncb;
    const int ph = a.KH / 2, pw = a.KW / 2;

    // load plan: A instruction i of wave w covers tile rows (w*LPW+i)*8 .. +7, B instruction
    // j = w*BPW + r rows j*8 .. +7; lane l writes LDS bytes l*16 .. +15 of the 1 KB block = row
    // l/8, position l%8, holding chunk (l%8) ^ swz(row)
    int pix[LPW], ph_[LPW], pw_[LPW], pt_[LPW], chunk[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int row = (wave * LPW + i) * 8 + (lane >> 3);
        chunk[i] = (lane & 7) ^ cswz(row);
        const int p = min(m0 + row, M - 1);
        pix[i] = p;
        pw_[i] = p % a.W;
        ph_[i] = (p / a.W) % a.H;
        pt_[i] = (p / HW) % a.T;
    }
    const bf16_t* gB[BPW];
    int chunkb[BPW];
#pragma unroll
    for (int r = 0; r < BPW; ++r) {
        const int row = (wave * BPW + r) * 8 + (lane >> 3);
        chunkb[r] = (lane & 7) ^ cswz(row);
        gB[r] = reinterpret_cast<const bf16_t*>(a.w) + (size_t)min(n0 + row, a.Cout - 1) * K + chunkb[r] * 8;
    }
    const bf16_t* X = reinterpret_cast<const bf16_t*>(a.x);
    auto issue = [&](int buf, int kk) {
        const int tap = kk / ncb, cb = kk - tap * ncb;
        const int ts = tap / KHW, tr = tap - ts * KHW;
        const int ti = tr / a.KW, tj = tr - ti * a.KW;
        const int dt = ts - (a.KT - 1), dh = ti - ph, dw = tj - pw;
        char* sa = smem + buf * G::kStage;
        const int c0 = cb * CBK;                                // first channel of the block
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            char* dst = sa + (wave * LPW + i) * 1024;
            const bool cv = c0 + chunk[i] * 8 < a.Cin;          // this lane's 8 channels exist
            const int ih = ph_[i] + dh, iw = pw_[i] + dw;
            if (cv && pt_[i] + dt >= 0 && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W) {
                const bf16_t* src = X + ((long)pix[i] + (long)dt * HW + (long)dh * a.W + dw) * a.Cin + c0 + chunk[i] * 8;
                __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
            } else {
                *reinterpret_cast<u32x4_v*>(dst + lane * 16) = u32x4_v{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int r = 0; r < BPW; ++r) {
            const int j = wave * BPW + r;
            if (j >= G::kBLoads) break;                         // wave-uniform
            char* dstb = sa + CBM * CBK * 2 + j * 1024;
            if (c0 + chunkb[r] * 8 < a.Cin)
                __builtin_amdgcn_global_load_lds(gB[r] + (size_t)tap * a.Cin + c0, (lds_void*)dstb, 16, 0, 0);
            else
                *reinterpret_cast<u32x4_v*>(dstb + lane * 16) = u32x4_v{0u, 0u, 0u, 0u};
        }
    };
    const int h = lane >> 5;
    int a_row[MB], b_row[NB];
#pragma unroll
    for (int j = 0; j < MB; ++j) a_row[j] = wm * (MB * 32) + j * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < NB; ++j) b_row[j] = wn * (NB * 32) + j * 32 + (lane & 31);
    auto frag = [&](const char* base, int row, int s) -> u32x4_v {
        const int c = 2 * s + h;
        return *reinterpret_cast<const u32x4_v*>(base + row * 128 + ((c ^ cswz(row)) << 4));
    };

    f32x16_v acc[NB][MB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
        const int buf = it & 1;
        if (it + 1 < nk) issue(buf ^ 1, it + 1);
        const char* la = smem + buf * G::kStage;
        const char* lb = la + CBM * CBK * 2;
#pragma unroll
        for (int s = 0; s < CBK / 16; ++s) {
            u32x4_v fa[MB], fb[NB];
#pragma unroll
            for (int j = 0; j < MB; ++j) fa[j] = frag(la, a_row[j], s);
#pragma unroll
            for (int j = 0; j < NB; ++j) fb[j] = frag(lb, b_row[j], s);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = cmfma<DT>(fb[nb], fa[mb], acc[nb][mb]);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // epilogue: acc[nb][mb][q] -> pixel m0 + wm*MB*32 + mb*32 + (lane & 31), channel
    // n0 + wn*NB*32 + nb*32 + 8 (q >> 2) + 4 h + (q & 3).  With Cout a multiple of 4 the bias of the
    // lane's columns is loaded once, up front (clamped into Cout; loaded per store group under the
    // bounds test, each load waited at the branch's join).
    const bool c4 = (a.Cout & 3) == 0;
    f32x4_v bv[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[nb][i] = f32x4_v{0.0f, 0.0f, 0.0f, 0.0f};
    if (c4 && a.bias) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                bv[nb][i] = ldf4(a.bias + min(n0 + wn * (NB * 32) + nb * 32 + 8 * i + 4 * h, a.Cout - 4));
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = m0 + wm * (MB * 32) + mb * 32 + (lane & 31);
        if (m >= M) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int col = n0 + wn * (NB * 32) + nb * 32 + 8 * i + 4 * h;
                if (col >= a.Cout) continue;
                float o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = acc[nb][mb][4 * i + j];
                char* yp = reinterpret_cast<char*>(a.y) + ((size_t)m * a.Cout + col) * (OT == F32 ? 4 : 2);
                if (c4) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] += bv[nb][i][j];
                    store4<OT>(yp, o);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (col + j < a.Cout) store1<OT>(yp + j * (OT == F32 ? 4 : 2), o[j] + (a.bias ? a.bias[col + j] : 0.0f));
                }
            }
    }
}

// One kernel per tile width, each with its own LDS size (hipcc emits no host launch stub for a kernel
// template whose static LDS array is sized by a template parameter).
template <int OT>
__global__ __launch_bounds__(512, 1) void conv2d_kernel_w256(ConvArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * ConvGeom<2>::kStage];
    conv_body<BF16, OT, 2>(a, smem);
}
template <int OT>
__global__ __launch_bounds__(512, 1) void conv2d_kernel_w128(ConvArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * ConvGeom<4>::kStage];
    conv_body<BF16, OT, 4>(a, smem);
}
template <int OT>
__global__ __launch_bounds__(512, 1) void conv2d_kernel_w32(ConvArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * ConvGeom<8>::kStage];
    conv_body<BF16, OT, 8>(a, smem);
}

// ---- Direct convolution for narrow layers (Cout <= 32: the decoder head, 96 -> 3).  The implicit
// GEMM stages every input pixel once per tap; here a workgroup stages the input window of a
// 16 x 16-pixel output tile (KT frames of (15 + KH) x (15 + KW) pixels, zeros outside the image
// and before the clip) once per 32-channel block and runs all taps from LDS.  Pixels are 80 bytes
// apart in LDS (32 channels + 16 bytes), so the 16 lanes of a fragment read, 16 consecutive pixels,
// hit distinct banks.  8 waves of 32 pixels x 32 output channels (rows past Cout are zeros) on
// v_mfma_f32_32x32x16_bf16; weight fragments come from global memory (L1 / L2: the weights are a
// few KB), one tap ahead.
constexpr int kDirTile = 16;                       // output tile: 16 x 16 pixels of one frame
constexpr int kDirPix = 80;                        // LDS bytes per staged pixel
constexpr int kDirLds = 80 * 1024;                 // two workgroups per CU
// Staged window of a layer, in bytes (the launcher uses the direct kernel when it fits).
inline long conv_direct_lds(int KT, int KH, int KW) { return (long)KT * (kDirTile - 1 + KH) * (kDirTile - 1 + KW) * kDirPix; }

template <int OT>
__global__ __launch_bounds__(512, 2) void conv_direct_kernel(ConvArgs a) {
    __shared__ __attribute__((aligned(16))) char win[kDirLds];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
    const int tiles_w = (a.W + kDirTile - 1) / kDirTile, tiles_h = (a.H + kDirTile - 1) / kDirTile;
    int L = blockIdx.x;
    const int tx = L % tiles_w; L /= tiles_w;
    const int ty = L % tiles_h; L /= tiles_h;
    const int t = L % a.T, b = L / a.T;               // output frame t of clip b
    const int y0 = ty * kDirTile, x0 = tx * kDirTile;
    const int TH2 = kDirTile - 1 + a.KH, TW2 = kDirTile - 1 + a.KW;
    const int nwin = a.KT * TH2 * TW2;                 // staged pixels
    const float inv_tw = 1.0f / (float)TW2, inv_th = 1.0f / (float)TH2;
    const int ph = a.KH / 2, pw = a.KW / 2;
    const int KHW = a.KH * a.KW, taps = a.KT * KHW;
    const long K = (long)taps * a.Cin;                 // weight row length
    const bf16_t* X = reinterpret_cast<const bf16_t*>(a.x);
    const bf16_t* Wt = reinterpret_cast<const bf16_t*>(a.w);

    // this lane's output pixel (A rows) and weight row (B rows)
    const int pp = wave * 32 + (lane & 31);
    const int py = pp >> 4, px = pp & 15;
    const int wr = lane & 31;                          // output channel of the B fragment
    f32x16_v acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.0f;

    for (int c0 = 0; c0 < a.Cin; c0 += 32) {
        if (c0 > 0) __syncthreads();                   // every wave is done with the last block
        // stage the window: chunk c = pixel * 4 + quarter (8 channels); at most 1024 pixels, so at
        // most 8 chunks per thread, all loaded before the first LDS write
        constexpr int kMaxChunks = kDirLds / kDirPix * 4 / 512;
        u32x4_v v[kMaxChunks];
#pragma unroll
        for (int r = 0; r < kMaxChunks; ++r) {
            const int c = tid + 512 * r;
            v[r] = u32x4_v{0u, 0u, 0u, 0u};
            if (c < nwin * 4) {
                // quotients of numbers below 2^10 by divisors below 32: (n + 0.5) / d is at least
                // 0.5 / d from an integer, far above the float error, so truncation is exact
                const int pix = c >> 2, qq = c & 3;
                const int rr = (int)(((float)pix + 0.5f) * inv_tw), xs = pix - rr * TW2;
                const int s = (int)(((float)rr + 0.5f) * inv_th), ys = rr - s * TH2;
                const int tt = t + s - (a.KT - 1), yy = y0 + ys - ph, xx = x0 + xs - pw;
                const int ch = c0 + qq * 8;
                if (tt >= 0 && (unsigned)yy < (unsigned)a.H && (unsigned)xx < (unsigned)a.W && ch < a.Cin)
                    v[r] = ld16(X + ((((long)b * a.T + tt) * a.H + yy) * a.W + xx) * a.Cin + ch);
            }
        }
#pragma unroll
        for (int r = 0; r < kMaxChunks; ++r) {
            const int c = tid + 512 * r;
            if (c < nwin * 4) *reinterpret_cast<u32x4_v*>(win + (c >> 2) * kDirPix + (c & 3) * 16) = v[r];
        }
        __syncthreads();
        // weight fragment of tap k, k16 step ks: row wr, channels c0 + 16 ks + 8 h .. +7, the row and
        // channel clamped into the weights (rows past Cout feed outputs that are not stored; channels
        // past Cin meet the window's zeros), so every load is unconditional
        const bf16_t* wrow = Wt + (long)min(wr, a.Cout - 1) * K;
        auto wfrag = [&](int k, int ks) -> u32x4_v {
            return ld16(wrow + (long)k * a.Cin + min(c0 + 16 * ks + 8 * h, a.Cin - 8));
        };
        // taps frame by frame, row by row (no division in the loop), two taps per pass with the
        // weight fragments in two register pairs of alternating roles: each pair loads while the
        // other pair's tap runs (one pair copied into the other after every tap, or loaded under
        // a branch, made every tap wait for the next tap's weights)
        int sf = 0, ti = 0, tj = 0;                    // the next tap to run
        auto run_tap = [&](const u32x4_v& w0, const u32x4_v& w1) {
            const char* p = win + ((sf * TH2 + py + ti) * TW2 + px + tj) * kDirPix + 16 * h;
            const u32x4_v fa0 = *reinterpret_cast<const u32x4_v*>(p);
            const u32x4_v fa1 = *reinterpret_cast<const u32x4_v*>(p + 32);
            acc = cmfma<BF16>(w0, fa0, acc);
            acc = cmfma<BF16>(w1, fa1, acc);
            if (++tj == a.KW) {
                tj = 0;
                if (++ti == a.KH) { ti = 0; ++sf; }
            }
        };
        u32x4_v wa0 = wfrag(0, 0), wa1 = wfrag(0, 1);
        for (int k = 0; k < taps; k += 2) {
            const int k1 = min(k + 1, taps - 1), k2 = min(k + 2, taps - 1);
            const u32x4_v wb0 = wfrag(k1, 0), wb1 = wfrag(k1, 1);
            run_tap(wa0, wa1);
            wa0 = wfrag(k2, 0);
            wa1 = wfrag(k2, 1);
            if (k + 1 < taps) run_tap(wb0, wb1);
        }
    }

    // acc[q] -> pixel pp, output channel 8 (q >> 2) + 4 h + (q & 3)
    const int yo = y0 + py, xo = x0 + px;
    if (yo >= a.H || xo >= a.W) return;
    const long m = (((long)b * a.T + t) * a.H + yo) * a.W + xo;
    float bias[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) bias[q] = a.bias ? a.bias[min(8 * (q >> 2) + 4 * h + (q & 3), a.Cout - 1)] : 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int co = 8 * (q >> 2) + 4 * h + (q & 3);
        if (co < a.Cout)
            store1<OT>(reinterpret_cast<char*>(a.y) + (m * a.Cout + co) * (OT == F32 ? 4 : 2), acc[q] + bias[q]);
    }
}

template <int WM>
static void launch_conv_w(ConvArgs& a, long M, hipStream_t s) {
    a.tiles_m = (int)((M + CBM - 1) / CBM);
    a.tiles_n = (a.Cout + ConvGeom<WM>::BN - 1) / ConvGeom<WM>::BN;
    const dim3 grid(a.tiles_m * a.tiles_n), block(512);
    const bool f32 = a.y_dtype == F32;
    if constexpr (WM == 2) {
        if (f32) hipLaunchKernelGGL((conv2d_kernel_w256<F32>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((conv2d_kernel_w256<BF16>), grid, block, 0, s, a);
    } else if constexpr (WM == 4) {
        if (f32) hipLaunchKernelGGL((conv2d_kernel_w128<F32>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((conv2d_kernel_w128<BF16>), grid, block, 0, s, a);
    } else {
        if (f32) hipLaunchKernelGGL((conv2d_kernel_w32<F32>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((conv2d_kernel_w32<BF16>), grid, block, 0, s, a);
    }
}

hipError_t launch_conv2d(ConvArgs& a, hipStream_t s) {
    const long M = (long)a.B * a.T * a.H * a.W;
    if (M == 0) return hipSuccess;
    // narrow layers whose staged window fits: the direct kernel; otherwise the narrowest implicit-GEMM
    // tile that covers the output channels (fewer idle MFMA columns)
    if (a.Cout <= 32 && conv_direct_lds(a.KT, a.KH, a.KW) <= kDirLds) {
        const long tiles = (long)a.B * a.T * ((a.H + kDirTile - 1) / kDirTile) * ((a.W + kDirTile - 1) / kDirTile);
        if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
        const dim3 grid((unsigned)tiles), block(512);
        if (a.y_dtype == F32) hipLaunchKernelGGL((conv_direct_kernel<F32>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((conv_direct_kernel<BF16>), grid, block, 0, s, a);
    } else if (a.Cout <= 32) launch_conv_w<8>(a, M, s);
    else if (a.Cout <= 128) launch_conv_w<4>(a, M, s);
    else launch_conv_w<2>(a, M, s);
    return hipGetLastError();
}

}  // namespace dit
