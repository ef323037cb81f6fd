// Windowed (neighborhood) attention on gfx950: each query of a [T, H, W] token grid attends to
// the keys of a 3-D window around it, odd-sized per axis; near an edge the window shifts inwards,
// and an axis narrower than the window is attended in full (the boundary rule of the
// neighborhood-attention port on the diffusion-VAE decoder page, where LTX-2.5's decoder uses a
// fixed [11, 11, 11] window).
//
// 16-bit kernel (bf16 or fp16 q, k, v): the joint-attention kernel's machinery (S^T = K Q^T on
// v_mfma_f32_32x32x16, base-2 online softmax with a lazily raised max, O^T += V^T P^T with the
// V^T operand from ds_read_b64_tr_b16) over a gathered key set.  A workgroup owns a 16 x 16 patch
// of queries of one frame; the union of their windows is a box of kT frames x bh rows x bw
// columns.  Box rows are padded to P = 32 or 64 keys, so a 64-key tile holds 64 / P whole box
// rows and every score register of a lane sits at a column known at compile time: a key is valid
// for a lane's query when its box row lies in the query's row range (one compare per 32-key
// block) and its column bit is set in the lane's 64-bit column mask.  Invalid keys (outside the
// window, the padding, past the last box row) score -inf.  Keys are gathered row by row with
// global_load_lds from their token rows.
//
// fp32 kernel: one wave per query, scores of its window in LDS, fp32 arithmetic throughout.
#include "attn_common.h"
#include "dev_common.h"
#include "launch.h"

namespace dit {

constexpr int kWinWaves = 8;
constexpr int WQH = 16, WQW = 16;       // query patch of a workgroup (256 queries)

// First position of the window (effective size ke, requested kr) of query position i on an axis
// of extent n.
__device__ __forceinline__ int win_start(int i, int kr, int ke, int n) { return min(max(i - kr / 2, 0), n - ke); }

// a / b for 0 <= a < 2^23, 1 <= b (float estimate, corrected by one step)
__device__ __forceinline__ int div_small(int a, int b, float inv_b) {
    int q = (int)((float)a * inv_b);
    if (q * b > a) --q;
    else if ((q + 1) * b <= a) ++q;
    return q;
}

template <int DT, int PITCH>
__device__ __forceinline__ void window_attention_body(const WinAttnArgs& a) {
    constexpr int R = 64 / PITCH;           // box rows per 64-key tile
    constexpr int LPW = 16 / kWinWaves;     // 1 KB load instructions per wave per K (or V) tile
    typedef typename AFrag<DT>::T FragT;
    __shared__ __attribute__((aligned(1024))) char smem[4 * kTile];     // K ring, then V ring
    constexpr int kV = 2 * kTile;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h32 = lane >> 5, l32 = lane & 31;
    const int H = a.H, W = a.W;
    // unit: (head, frame, patch row, patch column), XCD-contiguous
    int L = xcd_remap(blockIdx.x, gridDim.x);
    const int tw = L % a.tiles_w;
    L /= a.tiles_w;
    const int th = L % a.tiles_h;
    L /= a.tiles_h;
    const int t = L % a.T, head = L / a.T;
    const int h0 = th * WQH, w0 = tw * WQW;
    const float c2 = a.scale * 1.4426950408889634f;     // scores in base 2

    // this lane's query (patch position wave*32 + l32, row-major in the patch)
    const int qi = wave * 32 + l32;
    const int qh = h0 + qi / WQW, qw = w0 + qi % WQW;
    const bool q_ok = qh < H && qw < W;
    const int qhc = min(qh, H - 1), qwc = min(qw, W - 1);
    const long qtok = ((long)t * H + qhc) * W + qwc;

    // the union of the patch's windows: frames [ts, ts + kT), rows [bh0, bh0 + bh), columns
    // [bw0, bw0 + bw), bw <= PITCH
    const int ts = win_start(t, a.rT, a.kT, a.T);
    const int bh0 = win_start(h0, a.rH, a.kH, H);
    const int bh = win_start(min(h0 + WQH - 1, H - 1), a.rH, a.kH, H) + a.kH - bh0;
    const int bw0 = win_start(w0, a.rW, a.kW, W);
    const int bw = win_start(min(w0 + WQW - 1, W - 1), a.rW, a.kW, W) + a.kW - bw0;
    const int NR = a.kT * bh;
    const int nt = (NR + R - 1) / R;
    const float inv_bh = 1.0f / (float)bh;
    // this lane's window inside the box: rows [hs, hs + kH), columns [ws, ws + kW)
    const int hs = win_start(qhc, a.rH, a.kH, H) - bh0;
    const int ws = win_start(qwc, a.rW, a.kW, W) - bw0;
    const unsigned long long cm = ((a.kW >= 64 ? ~0ull : (1ull << a.kW) - 1ull)) << ws;
    // column bits of the keys in this lane's score registers (register q of 32-key block kb
    // holds the key at offset 16 (q >> 3) + 8 h32 + (q & 7) of the block)
    uint32_t m32[2];
    if constexpr (PITCH == 32) {
        m32[0] = m32[1] = (uint32_t)(cm >> (8 * h32));
    } else {
        m32[0] = (uint32_t)(cm >> (8 * h32));
        m32[1] = (uint32_t)(cm >> (32 + 8 * h32));
    }

    const bf16_t* Qg = reinterpret_cast<const bf16_t*>(a.q) + head * HD;
    const bf16_t* Kg = reinterpret_cast<const bf16_t*>(a.k) + head * HD;
    const bf16_t* Vg = reinterpret_cast<const bf16_t*>(a.v) + head * HD;

    FragT qf[8];
    {
        const bf16_t* qp = Qg + qtok * a.ld_q + 8 * h32;
#pragma unroll
        for (int es = 0; es < 8; ++es) qf[es] = *reinterpret_cast<const FragT*>(qp + 16 * es);
    }

    // token row of key kk (0..63) of key tile j; keys outside the box map to the box origin
    const long tok0 = ((long)ts * H + bh0) * W + bw0;
    auto key_token = [&](int j, int kk) -> long {
        const int br = j * R + kk / PITCH, c = kk % PITCH;
        if (br >= NR || c >= bw) return tok0;
        const int f = div_small(br, bh, inv_bh);
        const int r = br - f * bh;
        return tok0 + ((long)f * H + r) * W + c;
    };
    // load plan as in the joint-attention kernel: instruction i of a tile fills rows
    // 16 (i%4) .. +15 of slab i/4; lane l writes row 16 (i%4) + l/4, position l%4
    const int slab = (LPW * wave) >> 2, rg0 = (LPW * wave) & 3;
    auto load_k = [&](int slot, int j) {
        char* dst = smem + slot * kTile;
#pragma unroll
        for (int r = 0; r < LPW; ++r) {
            const long tok = key_token(j, 16 * (rg0 + r) + (lane >> 2));
            __builtin_amdgcn_global_load_lds(Kg + tok * a.ld_k + 32 * slab + 8 * ((lane & 3) ^ (lane >> 4)),
                                             (lds_void*)(dst + (LPW * wave + r) * 1024), 16, 0, 0);
        }
    };
    auto load_v = [&](int slot, int j) {
        char* dst = smem + kV + slot * kTile;
#pragma unroll
        for (int r = 0; r < LPW; ++r) {
            const long tok = key_token(j, 16 * (rg0 + r) + (lane >> 2));
            __builtin_amdgcn_global_load_lds(Vg + tok * a.ld_v + 32 * slab + 8 * (lane & 3),
                                             (lds_void*)(dst + (LPW * wave + r) * 1024), 16, 0, 0);
        }
    };

    int k_off[2];
    {
        const int kr = key_of_row(l32);
        k_off[0] = kr * 64 + (kpos(kr, h32) << 4);
        k_off[1] = kr * 64 + (kpos(kr, 2 + h32) << 4);
    }
    const int v_off = (8 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) * 64 + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

    auto scores = [&](f32x16_v* sd, int slot) {
        const char* kt = smem + slot * kTile;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int es = 0; es < 8; ++es) {
                const FragT kf = *reinterpret_cast<const FragT*>(kt + (es >> 1) * 4096 + kb * 32 * 64 + k_off[es & 1]);
                sd[kb] = es == 0 ? amfma<DT>(kf, qf[es], f32x16_v{}) : amfma<DT>(kf, qf[es], sd[kb]);
            }
    };

    f32x16_v o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) o[i][q] = 0.0f;
    // a finite start: a lane may see whole tiles with no valid key before its first valid one
    float m_run = -1e30f, l_run = 0.0f;
    f32x16_v sA[2], sB[2];

    auto step = [&]<int S, bool LAST>(int j, f32x16_v* SC, f32x16_v* SN) {
        if constexpr (!LAST) {
            if (j + 2 < nt) load_k(S, j + 2);
            load_v(S ^ 1, j + 1);
        }
        if constexpr (!LAST) scores(SN, S ^ 1);
        // validity: the block's box row inside the query's row range, the key's column bit set
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int br = j * R + (PITCH == 32 ? kb : 0);
            const int f = div_small(br, bh, inv_bh);
            const int rr = br - f * bh;
            const bool row_ok = br < NR && (unsigned)(rr - hs) < (unsigned)a.kH;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const bool ok = row_ok && ((m32[kb] >> (16 * (q >> 3) + (q & 7))) & 1u);
                SC[kb][q] = ok ? SC[kb][q] : -INFINITY;
            }
        }
        float e0 = SC[0][0], e1 = SC[1][0];
#pragma unroll
        for (int q = 1; q < 16; ++q) {
            e0 = fmaxf(e0, SC[0][q]);
            e1 = fmaxf(e1, SC[1][q]);
        }
        const float mt = half_swap_max(fmaxf(e0, e1)) * c2;
        const bool raise = mt > m_run + kLazyMax;
        const float m_new = raise ? mt : m_run;
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        const float nm = -m_new;
        uint32_t ph[16], pl[DT == BF16 ? 16 : 1];
        float lsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 16; q += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(SC[kb][q], c2, nm));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(SC[kb][q + 1], c2, nm));
                lsum += p0 + p1;
                const int w = 8 * kb + (q >> 1);
                if constexpr (DT == BF16) {
                    const uint32_t u0 = __float_as_uint(p0) & 0xffff0000u, u1 = __float_as_uint(p1) & 0xffff0000u;
                    ph[w] = (u0 >> 16) | u1;
                    pl[w] = pack_bf16x2(p0 - __uint_as_float(u0), p1 - __uint_as_float(u1));
                } else {
                    ph[w] = pack_f16x2(p0, p1);
                }
            }
        l_run = fmaf(l_run, corr, lsum);
        if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 16; ++q) o[i][q] *= corr;
        }
        const char* vt = smem + kV + S * kTile;
        auto read_v = [&](FragT* vf, int ks) {
#pragma unroll
            for (int eb = 0; eb < 4; ++eb) {
                const char* vp = vt + v_off + eb * 4096 + ks * 16 * 64;
                const s16x4_v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp));
                const s16x4_v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 4 * 64));
                const s16x8_v w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                vf[eb] = __builtin_bit_cast(FragT, w);
            }
        };
        FragT vf[2][4];
        read_v(vf[0], 0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks < 3) read_v(vf[(ks + 1) & 1], ks + 1);
            const u32x4_v hv = {ph[4 * ks], ph[4 * ks + 1], ph[4 * ks + 2], ph[4 * ks + 3]};
#pragma unroll
            for (int eb = 0; eb < 4; ++eb) o[eb] = amfma<DT>(vf[ks & 1][eb], __builtin_bit_cast(FragT, hv), o[eb]);
            if constexpr (DT == BF16) {
                const u32x4_v lv = {pl[4 * ks], pl[4 * ks + 1], pl[4 * ks + 2], pl[4 * ks + 3]};
#pragma unroll
                for (int eb = 0; eb < 4; ++eb) o[eb] = amfma<DT>(vf[ks & 1][eb], __builtin_bit_cast(FragT, lv), o[eb]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    load_k(0, 0);
    if (nt > 1) load_k(1, 1);
    load_v(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    scores(sA, 0);
    __syncthreads();

    int j = 0;
    for (; j + 2 < nt; j += 2) {
        step.template operator()<0, false>(j, sA, sB);
        step.template operator()<1, false>(j + 1, sB, sA);
    }
    if (j + 1 < nt) {
        step.template operator()<0, false>(j, sA, sB);
        step.template operator()<1, true>(j + 1, sB, sA);
    } else {
        step.template operator()<0, true>(j, sA, sB);
    }

    const float inv = 1.0f / half_swap_sum(l_run);
    if (q_ok) {
        bf16_t* op = reinterpret_cast<bf16_t*>(a.o) + qtok * a.ld_o + head * HD;
#pragma unroll
        for (int eb = 0; eb < 4; ++eb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = eb * 32 + 8 * i + 4 * h32;
                u32x2_v w = {pack2<DT>(o[eb][4 * i] * inv, o[eb][4 * i + 1] * inv),
                             pack2<DT>(o[eb][4 * i + 2] * inv, o[eb][4 * i + 3] * inv)};
                *reinterpret_cast<u32x2_v*>(op + e) = w;
            }
    }
}

template <int DT, int PITCH>
__global__ __launch_bounds__(64 * kWinWaves, 2) void window_attention_kernel(WinAttnArgs a) {
    window_attention_body<DT, PITCH>(a);
}

// fp32: one wave per (query, head); the window's scores in LDS (kT kH kW <= kWinMaxKeysF32).
__global__ __launch_bounds__(256) void window_attention_f32_kernel(WinAttnArgs a) {
    extern __shared__ float wsm[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nwin = a.kT * a.kH * a.kW;
    float* ss = wsm + wave * nwin;
    const int H = a.H, W = a.W;
    const long N = (long)a.T * H * W;
    const long qg = (long)blockIdx.x * 4 + wave;
    if (qg >= N * a.n_heads) return;          // whole waves only: no workgroup barrier below
    const int head = (int)(qg / N);
    const long tok = qg % N;
    const int t = (int)(tok / ((long)H * W)), h = (int)((tok / W) % H), w = (int)(tok % W);
    const int ts = win_start(t, a.rT, a.kT, a.T), hs = win_start(h, a.rH, a.kH, H), ws = win_start(w, a.rW, a.kW, W);
    const float* Q = reinterpret_cast<const float*>(a.q) + tok * a.ld_q + head * HD;
    const float* K = reinterpret_cast<const float*>(a.k) + head * HD;
    const float* V = reinterpret_cast<const float*>(a.v) + head * HD;
    auto key_tok = [&](int kk) -> long {
        const int ft = kk / (a.kH * a.kW), fh = (kk / a.kW) % a.kH, fw = kk % a.kW;
        return ((long)(ts + ft) * H + hs + fh) * W + ws + fw;
    };
    float mx = -INFINITY;
    for (int kk = lane; kk < nwin; kk += 64) {
        const float* kp = K + key_tok(kk) * a.ld_k;
        float s = 0.0f;
        for (int e = 0; e < HD; e += 4) {
            const f32x4_v qv = ldf4(Q + e), kv = ldf4(kp + e);
#pragma unroll
            for (int i = 0; i < 4; ++i) s = fmaf(qv[i], kv[i], s);
        }
        s *= a.scale;
        ss[kk] = s;
        mx = fmaxf(mx, s);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
    float sum = 0.0f;
    for (int kk = lane; kk < nwin; kk += 64) {
        const float p = expf(ss[kk] - mx);
        ss[kk] = p;
        sum += p;
    }
    sum = wave_sum(sum);
    // every lane's probabilities are in LDS before any lane reads another's
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float acc0 = 0.0f, acc1 = 0.0f;
    for (int kk = 0; kk < nwin; ++kk) {
        const float p = ss[kk];
        const float* vp = V + key_tok(kk) * a.ld_v;
        acc0 = fmaf(p, vp[lane], acc0);
        acc1 = fmaf(p, vp[lane + 64], acc1);
    }
    float* op = reinterpret_cast<float*>(a.o) + tok * a.ld_o + head * HD;
    op[lane] = acc0 / sum;
    op[lane + 64] = acc1 / sum;
}

hipError_t launch_window_attention(WinAttnArgs& a, hipStream_t s) {
    const long N = (long)a.T * a.H * a.W;
    if (N == 0 || a.n_heads == 0) return hipSuccess;
    if (a.dtype == BF16 || a.dtype == F16) {
        a.tiles_h = (a.H + WQH - 1) / WQH;
        a.tiles_w = (a.W + WQW - 1) / WQW;
        const dim3 grid((unsigned)((long)a.n_heads * a.T * a.tiles_h * a.tiles_w)), block(64 * kWinWaves);
        const bool narrow = WQW - 1 + a.kW <= 32;      // box rows fit 32 keys
        if (a.dtype == F16) {
            if (narrow) hipLaunchKernelGGL((window_attention_kernel<F16, 32>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((window_attention_kernel<F16, 64>), grid, block, 0, s, a);
        } else {
            if (narrow) hipLaunchKernelGGL((window_attention_kernel<BF16, 32>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((window_attention_kernel<BF16, 64>), grid, block, 0, s, a);
        }
    } else {
        const int nwin = a.kT * a.kH * a.kW;
        const long waves = N * a.n_heads;
        hipLaunchKernelGGL(window_attention_f32_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256),
                           (size_t)4 * nwin * sizeof(float), s, a);
    }
    return hipGetLastError();
}

}  // namespace dit
