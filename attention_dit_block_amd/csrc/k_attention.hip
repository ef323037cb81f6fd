// Joint softmax attention over the concatenated text+image sequence on gfx950 (the thread's
// "attention scores" matrix product and custom "softmax" kernel fused into one flash-style
// kernel; "joint attention" in the GGML update's bottom line of the "CUDA codepath !" thread,
// antirez/iris.c issue #15).  The scores are never written to memory.
//
// 16-bit kernel (bf16 or fp16 q, k, v).  A workgroup of 4 waves owns 128 queries of one head;
// each wave 32 queries.
// Per key tile of 64 keys (staged in LDS, K row-major and V transposed):
//   S^T = K Q^T  with v_mfma_f32_32x32x16_bf16 (K fragment = A operand, Q fragment = B), so a
//                lane holds 32 scores of ONE query: row max and row sum stay in the lane plus
//                one exchange with lane ^ 32;
//   online softmax in base 2, fp32;
//   O^T += V^T P^T  (V^T fragment = A operand, P^T = B operand).  The K fragment rows are
//                loaded in the key order that makes each lane's 8 consecutive score registers
//                exactly the 8 keys the P^T operand needs, so P goes from the score
//                accumulators to the PV MFMA without any cross-lane movement.  With bf16
//                operands P enters as two bf16 terms (high part + rounded remainder), so the PV
//                product carries the fp32 probabilities to 2^-16 relative instead of bf16's
//                2^-9; with fp16 operands one fp16 term (2^-11) is used.
// Each lane ends with 4 consecutive output features of one query per register group.
//
// fp32 kernel: LDS-tiled, 4 threads per query, fp32 FMA throughout.
#include "dev_common.h"
#include "launch.h"

namespace dit {

constexpr int AQ = 128;      // queries per workgroup
constexpr int AK = 64;       // keys per tile
constexpr int HD = 128;      // head dim

// Key held by S^T fragment row r of a 32-key block: bits 2 and 3 of r exchanged.
__device__ __forceinline__ int key_of_row(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <int DT> struct AFrag;
template <> struct AFrag<BF16> { typedef bf16x8_v T; };
template <> struct AFrag<F16> { typedef f16x8_v T; };

template <int DT>
__device__ __forceinline__ f32x16_v amfma(const typename AFrag<DT>::T& a, const typename AFrag<DT>::T& b,
                                          const f32x16_v& c) {
    if constexpr (DT == F16) return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int DT>
__global__ __launch_bounds__(256, 2) void attention_mfma_kernel(AttnArgs a) {
    typedef typename AFrag<DT>::T FragT;
    __shared__ __attribute__((aligned(1024))) char sK[AK * HD * 2];    // [key][e], 256 B rows
    __shared__ __attribute__((aligned(1024))) char sV[HD * AK * 2];    // [e][key], 128 B rows

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h32 = lane >> 5, l32 = lane & 31;
    // XCD-aware order: each XCD gets a contiguous range of (head, query tile) pairs.
    const int nq = (a.n_tok + AQ - 1) / AQ;
    const int nwg = gridDim.x;
    int L;
    {
        const int x = blockIdx.x & 7, idx = blockIdx.x >> 3, q = nwg >> 3, r = nwg & 7;
        L = x * q + min(x, r) + idx;
    }
    const int head = L / nq, qt = L % nq;
    const int N = a.n_tok;
    const float c2 = a.scale * 1.4426950408889634f;     // scores in base 2

    const bf16_t* Qg = reinterpret_cast<const bf16_t*>(a.q) + head * HD;
    const bf16_t* Kg = reinterpret_cast<const bf16_t*>(a.k) + head * HD;
    const bf16_t* Vg = reinterpret_cast<const bf16_t*>(a.v) + head * HD;

    // Q fragments (B operand of S^T): query l32 of this wave, features 16*es + 8*h32 .. +7.
    const int qrow = qt * AQ + wave * 32 + l32;
    FragT qf[8];
    {
        const bf16_t* qp = Qg + (size_t)min(qrow, N - 1) * a.ld_q + 8 * h32;
#pragma unroll
        for (int es = 0; es < 8; ++es) qf[es] = *reinterpret_cast<const FragT*>(qp + 16 * es);
    }

    // Loader assignment.  K: 1024 16-byte chunks per tile, chunk c = tid + 256 r (r < 4):
    // key c >> 4, feature chunk c & 15 (16 lanes per 256-byte row).  V: key pair kp = lane & 31,
    // feature chunk ec = (lane >> 5) + 2 * (wave + 4 r') (r' < 2): each lane reads keys 2kp and
    // 2kp+1 and writes packed key pairs into the transposed tile.
    u32x4_v kreg[4], vreg[2][2];
    auto load_tile = [&](int j0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = tid + 256 * r;
            const int key = min(j0 + (c >> 4), N - 1);
            kreg[r] = ld16(Kg + (size_t)key * a.ld_k + (c & 15) * 8);
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int ec = h32 + 2 * (wave + 4 * r);
            const int k0 = min(j0 + 2 * l32, N - 1), k1 = min(j0 + 2 * l32 + 1, N - 1);
            vreg[r][0] = ld16(Vg + (size_t)k0 * a.ld_v + ec * 8);
            vreg[r][1] = ld16(Vg + (size_t)k1 * a.ld_v + ec * 8);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = tid + 256 * r;
            const int key = c >> 4, ch = c & 15;
            *reinterpret_cast<u32x4_v*>(sK + key * 256 + ((ch ^ (key & 15)) << 4)) = kreg[r];
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int ec = h32 + 2 * (wave + 4 * r);
            const int kp = l32;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int e = ec * 8 + t;
                const uint32_t w0 = vreg[r][0][t >> 1], w1 = vreg[r][1][t >> 1];
                // (V[2kp][e], V[2kp+1][e]) packed low / high
                const uint32_t pk = (t & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                            : ((w0 & 0xffffu) | (w1 << 16));
                const int chunk = (kp >> 2) ^ (e & 7);
                *reinterpret_cast<uint32_t*>(sV + e * 128 + (chunk << 4) + ((kp & 3) << 2)) = pk;
            }
        }
    };

    f32x16_v o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) o[i][q] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    const int ntiles = (N + AK - 1) / AK;
    load_tile(0);
    store_tile();
    __syncthreads();

    for (int jt = 0; jt < ntiles; ++jt) {
        const int j0 = jt * AK;
        if (jt + 1 < ntiles) load_tile(j0 + AK);

        // ---- S^T = K Q^T for two 32-key blocks
        f32x16_v s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int q = 0; q < 16; ++q) s[kb][q] = 0.0f;
            const int key = kb * 32 + key_of_row(l32);
#pragma unroll
            for (int es = 0; es < 8; ++es) {
                const int ch = 2 * es + h32;
                const FragT kf = *reinterpret_cast<const FragT*>(sK + key * 256 + ((ch ^ (key & 15)) << 4));
                s[kb] = amfma<DT>(kf, qf[es], s[kb]);
            }
        }
        // register q of block kb holds key j0 + 32 kb + 16 (q >> 3) + 8 h32 + (q & 7)
        float tmax = -INFINITY;
        const bool tail = j0 + AK > N;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                float v = s[kb][q] * c2;
                if (tail) {
                    const int key = j0 + 32 * kb + 16 * (q >> 3) + 8 * h32 + (q & 7);
                    if (key >= N) v = -INFINITY;
                }
                s[kb][q] = v;
                tmax = fmaxf(tmax, v);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float corr = exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= corr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) o[i][q] *= corr;
        // bf16: P = P_hi + P_lo, both bf16: P_hi keeps the top 16 bits of the fp32 probability
        // (truncation), P_lo = bf16(p - P_hi) (exact difference, rounded to nearest even); the
        // pair carries p to 2^-16 relative (one bf16 term would be 2^-9).  fp16: one term,
        // rounded to nearest even (2^-11 relative).
        uint32_t ph[2][8], pl[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 16; q += 2) {
                const float p0 = exp2f(s[kb][q] - m_new), p1 = exp2f(s[kb][q + 1] - m_new);
                l_run += p0 + p1;
                if constexpr (DT == BF16) {
                    const uint32_t u0 = __float_as_uint(p0) & 0xffff0000u, u1 = __float_as_uint(p1) & 0xffff0000u;
                    ph[kb][q >> 1] = (u0 >> 16) | u1;
                    pl[kb][q >> 1] = pack_bf16x2(p0 - __uint_as_float(u0), p1 - __uint_as_float(u1));
                } else {
                    ph[kb][q >> 1] = pack_f16x2(p0, p1);
                }
            }
        // ---- O^T += V^T P^T: key step ks covers keys 16 ks .. 16 ks + 15 of the tile
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kb = ks >> 1, half = ks & 1;
            u32x4_v hv = {ph[kb][4 * half], ph[kb][4 * half + 1], ph[kb][4 * half + 2], ph[kb][4 * half + 3]};
            const FragT pfh = __builtin_bit_cast(FragT, hv);
            FragT vf[4];
#pragma unroll
            for (int eb = 0; eb < 4; ++eb) {
                const int e = eb * 32 + l32;
                const int ch = 2 * ks + h32;
                vf[eb] = *reinterpret_cast<const FragT*>(sV + e * 128 + ((ch ^ (e & 7)) << 4));
            }
#pragma unroll
            for (int eb = 0; eb < 4; ++eb) o[eb] = amfma<DT>(vf[eb], pfh, o[eb]);
            if constexpr (DT == BF16) {
                u32x4_v lv = {pl[kb][4 * half], pl[kb][4 * half + 1], pl[kb][4 * half + 2], pl[kb][4 * half + 3]};
                const FragT pfl = __builtin_bit_cast(FragT, lv);
#pragma unroll
                for (int eb = 0; eb < 4; ++eb) o[eb] = amfma<DT>(vf[eb], pfl, o[eb]);
            }
        }
        __syncthreads();
        if (jt + 1 < ntiles) {
            store_tile();
            __syncthreads();
        }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.0f / l_tot;
    if (qrow < N) {
        bf16_t* op = reinterpret_cast<bf16_t*>(a.o) + (size_t)qrow * a.ld_o + head * HD;
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

// ------------------------------------------------------------------------------------------
// fp32 attention: 64 queries per workgroup, 4 threads per query (32 features each), key tiles
// of 32 keys in LDS, online softmax in fp32.
// ------------------------------------------------------------------------------------------
constexpr int FQ = 64, FK = 32;

__global__ __launch_bounds__(256) void attention_f32_kernel(AttnArgs a) {
    __shared__ float sk[FK][HD + 4];
    __shared__ float sv[FK][HD + 4];
    const int nq = (a.n_tok + FQ - 1) / FQ;
    const int head = blockIdx.x / nq, qt = blockIdx.x % nq;
    const int tid = threadIdx.x;
    const int qi = tid >> 2, part = tid & 3;            // query, feature quarter
    const int N = a.n_tok;
    const int qrow = qt * FQ + qi;
    const float* qp = reinterpret_cast<const float*>(a.q) + (size_t)min(qrow, N - 1) * a.ld_q + head * HD + part * 32;
    float qv[32], ov[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) { qv[e] = qp[e] * a.scale; ov[e] = 0.0f; }
    float m_run = -INFINITY, l_run = 0.0f;
    const float* Kg = reinterpret_cast<const float*>(a.k) + head * HD;
    const float* Vg = reinterpret_cast<const float*>(a.v) + head * HD;
    for (int j0 = 0; j0 < N; j0 += FK) {
        __syncthreads();
        for (int c = tid; c < FK * HD / 4; c += 256) {
            const int key = c / (HD / 4), e4 = (c % (HD / 4)) * 4;
            const int kk = min(j0 + key, N - 1);
            const f32x4_v kv = ldf4(Kg + (size_t)kk * a.ld_k + e4), vv = ldf4(Vg + (size_t)kk * a.ld_v + e4);
#pragma unroll
            for (int t = 0; t < 4; ++t) { sk[key][e4 + t] = kv[t]; sv[key][e4 + t] = vv[t]; }
        }
        __syncthreads();
        const int nk = min(FK, N - j0);
        for (int j = 0; j < nk; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int e = 0; e < 32; ++e) s = fmaf(qv[e], sk[j][part * 32 + e], s);
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            const float m_new = fmaxf(m_run, s);
            const float corr = expf(m_run - m_new);
            const float p = expf(s - m_new);
            l_run = l_run * corr + p;
#pragma unroll
            for (int e = 0; e < 32; ++e) ov[e] = fmaf(p, sv[j][part * 32 + e], ov[e] * corr);
            m_run = m_new;
        }
    }
    if (qrow < N) {
        float* op = reinterpret_cast<float*>(a.o) + (size_t)qrow * a.ld_o + head * HD + part * 32;
        const float inv = 1.0f / l_run;
#pragma unroll
        for (int e = 0; e < 32; ++e) op[e] = ov[e] * inv;
    }
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
    if (a.n_tok == 0) return hipSuccess;
    if (a.dtype == BF16 || a.dtype == F16) {
        const int nq = (a.n_tok + AQ - 1) / AQ;
        if (a.dtype == F16) hipLaunchKernelGGL(attention_mfma_kernel<F16>, dim3(nq * a.n_heads), dim3(256), 0, s, a);
        else hipLaunchKernelGGL(attention_mfma_kernel<BF16>, dim3(nq * a.n_heads), dim3(256), 0, s, a);
    } else {
        const int nq = (a.n_tok + FQ - 1) / FQ;
        hipLaunchKernelGGL(attention_f32_kernel, dim3(nq * a.n_heads), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace dit
