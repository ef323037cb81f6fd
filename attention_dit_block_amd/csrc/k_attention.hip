// Joint softmax attention over the concatenated text+image sequence on gfx950 (the thread's
// "attention scores" matrix product and custom "softmax" kernel fused into one flash-style
// kernel; "joint attention" in the GGML update's bottom line of the "CUDA codepath !" thread,
// antirez/iris.c issue #15).  The scores are never written to memory.
//
// 16-bit kernel (bf16 or fp16 q, k, v).  A workgroup of 4 waves owns 128 queries of one head;
// each wave 32 queries.  K and V tiles of 64 keys go from HBM straight into LDS
// (global_load_lds, no VGPR staging), double-buffered: the next tile's loads are issued at the
// start of a tile and awaited at its end, behind one barrier per tile.
// Per key tile:
//   S^T = K Q^T  with v_mfma_f32_32x32x16 (K fragment = A operand, Q fragment = B), so a lane
//                holds 32 scores of ONE query: the row max needs one swap with lane ^ 32;
//   online softmax in base 2, fp32, with the softmax scale folded into the exponent's FMA.  The
//                running max is raised only when a tile's max exceeds it by more than 2^8
//                (probabilities then stay <= 256), so the O rescale is skipped on most tiles;
//   O^T += V^T P^T  (V^T fragment = A operand, P^T = B operand).  V stays row-major in LDS; the
//                V^T fragment comes from ds_read_b64_tr_b16, which hands lane j of each 16-lane
//                group element j%4 of the 8-byte rows addressed by lanes j/4, j/4+4, j/4+8,
//                j/4+12 -- with lane i addressing key k0 + i/4, features e0 + 4(i%4) .. +3, lane j
//                receives keys k0 .. k0+3 of feature e0 + j.  The K fragment rows are loaded in
//                the key order that makes each lane's 8 consecutive score registers exactly the
//                8 keys the P^T operand needs, so P goes from the score accumulators to the PV
//                MFMA without any cross-lane movement.  With fp16 operands P enters as one fp16
//                term (2^-11 relative); with bf16 operands as two bf16 terms (high part +
//                rounded remainder, 2^-16 relative instead of bf16's 2^-9).  The row sum is
//                taken over the fp32 probabilities.
// Each lane ends with 4 consecutive output features of one query per register group.
//
// fp32 kernel: LDS-tiled, 4 threads per query, fp32 FMA throughout.
#include "dev_common.h"
#include "launch.h"

namespace dit {

constexpr int AQ = 128;      // queries per workgroup
constexpr int AK = 64;       // keys per tile
constexpr int HD = 128;      // head dim
constexpr int kTile = AK * HD * 2;          // bytes of one K (or V) tile: 64 rows of 256 B
constexpr float kLazyMax = 8.0f;            // log2 of the largest unnormalised probability

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4_v __attribute__((ext_vector_type(4)));
typedef short s16x8_v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_v lds_s16x4;

// Key held by S^T fragment row r of a 32-key block: bits 2 and 3 of r exchanged.
__device__ __forceinline__ int key_of_row(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
// LDS rows are 16 chunks of 16 B.  K: chunk c of row r sits at position c ^ (r & 15), so the 16
// lanes of a ds_read_b128 (16 keys, one chunk) hit 16 different bank groups.  V: position
// c ^ ((r & 3) << 2), so the 4 rows read by each half-wave of a transposing read land in 4
// different 64-byte bank ranges.
__device__ __forceinline__ int kpos(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int vpos(int r, int c) { return c ^ ((r & 3) << 2); }

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

template <int DT>
__global__ __launch_bounds__(256, 2) void attention_mfma_kernel(AttnArgs a) {
    typedef typename AFrag<DT>::T FragT;
    // two stages of [K tile | V tile]
    __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * kTile];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h32 = lane >> 5, l32 = lane & 31;
    // XCD-aware order: each XCD gets a contiguous range of (head, query tile) pairs, so the
    // workgroups sharing one head's K and V run on one L2.
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

    // ---- load plan.  Each tile is 16 K and 16 V load instructions of 1 KB (4 rows); wave w
    //      issues instructions 4w .. 4w+3 of each.  Lane l writes LDS bytes l*16 .. +15 of the
    //      1 KB block: row 4i + l/16, position l%16, which holds chunk kpos / vpos of it.
    const int lrow = lane >> 4, lp = lane & 15;
    int k_el[4], v_el[4];        // element offset of the lane's chunk within its row
    int t_row[4];                // tile row of instruction r
    uint32_t k_b[4], v_b[4];     // byte offset of the lane's chunk from the tile's first row
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * (4 * wave + r) + lrow;
        t_row[r] = row;
        k_el[r] = kpos(row, lp) * 8;
        v_el[r] = vpos(row, lp) * 8;
        k_b[r] = (uint32_t)(row * a.ld_k + k_el[r]) * 2u;
        v_b[r] = (uint32_t)(row * a.ld_v + v_el[r]) * 2u;
    }
    auto load_tile = [&](int stage, int j0, bool clamp) {
        char* base = smem + stage * 2 * kTile;
        if (!clamp) {
            const char* kt = reinterpret_cast<const char*>(Kg + (size_t)j0 * a.ld_k);
            const char* vt = reinterpret_cast<const char*>(Vg + (size_t)j0 * a.ld_v);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                __builtin_amdgcn_global_load_lds(kt + k_b[r], (lds_void*)(base + (4 * wave + r) * 1024), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vt + v_b[r], (lds_void*)(base + kTile + (4 * wave + r) * 1024),
                                                 16, 0, 0);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = min(j0 + t_row[r], N - 1);
                __builtin_amdgcn_global_load_lds(Kg + (size_t)key * a.ld_k + k_el[r],
                                                 (lds_void*)(base + (4 * wave + r) * 1024), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(Vg + (size_t)key * a.ld_v + v_el[r],
                                                 (lds_void*)(base + kTile + (4 * wave + r) * 1024), 16, 0, 0);
            }
        }
    };

    // ---- fragment read offsets (bytes within a stage).
    // K fragment (block kb, feature step es): row 32 kb + key_of_row(l32), chunk 2 es + h32.
    int k_off[8];
    {
        const int kr = key_of_row(l32);
#pragma unroll
        for (int es = 0; es < 8; ++es) k_off[es] = kr * 256 + (kpos(kr, 2 * es + h32) << 4);
    }
    // V^T fragment (feature block eb, key step ks, half hf): lane i = lane % 16 of group
    // g = lane / 16 addresses row 16 ks + 8 (g >> 1) + 4 hf + i / 4, features
    // 32 eb + 16 (g & 1) + 4 (i % 4) .. +3.
    int v_off[4];
    {
        const int g = lane >> 4, i = lane & 15;
        const int row = 8 * (g >> 1) + (i >> 2);                 // + 16 ks + 4 hf (row & 3 unchanged)
#pragma unroll
        for (int eb = 0; eb < 4; ++eb) {
            const int e = 32 * eb + 16 * (g & 1) + 4 * (i & 3);
            v_off[eb] = kTile + row * 256 + (vpos(row, e >> 3) << 4) + (e & 7) * 2;
        }
    }

    f32x16_v o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) o[i][q] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    const int ntiles = (N + AK - 1) / AK;
    // One key tile on stage STAGE.  TAIL: the tile runs past the last key.
    auto tile = [&]<int STAGE, bool TAIL>(int jt) {
        const int j0 = jt * AK;
        if (jt + 1 < ntiles) load_tile(STAGE ^ 1, j0 + AK, j0 + 2 * AK > N);
        const char* st = smem + STAGE * 2 * kTile;

        // ---- S^T = K Q^T for two 32-key blocks
        f32x16_v s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int q = 0; q < 16; ++q) s[kb][q] = 0.0f;
#pragma unroll
            for (int es = 0; es < 8; ++es) {
                const FragT kf = *reinterpret_cast<const FragT*>(st + kb * 32 * 256 + k_off[es]);
                s[kb] = amfma<DT>(kf, qf[es], s[kb]);
            }
        }
        // register q of block kb holds key j0 + 32 kb + 16 (q >> 3) + 8 h32 + (q & 7).  The row
        // max of s * c2 is c2 times the max of s (c2 >= 0) or the min of s (c2 < 0); keys past
        // the end take the value that drops out of that reduction, and probability 0 below.
        auto masked = [&](int kb, int q) { return j0 + 32 * kb + 16 * (q >> 3) + 8 * h32 + (q & 7) >= N; };
        float mt;
        if (c2 >= 0.0f) {
            if constexpr (TAIL) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        if (masked(kb, q)) s[kb][q] = -INFINITY;
            }
            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q = 0; q < 16; ++q) mx = fmaxf(mx, s[kb][q]);
            mt = half_swap_max(mx) * c2;
        } else {
            if constexpr (TAIL) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        if (masked(kb, q)) s[kb][q] = INFINITY;
            }
            float mn = s[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q = 0; q < 16; ++q) mn = fminf(mn, s[kb][q]);
            mt = -half_swap_max(-mn) * c2;
        }
        // raise the running max only when this tile's max exceeds it by more than 2^kLazyMax
        const bool raise = mt > m_run + kLazyMax;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float m_new = raise ? mt : m_run;
            const float corr = __builtin_amdgcn_exp2f(m_run - m_new);    // 0 on the first tile
            m_run = m_new;
            l_run *= corr;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 16; ++q) o[i][q] *= corr;
        }
        // probabilities, in place of the scores
        const float nm = -m_run;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                s[kb][q] = __builtin_amdgcn_exp2f(fmaf(s[kb][q], c2, nm));
                if constexpr (TAIL) {
                    if (masked(kb, q)) s[kb][q] = 0.0f;
                }
            }
        // ---- O^T += V^T P^T: key step ks covers keys 16 ks .. 16 ks + 15 of the tile, held in
        //      registers 8 (ks & 1) .. +7 of block ks >> 1
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kb = ks >> 1, q0 = 8 * (ks & 1);
            u32x4_v hv, lv;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float p0 = s[kb][q0 + 2 * t], p1 = s[kb][q0 + 2 * t + 1];
                l_run += p0 + p1;
                if constexpr (DT == BF16) {
                    const uint32_t u0 = __float_as_uint(p0) & 0xffff0000u, u1 = __float_as_uint(p1) & 0xffff0000u;
                    hv[t] = (u0 >> 16) | u1;
                    lv[t] = pack_bf16x2(p0 - __uint_as_float(u0), p1 - __uint_as_float(u1));
                } else {
                    hv[t] = pack_f16x2(p0, p1);
                }
            }
            const FragT pfh = __builtin_bit_cast(FragT, hv);
            FragT vf[4];
#pragma unroll
            for (int eb = 0; eb < 4; ++eb) {
                const char* vp = st + v_off[eb] + ks * 16 * 256;
                const s16x4_v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp));
                const s16x4_v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 4 * 256));
                const s16x8_v w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                vf[eb] = __builtin_bit_cast(FragT, w);
            }
#pragma unroll
            for (int eb = 0; eb < 4; ++eb) o[eb] = amfma<DT>(vf[eb], pfh, o[eb]);
            if constexpr (DT == BF16) {
                const FragT pfl = __builtin_bit_cast(FragT, lv);
#pragma unroll
                for (int eb = 0; eb < 4; ++eb) o[eb] = amfma<DT>(vf[eb], pfl, o[eb]);
            }
        }
        // the next tile has landed in LDS (own loads), for every wave (barrier); every wave is
        // done reading this stage before the following tile's loads overwrite it
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    load_tile(0, 0, AK > N);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int nfull = N / AK;                 // tiles with no key past the end
    int jt = 0;
    for (; jt + 1 < nfull; jt += 2) {
        tile.template operator()<0, false>(jt);
        tile.template operator()<1, false>(jt + 1);
    }
    if (jt < nfull) {
        tile.template operator()<0, false>(jt);
        if (++jt < ntiles) tile.template operator()<1, true>(jt);
    } else if (jt < ntiles) {
        tile.template operator()<0, true>(jt);
    }

    const float inv = 1.0f / half_swap_sum(l_run);
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
