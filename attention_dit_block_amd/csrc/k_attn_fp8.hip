// Joint softmax attention with fp8 (OCP e4m3) operands on gfx950: both of its products, the scores
// Q K^T and the output P V, run on v_mfma_scale_f32_32x32x64_f8f6f4, whose dense rate is twice the
// 16-bit MFMA's.  The pages weigh speed against accuracy (the "slight (invisible) loss of
// accuracy" reply that follows the cuBLAS split in the "CUDA codepath !" thread, antirez/iris.c
// issue #15); this is that trade for the attention.
//
// Operands: q, k, v as e4m3 codes [n_tok, n_heads * 128]; q carries one fp32 scale per token and
// head, k and v one per head, so every scale folds into a per-query factor (the exponent's FMA for
// q and k, the final normalisation for v) and costs nothing inside the key loop.
//
// A workgroup of 8 waves owns 256 queries of one head, each wave 32.  K and V tiles of 64 keys x
// 128 codes (8 KB) go from HBM straight into LDS (global_load_lds) through two 2-slot rings, as in
// the 16-bit kernel: at step j the workgroup loads K tile j+2 and V tile j+1 while it computes the
// scores of tile j+1 next to the softmax of tile j, then O += P_j V_j; one barrier per step.
//   S^T = K Q^T: K rows are the A operand, Q the B operand; a 32x32x64 MFMA takes 32 codes of
//     one row per lane (lanes 0-31 codes 0-31 of a 64-code slice, lanes 32-63 codes 32-63, on both
//     operands), so a head of 128 codes is two MFMAs per 32-key block.  The key loaded into A row
//     i of block b is chosen so that lane half h ends up holding the scores of keys
//     32 h + 16 b + r in its accumulator registers r = 0..15, in that order;
//   online softmax in base 2 and fp32, with the lazy running max of the 16-bit kernel (raised
//     only when a tile's max exceeds it by more than 2^8, so probabilities stay <= 256, inside
//     e4m3's range); the probabilities are rounded to e4m3 (v_cvt_pk_fp8_f32, nearest even) and
//     packed four to a register in register order: byte rho of lane half h is key 32 h + rho,
//     exactly the B operand (P^T) of the PV product, with no data movement between lanes;
//   O^T += V^T P^T: the A operand needs 32 keys of one feature per lane, a column of the
//     row-major V tile; ds_read_b64_tr_b8 transposes within 16-lane groups (lane j of a group
//     receives byte j % 8 of the 8-byte rows addressed by lanes j / 8, j / 8 + 2, .., j / 8 + 14),
//     so four such reads give lane l feature l % 32 of keys 32 h + 0 .. 31 in byte order rho.
// The running sum is taken over the fp32 probabilities (before their rounding to e4m3).  Each lane
// ends with 4 consecutive output features of one query per register group.  With a split scratch
// buffer (the block path) the units' key tiles are split as for the 16-bit kernel (attn_split.h).
#include "attn_common.h"
#include "attn_split.h"
#include "dev_common.h"
#include "launch.h"

namespace dit {

typedef int i32x8_v __attribute__((ext_vector_type(8)));
typedef int i32x2_v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_v lds_i32x2;

constexpr int kF8Tile = AK * HD;            // bytes of a K or V tile: 64 rows of 128 codes

__device__ __forceinline__ f32x16_v mfma_e4m3(const i32x8_v& a, const i32x8_v& b, const f32x16_v& c) {
    // e4m3 on both operands (format selectors 0), unit block scales (exponent 127 = 2^0)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Tile rows are 128 B, eight 16-byte chunks; chunk c of row r sits at position c ^ f8_swz(r).  The
// K fragment reads (16 lanes: rows differing in bits 0, 1, 2 and 5, one chunk) and the transposing
// V reads (32 lanes: 8 consecutive rows, two chunks, both 8-byte halves) then each cover distinct
// banks.
__device__ __forceinline__ int f8_swz(int r) { return (r & 6) | ((r >> 5) & 1); }
// Key (within the tile) loaded into A row i of S^T block b: lane half h = bit 2 of i holds rows
// 8 (r / 4) + 4 h + r % 4 in its registers r, which are then keys 32 h + 16 b + r.
__device__ __forceinline__ int f8_key(int b, int i) {
    return 32 * ((i >> 2) & 1) + 16 * b + 4 * (i >> 3) + (i & 3);
}

template <int OT>
__device__ __forceinline__ void store4(void* o, long ld_o, int row, int col, float a, float b, float c, float d) {
    if constexpr (OT == F32) {
        *reinterpret_cast<f32x4_v*>(reinterpret_cast<float*>(o) + (size_t)row * ld_o + col) = f32x4_v{a, b, c, d};
    } else {
        const u32x2_v w = {pack2<OT>(a, b), pack2<OT>(c, d)};
        *reinterpret_cast<u32x2_v*>(reinterpret_cast<bf16_t*>(o) + (size_t)row * ld_o + col) = w;
    }
}

// One (head, query tile) unit L = head * nq + query tile over key tiles [kb, ke); kind, g, gb, Gs,
// S, t_end, jn0, ckb, cke as for the split driver (attn_split.h).  Returns -1 or an owner's
// continuation.
template <int OT>
__device__ __forceinline__ int attention_unit_fp8(const AttnFp8Args& a, char* smem_k0, char* smem_k1, char* smem_v0,
                                                  char* smem_v1, int L, int kb, int ke, int kind, int g, int gb,
                                                  int Gs, long S, long t_end, int jn0, int& ckb, int& cke) {
    // The thread index goes through an opaque zero: the per-lane address arithmetic below is then
    // redone for each unit instead of being hoisted out of the persistent loop, where it would
    // hold registers across the whole kernel.
    int zero;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
    const int tid = threadIdx.x + zero, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h32 = lane >> 5, l32 = lane & 31;
    const int N = a.n_tok;
    const int nq = (N + AQ - 1) / AQ;
    const int head = L / nq, qt = L % nq;

    const char* Qg = reinterpret_cast<const char*>(a.q) + head * HD;
    const char* Kg = reinterpret_cast<const char*>(a.k) + head * HD;
    const char* Vg = reinterpret_cast<const char*>(a.v) + head * HD;

    // Q fragments (B operand of S^T): query qrow, codes 64 s + 32 h32 .. +31 of slice s
    const int qrow = qt * AQ + wave * 32 + l32;
    const int qr = min(qrow, N - 1);
    i32x8_v qf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const u32x4_v* p = reinterpret_cast<const u32x4_v*>(Qg + (size_t)qr * a.ld_q + 64 * s + 32 * h32);
        const u32x4_v lo = p[0], hi = p[1];
        qf[s] = i32x8_v{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    // scores in base 2: S_raw * (sq * sk * softmax_scale * log2(e)), one factor per query
    const float c2 = a.q_scale[(size_t)qr * a.n_heads + head] * a.k_scale[head] * a.scale * 1.4426950408889634f;

    // ---- load plan: wave w fills tile rows 8 w .. 8 w + 7 (1 KB, one instruction per tile); lane
    //      l writes LDS bytes 16 l .. +15 of that block: row 8 w + l / 8, position l % 8, which holds
    //      chunk (l % 8) ^ f8_swz(row)
    const int lrow = 8 * wave + (lane >> 3);
    const int lchunk = 16 * ((lane & 7) ^ f8_swz(lrow));
    const uint32_t k_b = (uint32_t)(lrow * a.ld_k + lchunk);
    const uint32_t v_b = (uint32_t)(lrow * a.ld_v + lchunk);
    // tile starting at key j0; rows past the last key repeat it (their scores are masked)
    auto load_tile = [&](const char* base, long ld, uint32_t off_b, char* dst, int j0) {
        const char* src = j0 + AK <= N ? base + (size_t)j0 * ld + off_b
                                       : base + (size_t)min(j0 + lrow, N - 1) * ld + lchunk;
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + wave * 1024), 16, 0, 0);
    };
    auto load_k = [&](int slot, int j0) { load_tile(Kg, a.ld_k, k_b, slot ? smem_k1 : smem_k0, j0); };
    auto load_v = [&](int slot, int j0) { load_tile(Vg, a.ld_v, v_b, slot ? smem_v1 : smem_v0, j0); };

    // ---- fragment read offsets (bytes within a ring slot)
    // K (A operand), slice s, half e: row f8_key(b, l32) (block b adds 16 rows), chunk 4 s + 2 h32 + e
    int k_off[2][2];
    {
        const int kr = f8_key(0, l32);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 2; ++e) k_off[s][e] = kr * 128 + 16 * ((4 * s + 2 * h32 + e) ^ f8_swz(kr));
    }
    // V^T (A operand), feature block fb, read r: lane j of 16-lane group G addresses row
    // 32 (G / 2) + 8 r + j / 2, chunk 2 fb + G % 2, half j % 2 (read r adds 8 rows)
    int v_off[4];
    {
        const int G = lane >> 4, j = lane & 15;
        const int vr = 32 * (G >> 1) + (j >> 1);
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) v_off[fb] = vr * 128 + 16 * ((2 * fb + (G & 1)) ^ f8_swz(vr)) + 8 * (j & 1);
    }

    // S^T = K Q^T for the 64 keys in K slot `slot` (two 32-key blocks, two 64-code slices each)
    auto scores = [&](f32x16_v* sd, int slot) {
        const char* kt = slot ? smem_k1 : smem_k0;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u32x4_v lo = *reinterpret_cast<const u32x4_v*>(kt + b * 2048 + k_off[s][0]);
                const u32x4_v hi = *reinterpret_cast<const u32x4_v*>(kt + b * 2048 + k_off[s][1]);
                const i32x8_v kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                sd[b] = s == 0 ? mfma_e4m3(kf, qf[0], f32x16_v{}) : mfma_e4m3(kf, qf[1], sd[b]);
            }
    };

    f32x16_v o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) o[i][q] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    f32x16_v sA[2], sB[2];

    // One pipeline step on tile j (ring slot P = j & 1): its scores are in SC; issue the loads of
    // K tile j + 2 and V tile j + 1, compute the scores of tile j + 1 into SN (unless LAST) while
    // the softmax of tile j runs, then O += P_j V_j.
    auto step = [&]<int P, bool LAST>(int j, f32x16_v* SC, f32x16_v* SN) {
        const int j0 = j * AK;
        if constexpr (!LAST) {
            if (j + 2 < ke) load_k(P, j0 + 2 * AK);
            load_v(P ^ 1, j0 + AK);
        }
        if constexpr (!LAST) scores(SN, P ^ 1);
        // register r of block b holds key j0 + 32 h32 + 16 b + r
        auto masked = [&](int b, int r) { return j0 + 32 * h32 + 16 * b + r >= N; };
        // probabilities against the running max -nm, rounded to e4m3 and packed: byte r % 4 of
        // word 4 b + r / 4 holds key 32 h32 + 16 b + r
        int pk[8];
        float lsum;
        auto probs = [&](float nm) {
            lsum = 0.0f;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    float p[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        p[u] = __builtin_amdgcn_exp2f(fmaf(SC[b][4 * t + u], c2, nm));
                        if constexpr (LAST)
                            if (masked(b, 4 * t + u)) p[u] = 0.0f;
                    }
                    lsum += (p[0] + p[1]) + (p[2] + p[3]);
                    int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                    pk[4 * b + t] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
                }
        };
        // First against the running max as it stands.  A lane whose sum stays below 2^kLazyMax has
        // every probability below it; only when some lane of the wave reaches it (a large score, or
        // the first tile: running max -inf) does the wave take the tile's max and recompute.
        probs(-m_run);
        float corr = 1.0f;
        bool raise = false;
        if (__builtin_amdgcn_ballot_w64(!(lsum < kLazyP))) {
            // the tile's max of S * c2 over this query's unmasked keys (c2 may be negative)
            float hi = -INFINITY, lo = INFINITY;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float s = SC[b][r];
                    const bool m = LAST && masked(b, r);
                    hi = fmaxf(hi, m ? -INFINITY : s);
                    lo = fminf(lo, m ? INFINITY : s);
                }
            const float mt = half_swap_max(c2 >= 0.0f ? hi * c2 : lo * c2);
            raise = mt > m_run + kLazyMax;
            const float m_new = raise ? mt : m_run;
            corr = __builtin_amdgcn_exp2f(m_run - m_new);    // 1 unless raised; 0 on tile 0
            m_run = m_new;
            if (__builtin_amdgcn_ballot_w64(raise)) probs(-m_new);
        }
        l_run = fmaf(l_run, corr, lsum);
        if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 16; ++q) o[i][q] *= corr;
        }
        // O^T += V^T P^T over the tile's 64 keys, one MFMA per 32-feature block
        const char* vt = P ? smem_v1 : smem_v0;
        const i32x8_v pv = {pk[0], pk[1], pk[2], pk[3], pk[4], pk[5], pk[6], pk[7]};
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) {
            i32x2_v r[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                r[rr] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vt + v_off[fb] + rr * 1024));
            const i32x8_v vf = {r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
            o[fb] = mfma_e4m3(vf, pv, o[fb]);
        }
        // the loads issued above have landed (own: waitcnt; every wave's: barrier), and every
        // wave is done with the slots the next step's loads overwrite
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    // prologue: K tiles kb and kb + 1, V tile kb; scores of tile kb
    load_k(0, kb * AK);
    if (kb + 1 < ke) load_k(1, (kb + 1) * AK);
    load_v(0, kb * AK);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    scores(sA, 0);
    __syncthreads();        // K slot 0 is refilled by step 0

    int j = kb;
    for (; j + 2 < ke; j += 2) {
        step.template operator()<0, false>(j, sA, sB);
        step.template operator()<1, false>(j + 1, sB, sA);
    }
    if (j + 1 < ke) {
        step.template operator()<0, false>(j, sA, sB);
        step.template operator()<1, true>(j + 1, sB, sA);
    } else {
        step.template operator()<0, true>(j, sA, sB);
    }

    const int fin = attn_split_finish(a, o, m_run, l_run, kind, g, gb, Gs, S, t_end, jn0, ckb, cke, wave, lane);
    if (fin != kAttnStore) return fin;
    if (qrow < N) {
        const float inv = a.v_scale[head] / half_swap_sum(l_run);
        const int col0 = head * HD + 4 * h32;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                store4<OT>(a.o, a.ld_o, qrow, col0 + 32 * fb + 8 * i, o[fb][4 * i] * inv, o[fb][4 * i + 1] * inv,
                           o[fb][4 * i + 2] * inv, o[fb][4 * i + 3] * inv);
    }
    return -1;
}

template <int OT>
__global__ __launch_bounds__(64 * kAttnWaves, 2) void attention_fp8_kernel(AttnFp8Args a) {
    __shared__ __attribute__((aligned(1024))) char smem_k0[kF8Tile];
    __shared__ __attribute__((aligned(1024))) char smem_k1[kF8Tile];
    __shared__ __attribute__((aligned(1024))) char smem_v0[kF8Tile];
    __shared__ __attribute__((aligned(1024))) char smem_v1[kF8Tile];
    attn_split_driver(a, [&](int L, int kb, int ke, int kind, int g, int gb, int Gs, long S, long t_end, int jn0,
                             int& ckb, int& cke) {
        return attention_unit_fp8<OT>(a, smem_k0, smem_k1, smem_v0, smem_v1, L, kb, ke, kind, g, gb, Gs, S, t_end,
                                      jn0, ckb, cke);
    });
}

hipError_t launch_attention_fp8(AttnFp8Args& a, hipStream_t s) {
    if (a.n_tok == 0) return hipSuccess;
    // 32-bit lane offsets: 63 rows of a tile past its start
    if (a.ld_k >= (1L << 25) || a.ld_v >= (1L << 25)) return hipErrorInvalidValue;
    const int nq = (a.n_tok + AQ - 1) / AQ;
    a.units = nq * a.n_heads;
    a.k_tiles = (a.n_tok + AK - 1) / AK;
    attn_plan_split(a, device_cu_count());
    const dim3 grid(a.sk_grid ? a.sk_grid : a.units), block(64 * kAttnWaves);
    // split: one workgroup per CU (the registers already allow only one; 64 KB of dynamic LDS past
    // the 32 KB rings makes that hold whatever the register budget)
    const unsigned pad = a.sk_grid ? 65536u : 0u;
    switch (a.o_dtype) {
        case F32: hipLaunchKernelGGL(attention_fp8_kernel<F32>, grid, block, pad, s, a); break;
        case F16: hipLaunchKernelGGL(attention_fp8_kernel<F16>, grid, block, pad, s, a); break;
        case BF16: hipLaunchKernelGGL(attention_fp8_kernel<BF16>, grid, block, pad, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dit
