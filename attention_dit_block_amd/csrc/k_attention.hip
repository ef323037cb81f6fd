// Joint softmax attention over the concatenated text+image sequence on gfx950 (the thread's
// "attention scores" matrix product and custom "softmax" kernel fused into one flash-style
// kernel; "joint attention" in the GGML update's bottom line of the "CUDA codepath !" thread,
// antirez/iris.c issue #15).  The scores are never written to memory.
//
// 16-bit kernel (bf16 or fp16 q, k, v).  A workgroup of 8 waves owns 256 queries of one head;
// each wave 32 queries.  K and V tiles of 64 keys go from HBM straight into LDS
// (global_load_lds, no VGPR staging) through two 2-slot rings: at step j the workgroup loads
// K tile j+2 and V tile j+1 while it computes the scores of tile j+1 (MFMA) next to the softmax
// of tile j (VALU) -- one pair of probabilities between consecutive score MFMAs, an order
// scheduling barriers hold -- then O += V_j P_j; one barrier per step.
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
// Work units are (head, 256-query tile) pairs.  With a stream-K scratch buffer (the block path) and
// a partly filled last round of units, a persistent grid of one workgroup per CU splits the
// remaining units' key tiles evenly; a unit's pieces are combined exactly like two halves of the
// online softmax (running max, running sum, unnormalised O), in a fixed order.  The split is local
// to each XCD: the XCD's workgroups take a contiguous block of units (a few heads), run their full
// rounds in step, then split only the rest of their block, so the K and V they read at any time
// are about one head's, which the XCD's L2 holds.
//
// fp32 kernel: LDS-tiled, 4 threads per query, fp32 FMA throughout.
#include "attn_common.h"
#include "attn_split.h"
#include "dev_common.h"
#include "launch.h"

namespace dit {

// One (head, query tile) unit L = head * nq + query tile over key tiles [kb, ke).
// NEG: softmax_scale < 0 (the row max of the scaled scores is then the min of the raw ones).
// Split units: g is the workgroup, gb the first workgroup of its segment (its XCD), Gs the
// segment's workgroups and S its stream-K key tiles; pieces are indexed within the segment.
// Returns -1, or (an owner whose piece jn did not arrive; its state is in its carry slot) the
// segment index jn of the next workgroup whose piece is still to be merged, with the missing
// piece's key tiles in [ckb, cke): the driver then runs that continuation as its next item.
template <int DT, bool NEG>
__device__ __forceinline__ int attention_unit(const AttnArgs& a, char* smem_k0, char* smem_k1, char* smem_v0,
                                              char* smem_v1, int L, int kb, int ke, int kind, int g, int gb, int Gs,
                                              long S, long t_end, int jn0, int& ckb, int& cke) {
    constexpr int LPW = 16 / kAttnWaves;    // 1 KB load instructions per wave per K (or V) tile
    typedef typename AFrag<DT>::T FragT;
    // The two slots of the K ring and of the V ring are LDS arrays of their own, so the compiler
    // can tell that the fragment reads of one slot do not touch the slot whose global -> LDS
    // loads are in flight (it would otherwise wait for those loads before the reads)

    // The thread index goes through an opaque zero: the per-lane address arithmetic below is then
    // redone for each unit instead of being hoisted out of the persistent loop, where it would
    // hold registers across the whole kernel.
    int zero;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
    const int tid = threadIdx.x + zero, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h32 = lane >> 5, l32 = lane & 31;
    // the key range is wave-uniform (an owner's continuation takes it from a flag word every lane
    // read): scalar loop control and scalar tile addresses
    kb = __builtin_amdgcn_readfirstlane(kb);
    ke = __builtin_amdgcn_readfirstlane(ke);
    const int nq = (a.n_tok + AQ - 1) / AQ;
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

    // ---- load plan.  A tile is 16 load instructions of 1 KB; wave w issues instructions
    //      LPW*w .. LPW*w + LPW-1 of the K tile and of the V tile.  Instruction i fills rows
    //      16 (i%4) .. +15 of slab i/4; lane l writes LDS bytes l*16 .. +15 of the 1 KB block: row
    //      16 (i%4) + l/4, position l%4, which holds chunk kpos(row, l%4) = (l%4) ^ (l/16) (K) or
    //      chunk l%4 (V) of the slab row.
    const int slab = (LPW * wave) >> 2, rg0 = (LPW * wave) & 3;
    const uint32_t k_b = (uint32_t)((lane >> 2) * a.ld_k + 32 * slab + 8 * ((lane & 3) ^ (lane >> 4))) * 2u;
    const uint32_t v_b = (uint32_t)((lane >> 2) * a.ld_v + 32 * slab + 8 * (lane & 3)) * 2u;
    const size_t k_rstep = (size_t)16 * a.ld_k * 2;          // bytes between instructions r, r+1
    const size_t v_rstep = (size_t)16 * a.ld_v * 2;
    // tiles starting at key j0 into ring slot `slot`; rows past the last key repeat it
    auto load_k = [&](int slot, int j0) {
        char* dst = slot ? smem_k1 : smem_k0;
        if (j0 + AK <= N) {
            const char* t = reinterpret_cast<const char*>(Kg + (size_t)j0 * a.ld_k);
#pragma unroll
            for (int r = 0; r < LPW; ++r)
                __builtin_amdgcn_global_load_lds(t + (rg0 + r) * k_rstep + k_b,
                                                 (lds_void*)(dst + (LPW * wave + r) * 1024), 16, 0, 0);
        } else {
#pragma unroll
            for (int r = 0; r < LPW; ++r) {
                const int key = min(j0 + 16 * (rg0 + r) + (lane >> 2), N - 1);
                __builtin_amdgcn_global_load_lds(Kg + (size_t)key * a.ld_k + 32 * slab + 8 * ((lane & 3) ^ (lane >> 4)),
                                                 (lds_void*)(dst + (LPW * wave + r) * 1024), 16, 0, 0);
            }
        }
    };
    auto load_v = [&](int slot, int j0) {
        char* dst = slot ? smem_v1 : smem_v0;
        if (j0 + AK <= N) {
            const char* t = reinterpret_cast<const char*>(Vg + (size_t)j0 * a.ld_v);
#pragma unroll
            for (int r = 0; r < LPW; ++r)
                __builtin_amdgcn_global_load_lds(t + (rg0 + r) * v_rstep + v_b,
                                                 (lds_void*)(dst + (LPW * wave + r) * 1024), 16, 0, 0);
        } else {
#pragma unroll
            for (int r = 0; r < LPW; ++r) {
                const int key = min(j0 + 16 * (rg0 + r) + (lane >> 2), N - 1);
                __builtin_amdgcn_global_load_lds(Vg + (size_t)key * a.ld_v + 32 * slab + 8 * (lane & 3),
                                                 (lds_void*)(dst + (LPW * wave + r) * 1024), 16, 0, 0);
            }
        }
    };

    // ---- fragment read offsets (bytes within a ring slot).
    // K fragment (block kb, feature step es): row 32 kb + key_of_row(l32) of slab es / 2, chunk
    // 2 (es % 2) + h32 of the slab row.
    int k_off[2];
    {
        const int kr = key_of_row(l32);
        k_off[0] = kr * 64 + (kpos(kr, h32) << 4);
        k_off[1] = kr * 64 + (kpos(kr, 2 + h32) << 4);
    }
    // V^T fragment (feature block eb, key step ks, half hf): lane i = lane % 16 of group
    // g = lane / 16 addresses slab eb, row 16 ks + 8 (g >> 1) + 4 hf + i / 4, features
    // 16 (g & 1) + 4 (i % 4) .. +3 of the slab.
    const int v_off = (8 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) * 64 + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

    // S^T = K Q^T for the 64 keys in K slot `slot` (two 32-key blocks)
    auto scores = [&](f32x16_v* sd, int slot) {
        const char* kt = slot ? smem_k1 : smem_k0;
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
    float m_run = -INFINITY, l_run = 0.0f;
    f32x16_v sA[2], sB[2];

    // One pipeline step on tile j (P = (j - kb) & 1): its scores are in SC; issue the loads of K
    // tile j + 2 and V tile j + 1, compute the scores of tile j + 1 into SN (unless LAST) while the
    // softmax of tile j runs, then O += V_j P_j.
    auto step = [&]<int P, bool LAST>(int j, f32x16_v* SC, f32x16_v* SN) {
        const int j0 = j * AK;
        if constexpr (!LAST) {
            if (j + 2 < ke) load_k(P, j0 + 2 * AK);
            load_v(P ^ 1, j0 + AK);
        }
        // ---- region 1: S(j+1) MFMAs with the softmax of tile j
        // register q of block kb holds key j0 + 32 kb + 16 (q >> 3) + 8 h32 + (q & 7)
        auto masked = [&](int kb, int q) { return j0 + 32 * kb + 16 * (q >> 3) + 8 * h32 + (q & 7) >= N; };
        if constexpr (LAST) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (masked(kb, q)) SC[kb][q] = NEG ? INFINITY : -INFINITY;
        }
        // probabilities against running max nm = -m, packed as the PV operand: word 4 ks + t of ph
        // (pl) holds keys 16 ks + 8 h32 + 2t, +1 (registers 8 (ks & 1) + 2t, +1 of block ks >> 1)
        uint32_t ph[16], pl[DT == BF16 ? 16 : 1];
        float lsum;
        auto probs = [&](float nm) {
            lsum = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q = 0; q < 16; q += 2) {
                    float p0 = __builtin_amdgcn_exp2f(fmaf(SC[kb][q], c2, nm));
                    float p1 = __builtin_amdgcn_exp2f(fmaf(SC[kb][q + 1], c2, nm));
                    if constexpr (LAST) {
                        if (masked(kb, q)) p0 = 0.0f;
                        if (masked(kb, q + 1)) p1 = 0.0f;
                    }
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
        };
        // First against the running max as it stands.  A lane whose sum stays below 2^kLazyMax has
        // every probability below it, so no score of its query exceeds the running max by
        // kLazyMax and the max is not raised; only when some lane of the wave reaches it (a large
        // score, or the first tile: running max -inf) does the wave take the tile's max and
        // recompute, which gives the same values as taking the max first.
        if constexpr (LAST) {
            probs(-m_run);
        } else {
            // the 16 score MFMAs of tile j + 1 (the two 32-key chains alternating, each in feature
            // order), each K fragment read one MFMA ahead, and between consecutive MFMAs one pair of
            // tile j's probabilities (in probs' order); the scheduling barriers keep this order, so
            // the exponentials issue while the matrix pipe works
            const char* kt = (P ^ 1) ? smem_k1 : smem_k0;
            auto kfrag = [&](int i) {
                const int kb = i & 1, es = i >> 1;
                return *reinterpret_cast<const FragT*>(kt + (es >> 1) * 4096 + kb * 32 * 64 + k_off[es & 1]);
            };
            const float nm = -m_run;
            lsum = 0.0f;
            FragT kf_next = kfrag(0), kf_next2 = kfrag(1);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const FragT kf = kf_next;
                kf_next = kf_next2;
                if (i < 14) kf_next2 = kfrag(i + 2);
                const int kb = i & 1, es = i >> 1;
                SN[kb] = es == 0 ? amfma<DT>(kf, qf[es], f32x16_v{}) : amfma<DT>(kf, qf[es], SN[kb]);
                const int kc = i >> 3, q = 2 * (i & 7);
                const float p0 = __builtin_amdgcn_exp2f(fmaf(SC[kc][q], c2, nm));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(SC[kc][q + 1], c2, nm));
                lsum += p0 + p1;
                const int w = 8 * kc + (q >> 1);
                if constexpr (DT == BF16) {
                    const uint32_t u0 = __float_as_uint(p0) & 0xffff0000u, u1 = __float_as_uint(p1) & 0xffff0000u;
                    ph[w] = (u0 >> 16) | u1;
                    pl[w] = pack_bf16x2(p0 - __uint_as_float(u0), p1 - __uint_as_float(u1));
                } else {
                    ph[w] = pack_f16x2(p0, p1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        float corr = 1.0f;
        bool raise = false;
        if (__builtin_amdgcn_ballot_w64(!(lsum < kLazyP))) {
            float e0 = SC[0][0], e1 = SC[1][0];
#pragma unroll
            for (int q = 1; q < 16; ++q) {
                e0 = NEG ? fminf(e0, SC[0][q]) : fmaxf(e0, SC[0][q]);
                e1 = NEG ? fminf(e1, SC[1][q]) : fmaxf(e1, SC[1][q]);
            }
            const float mt = (NEG ? -half_swap_max(-fminf(e0, e1)) : half_swap_max(fmaxf(e0, e1))) * c2;
            // raise the running max only when this tile's max exceeds it by more than kLazyMax
            raise = mt > m_run + kLazyMax;
            const float m_new = raise ? mt : m_run;
            corr = __builtin_amdgcn_exp2f(m_run - m_new);    // 1 unless raised; 0 on tile 0
            m_run = m_new;
            if (__builtin_amdgcn_ballot_w64(raise)) probs(-m_new);
        }
        // keep the probabilities next to the score MFMAs of the following tile (they would
        // otherwise sink past the rescale branch below, into the PV phase); emits no code
        asm volatile("" ::"v"(ph[0]), "v"(ph[1]), "v"(ph[2]), "v"(ph[3]), "v"(ph[4]), "v"(ph[5]), "v"(ph[6]),
                     "v"(ph[7]), "v"(ph[8]), "v"(ph[9]), "v"(ph[10]), "v"(ph[11]), "v"(ph[12]), "v"(ph[13]),
                     "v"(ph[14]), "v"(ph[15]), "v"(lsum));
        if constexpr (DT == BF16)
            asm volatile("" ::"v"(pl[0]), "v"(pl[1]), "v"(pl[2]), "v"(pl[3]), "v"(pl[4]), "v"(pl[5]), "v"(pl[6]),
                         "v"(pl[7]), "v"(pl[8]), "v"(pl[9]), "v"(pl[10]), "v"(pl[11]), "v"(pl[12]), "v"(pl[13]),
                         "v"(pl[14]), "v"(pl[15]));
        l_run = fmaf(l_run, corr, lsum);
        if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 16; ++q) o[i][q] *= corr;
        }
        // ---- region 2: O^T += V^T P^T; key step ks covers keys 16 ks .. +15 of the tile
        const char* vt = P ? smem_v1 : smem_v0;
        // one V^T fragment read ahead of its MFMA
        auto read_v1 = [&](int i) {
            const int ks = i >> 2, eb = i & 3;
            const char* vp = vt + v_off + eb * 4096 + ks * 16 * 64;
            const s16x4_v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp));
            const s16x4_v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 4 * 64));
            const s16x8_v w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(FragT, w);
        };
        FragT vn = read_v1(0), vn2 = read_v1(1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const FragT vc = vn;
            vn = vn2;
            if (i < 14) vn2 = read_v1(i + 2);
            const int ks = i >> 2, eb = i & 3;
            const u32x4_v hv = {ph[4 * ks], ph[4 * ks + 1], ph[4 * ks + 2], ph[4 * ks + 3]};
            o[eb] = amfma<DT>(vc, __builtin_bit_cast(FragT, hv), o[eb]);
            if constexpr (DT == BF16) {
                const u32x4_v lv = {pl[4 * ks], pl[4 * ks + 1], pl[4 * ks + 2], pl[4 * ks + 3]};
                o[eb] = amfma<DT>(vc, __builtin_bit_cast(FragT, lv), o[eb]);
            }
            __builtin_amdgcn_sched_barrier(0);
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
    return -1;
}

// The split driver (attn_split.h) runs the work items of workgroup blockIdx.x.
template <int DT, bool NEG>
__device__ __forceinline__ void attention_mfma_body(const AttnArgs& a) {
    __shared__ __attribute__((aligned(1024))) char smem_k0[kTile];
    __shared__ __attribute__((aligned(1024))) char smem_k1[kTile];
    __shared__ __attribute__((aligned(1024))) char smem_v0[kTile];
    __shared__ __attribute__((aligned(1024))) char smem_v1[kTile];
    attn_split_driver(a, [&](int L, int kb, int ke, int kind, int g, int gb, int Gs, long S, long t_end, int jn0,
                             int& ckb, int& cke) {
        return attention_unit<DT, NEG>(a, smem_k0, smem_k1, smem_v0, smem_v1, L, kb, ke, kind, g, gb, Gs, S, t_end,
                                       jn0, ckb, cke);
    });
}

// Fixed launch bounds (they must not depend on a template parameter: hipcc then emits no host
// launch stub).
template <int DT, bool NEG>
__global__ __launch_bounds__(64 * kAttnWaves, 2) void attention_mfma_kernel(AttnArgs a) {
    attention_mfma_body<DT, NEG>(a);
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

size_t attention_sk_scratch_bytes() {
    const int G = device_cu_count();
    return G > 0 ? (size_t)G * (2 * (size_t)kSlotF4 * 16 + 8) : 0;
}

hipError_t launch_attention(AttnArgs& a, hipStream_t s) {
    if (a.n_tok == 0) return hipSuccess;
    if (a.dtype == BF16 || a.dtype == F16) {
        const int nq = (a.n_tok + AQ - 1) / AQ;
        const int G = device_cu_count();
        a.units = nq * a.n_heads;
        a.k_tiles = (a.n_tok + AK - 1) / AK;
        attn_plan_split(a, G);
        const dim3 grid(a.sk_grid ? a.sk_grid : a.units), block(64 * kAttnWaves);
        // Stream-K: one workgroup per CU, all resident at once (owners wait for later workgroups).
        // The register budget already allows only one per CU; unused dynamic LDS past the 64 KB
        // rings (more than half of the CU's 160 KB taken) makes that hold whatever the budget.
        const unsigned pad = a.sk_grid ? 32768u : 0u;
        const bool neg = a.scale < 0.0f;
        if (a.dtype == F16) {
            if (neg) hipLaunchKernelGGL((attention_mfma_kernel<F16, true>), grid, block, pad, s, a);
            else hipLaunchKernelGGL((attention_mfma_kernel<F16, false>), grid, block, pad, s, a);
        } else {
            if (neg) hipLaunchKernelGGL((attention_mfma_kernel<BF16, true>), grid, block, pad, s, a);
            else hipLaunchKernelGGL((attention_mfma_kernel<BF16, false>), grid, block, pad, s, a);
        }
    } else {
        const int nq = (a.n_tok + FQ - 1) / FQ;
        hipLaunchKernelGGL(attention_f32_kernel, dim3(nq * a.n_heads), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace dit
