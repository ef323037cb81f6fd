// The key split of the joint-attention kernels (16-bit and e4m3 operands): when the last round of
// (head, 256-query) units leaves CUs idle, a persistent grid of one workgroup per CU runs the full
// rounds but one and splits the remaining units' key tiles evenly, within each XCD.  A unit's
// pieces are partial online-softmax states (running max m, running sum l, unnormalised O, per
// query); the workgroup holding the unit's first keys merges the others' in a fixed order:
// m = max(m_a, m_b), O = O_a 2^(m_a - m) + O_b 2^(m_b - m), l likewise -- the rule the online softmax
// applies between two key tiles.  The hand-over (partial, flag, claiming a piece that did not
// arrive) is the plumbing of dev_common.h.
//
// Both kernels keep the same per-lane state: 8 waves of 32 queries, O^T in four 32 x 32 MFMA
// accumulator blocks (lane l: query l % 32), and a running max and a running sum per lane.  A
// kernel's argument struct A carries sk_scratch, sk_grid, sk_segs, units, k_tiles, epoch and
// sk_spins.
#pragma once

#include "dev_common.h"
#include "launch.h"

namespace dit {

// waves (of 32 queries each) per workgroup: 8, one workgroup per CU, so each staged K/V tile
// serves 256 queries (4-wave workgroups, two per CU, measured slower: 342 against 277 us at 4608
// tokens, 4.33 against 3.36 ms at 16896)
constexpr int kAttnWaves = 8;
constexpr int AQ = 32 * kAttnWaves;     // queries per workgroup
// How a workgroup finishes a (head, query tile) unit it ran key tiles [kb, ke) of:
enum UnitKind {
    UNIT_FULL = 0,      // all key tiles: normalise and store O
    UNIT_OWNER = 1,     // key tiles from 0: merge the partials of the workgroups holding the rest, store
    UNIT_PARTIAL = 2,   // later key tiles: publish (running max, running sum, unnormalised O)
    UNIT_OWNER_CONT = 3 // an owner's continuation: key tiles of a piece whose partial did not arrive,
                        // merged with the owner's state from its carry slot, then as UNIT_OWNER
};

// Split scratch: [sk_grid] partial slots, [sk_grid] carry slots (an owner's state while it
// computes a missing piece), then [sk_grid] 32-bit flags.  In a slot, lane l of wave w keeps float4
// c (c < 16: its O accumulators; c = 16: running max, running sum) at index (w * 17 + c) * 64 + l.
constexpr int kPartF4 = 17;
constexpr int kSlotF4 = kAttnWaves * kPartF4 * 64;
template <class A>
__device__ __forceinline__ float4* attn_partial(const A& a, int g) {
    return reinterpret_cast<float4*>(a.sk_scratch) + (size_t)g * kSlotF4;
}
template <class A>
__device__ __forceinline__ float4* attn_carry(const A& a, int g) {
    return reinterpret_cast<float4*>(a.sk_scratch) + (size_t)(a.sk_grid + g) * kSlotF4;
}
template <class A>
__device__ __forceinline__ unsigned* attn_flag(const A& a, int g) {
    return reinterpret_cast<unsigned*>(reinterpret_cast<float4*>(a.sk_scratch) + (size_t)2 * a.sk_grid * kSlotF4) +
           g;
}

// per-lane byte offset of float4 0 in a slot (computed where it is used, so it is not held in a
// register across a kernel's key loop)
__device__ __forceinline__ uint32_t attn_slot_lane(int wave, int lane) {
    return (uint32_t)((wave * kPartF4 * 64 + lane) * 16);
}

// merges the state in a slot (a piece's partial or the carry) into (o, m_run, l_run)
__device__ __forceinline__ void attn_merge_slot(const float4* slot, f32x16_v (&o)[4], float& m_run, float& l_run,
                                                int wave, int lane) {
    const __amdgpu_buffer_rsrc_t src = sk_slot(slot);
    const uint32_t slot_off = attn_slot_lane(wave, lane);
    const float4 ml = sk_load(src, slot_off + 16 * 64 * 16, 0);
    // all 16 loads in flight at once: after the key loop only O and a few addresses are live
    float4 v[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) v[c] = sk_load(src, slot_off + c * 64 * 16, 0);
    const float m_new = fmaxf(m_run, ml.x);
    const float ca = __builtin_amdgcn_exp2f(m_run - m_new), cb = __builtin_amdgcn_exp2f(ml.x - m_new);
    m_run = m_new;
    l_run = fmaf(l_run, ca, ml.y * cb);
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 w = v[4 * eb + i];
            o[eb][4 * i] = fmaf(o[eb][4 * i], ca, w.x * cb);
            o[eb][4 * i + 1] = fmaf(o[eb][4 * i + 1], ca, w.y * cb);
            o[eb][4 * i + 2] = fmaf(o[eb][4 * i + 2], ca, w.z * cb);
            o[eb][4 * i + 3] = fmaf(o[eb][4 * i + 3], ca, w.w * cb);
        }
}

// stores the state (unnormalised O, running max, running sum) into a slot
__device__ __forceinline__ void attn_store_slot(float4* slot, const f32x16_v (&o)[4], float m_run, float l_run,
                                                int wave, int lane) {
    const __amdgpu_buffer_rsrc_t dst = sk_slot(slot);
    const uint32_t slot_off = attn_slot_lane(wave, lane);
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sk_store(dst, slot_off + (4 * eb + i) * 64 * 16, 0, o[eb][4 * i], o[eb][4 * i + 1], o[eb][4 * i + 2],
                     o[eb][4 * i + 3]);
    sk_store(dst, slot_off + 16 * 64 * 16, 0, m_run, l_run, 0.0f, 0.0f);
}

constexpr int kAttnStore = -2;          // attn_split_finish: the unit's O is complete, store it

// After a unit's key tiles [kb, ke): the owner of a split unit (or its continuation) merges the
// partial states of the workgroups holding the rest of the unit, up to split step t_end, which
// published them first thing in their shares; a piece whose partial does not arrive in time is
// claimed, the owner's state parked in its carry slot, and the piece's key tiles returned in
// [ckb, cke) with the next piece's index (>= 0) for the driver to run as a continuation.  A
// partial piece publishes its state and returns -1.  Otherwise kAttnStore.  g is the workgroup, gb
// the first workgroup of its segment, Gs the segment's workgroups, S its split key tiles.
template <class A>
__device__ __forceinline__ int attn_split_finish(const A& a, f32x16_v (&o)[4], float& m_run, float& l_run, int kind,
                                                 int g, int gb, int Gs, long S, long t_end, int jn0, int& ckb,
                                                 int& cke, int wave, int lane) {
    if (kind == UNIT_OWNER || kind == UNIT_OWNER_CONT) {
        int miss = -1;
        // jn = -1: the state parked in the carry slot (a continuation), then pieces from jn0
        for (int jn = kind == UNIT_OWNER_CONT ? -1 : jn0; jn < Gs && (jn < 0 || sk_begin(S, jn, Gs) < t_end);
             jn = jn < 0 ? jn0 : jn + 1) {
            const float4* src = attn_carry(a, g);
            if (jn >= 0) {
                if (sk_begin(S, jn + 1, Gs) == sk_begin(S, jn, Gs)) continue;     // empty share
                if (!sk_take(attn_flag(a, gb + jn), a.epoch, a.sk_spins)) {
                    miss = jn;
                    break;
                }
                src = attn_partial(a, gb + jn);
            }
            attn_merge_slot(src, o, m_run, l_run, wave, lane);
        }
        if (miss >= 0) {
            attn_store_slot(attn_carry(a, g), o, m_run, l_run, wave, lane);
            __builtin_amdgcn_s_waitcnt(0);
            const long t_first = t_end - a.k_tiles;        // split step of this unit's key tile 0
            ckb = (int)(sk_begin(S, miss, Gs) - t_first);
            cke = (int)(min(sk_begin(S, miss + 1, Gs), t_end) - t_first);
            return miss + 1;
        }
    }
    if (kind == UNIT_PARTIAL) {
        attn_store_slot(attn_partial(a, g), o, m_run, l_run, wave, lane);
        sk_raise(attn_flag(a, g), a.epoch, a.sk_spins);
        return -1;
    }
    return kAttnStore;
}

// Persistent split driver (sk_grid > 0) or one unit per workgroup.  Workgroup g (XCD-remapped, so
// the Gs workgroups of a segment share an XCD and its L2) runs its segment's units gl, gl + Gs, ...
// below dp (gl = its index in the segment), then its even share of the segment's remaining key
// tiles in order: the end of a unit some earlier workgroup started (published as a partial), whole
// units, and the start of a unit later workgroups finish (it owns that one and merges their
// partials).  A unit's owner computes its piece last, after the workgroups holding the other pieces
// computed theirs first.  unit(L, kb, ke, kind, g, gb, Gs, S, t_end, jn0, ckb, cke) runs one item
// and returns an owner's continuation (>= 0) or -1.
template <class A, class Unit>
__device__ __forceinline__ void attn_split_driver(const A& a, Unit&& unit) {
    const int g = xcd_remap(blockIdx.x, gridDim.x);
    const int G = a.sk_grid, I = a.k_tiles;
    // the segment (XCD) of workgroup g: workgroups [gb, gb + Gs), units [u0, u0 + Us), of which the
    // first dp run whole (full rounds but one) and the rest, S key tiles, are split evenly
    const int Gs = G ? G / a.sk_segs : 0;
    const int x = G ? g / Gs : 0, gb = x * Gs, gl = g - gb;
    const int u0 = G ? (int)((long)a.units * x / a.sk_segs) : 0;
    const int Us = G ? (int)((long)a.units * (x + 1) / a.sk_segs) - u0 : 0;
    const int dp = G && Us >= Gs ? (Us / Gs - 1) * Gs : 0;
    const long S = G ? (long)(Us - dp) * I : 0;
    const long e = G ? sk_begin(S, gl + 1, Gs) : 0;
    long it = G ? sk_begin(S, gl, Gs) : 0;
    int cont = -1, ckb = 0, cke = 0, cL = 0;     // an owner's continuation (the unit's return)
    long ct_end = 0;
    // one work item per pass, so the unit code is generated once
    for (int w = 0;; ++w) {
        int L, kb = 0, ke = I, kind = UNIT_FULL, jn0 = gl + 1;
        long t_end = 0;
        if (cont >= 0) {
            L = cL; kb = ckb; ke = cke; kind = UNIT_OWNER_CONT; t_end = ct_end; jn0 = cont;
        } else if (G == 0) {
            if (w > 0) break;
            L = g;
        } else if ((long)gl + (long)w * Gs < dp) {
            L = u0 + gl + w * Gs;
        } else {
            if (it >= e) break;
            const int t = (int)(it / I);
            kb = (int)(it - (long)t * I);
            ke = (int)min((long)I, e - (long)t * I);
            kind = kb > 0 ? UNIT_PARTIAL : (ke == I ? UNIT_FULL : UNIT_OWNER);
            L = u0 + dp + t;
            t_end = (long)(t + 1) * I;
            it = (long)t * I + ke;
        }
        if (w > 0) __syncthreads();                 // the K / V rings are reused by the next unit
        cont = unit(L, kb, ke, kind, g, gb, Gs, S, t_end, jn0, ckb, cke);
        cL = L;
        ct_end = t_end;
    }
}

// Host side: the split decision for `units` units of k_tiles key tiles on G CUs, with a scratch
// buffer (a.sk_scratch non-null): split when the last round of units leaves the CUs idle for at
// least four key tiles on average and every workgroup's share is at least eight key tiles (each
// piece handed over costs a pipeline fill and a partial's round trip).  At 512 text + 4096 image
// tokens the 432 units of 72 key tiles run on 256 CUs as 121.5 key tiles each instead of 2 x 72.
template <class A>
inline void attn_plan_split(A& a, int G) {
    a.sk_grid = 0;
    a.sk_segs = 1;
    if (a.sk_scratch && G > 0 && a.units % G != 0) {
        const long rounds = (a.units + G - 1) / G;
        const long work = (long)a.units * a.k_tiles;
        const long idle = rounds * G * a.k_tiles - work;
        if (idle >= 4L * G && work >= 8L * G) {
            a.sk_grid = G;
            // one segment per XCD (8 on gfx950; the remapped workgroup ids of an XCD are
            // contiguous), or one for the whole grid if the CUs do not divide evenly
            a.sk_segs = G % 8 == 0 ? 8 : 1;
            a.epoch = next_launch_tag();
            a.sk_spins = sk_spin_limit();
        }
    }
}

}  // namespace dit
