// Grouped GEMMs of the DiT block on gfx950: C = epilogue(A . B^T), A = activations [M, K],
// B = weights [N, K] ([out, in]).  These are the thread's "heavy matrix multiplications"
// (QKV projections, FFN; the "CUDA codepath !" thread, antirez/iris.c issue #15), with the
// per-block elementwise work fused into the epilogue:
//   EPI_STORE     C = acc                                   (QKV)
//                 with QK RMSNorm + RoPE applied to the q and k columns first when the batch
//                 carries an angle table (the block's QKV product, whole heads per tile)
//   EPI_GATED_RES C = R + gate[col] * acc                   (out-proj, FFN-down: gated residual)
//   EPI_SWIGLU    C = SiLU(acc_gate) * acc_up               (FFN-in)
// One launch covers several problems (text and image streams, or the two halves of the
// single-stream block's first linear).
//
// MFMA path (bf16 weights): a 256 x 256 x 64 block tile, 8 waves (2 along M x 4 along N), each a
// 128 x 64 sub-tile of 4 x 2 v_mfma_f32_32x32x16 tiles with fp32 accumulators (two waves per SIMD:
// one issues MFMAs while the other waits on LDS; a 4-wave layout of 128 x 128 sub-tiles, one wave
// per SIMD, measured 8-10% slower).  Activations are bf16 or fp16; with fp16
// activations the bf16 weight tile is converted to fp16 while it is staged (the MFMA needs one
// operand type; the conversion is exact).  Operands go global -> LDS with global_load_lds_dwordx4
// (no VGPR staging) where no conversion is needed, double-buffered.
// LDS rows are 128 B with the 16-byte chunk index XOR-swizzled (swz) so the fragment
// reads are bank-conflict free.  The MFMA computes D[n][m], so each lane ends with four
// consecutive output columns of one row and the epilogue reads / writes 8-16 B per lane.
// Workgroups are remapped so each XCD gets a contiguous range of tiles, rastered in groups of
// 4 M-tiles (8 and 16 were slower at 512 + 16384 tokens, the same at 512 + 4096).
//
// fp32 path: a plain LDS-tiled FMA kernel (no reduced-precision matrix math).
#include <atomic>
#include <chrono>
#include <type_traits>

#include "dev_common.h"
#include "launch.h"

namespace dit {

enum GemmMode { MODE_STORE = 0, MODE_RES = 1, MODE_SWIGLU = 2, MODE_MIXED = 3 };

constexpr int BM = 256, BN = 256, BK = 64;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void tile_of(const GemmBatch& b, int L, int& pi, int& tm, int& tn) {
    // Groups of G M-tiles; inside a group, consecutive tiles walk the G M-tiles of one N column,
    // then the next column.  The tiles one XCD runs at the same time then form a compact
    // block of about G x (32 / G) tiles, whose A and B tiles L2 shares.
    pi = (b.n > 1 && L >= b.p[1].tile_begin) ? 1 : 0;
    const GemmProblem& P = b.p[pi];
    const int G0 = b.group_m > 0 ? b.group_m : 4;
    const int t = L - P.tile_begin;
    const int per_group = G0 * P.tiles_n;
    const int g = t / per_group;
    const int first_m = g * G0;
    const int gsize = min(P.tiles_m - first_m, G0);
    const int r = t - g * per_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

// SiLU of an fp32 accumulator whose product is rounded to 16 bits or fewer: the reciprocal instruction
// (within 1 ulp) in place of a correctly rounded division, whose fix-up sequence is ~10 instructions
__device__ __forceinline__ float silu_acc(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// LDS row swizzle of the staged tiles (rows of 128 B = 8 chunks of 16 B).  gfx950 serves a
// ds_read_b128 16 lanes per cycle from 64 banks of 4 B (two 128-B rows per bank sweep), and a
// fragment read has 16 consecutive rows at one chunk index: XOR-ing the chunk with (row >> 1) & 7
// gives the 8 even rows 8 distinct chunks in one half of the banks and the 8 odd rows 8 in the
// other half.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

template <int AT> struct Frag;
template <> struct Frag<BF16> { typedef bf16x8_v T; };
template <> struct Frag<F16> { typedef f16x8_v T; };

template <int AT>
__device__ __forceinline__ f32x16_v mfma32(const typename Frag<AT>::T& a, const typename Frag<AT>::T& b,
                                           const f32x16_v& c) {
    if constexpr (AT == F16) return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Epilogue store of 4 consecutive columns of one row, output type chosen at run time.
__device__ __forceinline__ void store4_dt(void* base, size_t off, int dt, const float* o) {
    char* p = reinterpret_cast<char*>(base);
    if (dt == F32) store4<F32>(p + off * 4, o);
    else if (dt == F16) store4<F16>(p + off * 2, o);
    else store4<BF16>(p + off * 2, o);
}

// Operand types: AT = BF16 (bf16 activations and weights), F16 (fp16 activations, bf16 weights) or
// F16W (fp16 activations and fp16 copies of the weights).
constexpr int F16W = 4;
template <int AT> constexpr int mfma_type() { return AT == BF16 ? BF16 : F16; }

// A (activations, AT) is staged global -> LDS with global_load_lds_dwordx4.  B (weights)
// goes the same way when AT is BF16 or F16W; when AT == F16 it is loaded into VGPRs, converted to fp16
// (exact: bf16 values are fp16 values in fp16's normal range) and written to the same LDS
// layout, so both operands of the fp16 MFMA come from one swizzled layout.
constexpr int WN = 4;                                  // waves along N (2 along M)
constexpr int kGemmLds = 2 * (BM + BN) * BK * 2;      // two A+B stages: 128 KB, one workgroup per CU
constexpr int kPartialF4 = BM * BN / 4;               // float4s of one fp32 partial tile (256 KB)

// How a workgroup finishes a tile it computed k-steps [kb, ke) of:
enum TileKind {
    TILE_FULL = 0,      // all k-steps: epilogue
    TILE_OWNER = 1,     // k-steps from 0: add the partials of the workgroups holding the rest, epilogue
    TILE_PARTIAL = 2,   // a later run of k-steps: publish the fp32 partial for the owner
    TILE_OWNER_CONT = 3 // an owner's continuation: k-steps of a piece whose partial did not arrive,
                        // plus the owner's running sum from its carry slot, then as TILE_OWNER
};

// Stream-K scratch: [sk_grid] partial tiles, [sk_grid] carry tiles (an owner's running sum while it
// computes a missing piece), then [sk_grid] 32-bit flags.
__device__ __forceinline__ float4* sk_partial(const GemmBatch& b, int g) {
    return reinterpret_cast<float4*>(b.sk_scratch) + (size_t)g * kPartialF4;
}
__device__ __forceinline__ float4* sk_carry(const GemmBatch& b, int g) {
    return reinterpret_cast<float4*>(b.sk_scratch) + (size_t)(b.sk_grid + g) * kPartialF4;
}
__device__ __forceinline__ unsigned* sk_flag(const GemmBatch& b, int g) {
    return reinterpret_cast<unsigned*>(reinterpret_cast<float4*>(b.sk_scratch) +
                                                 (size_t)2 * b.sk_grid * kPartialF4) + g;
}

// QK RMSNorm + 4-axis RoPE on the fp32 accumulators of a q or k tile of the QKV product, before they
// are stored (the separate pass's arithmetic on the unrounded products: per-head mean square, rsq,
// times the norm weight, then each interleaved pair rotated by the (cos, sin) of its angle from
// the token's row of the angle table).  Wave (wm, wn) holds rows wm*128 + mb*32 + lane%32 and
// columns wn*64 + nb*32 + 8 i + 4 (lane/32) + j of the tile; a head's 128 columns are waves wn and
// wn ^ 1, whose partial sums of squares meet in LDS, where the tile's 128 norm weights wait too.
__device__ __forceinline__ void qk_rope_tile(const GemmBatch& b, int pi, char* smem, f32x16_v (&acc)[2][4], int m0,
                                             int n0, int M, int wm, int wn, int lane) {
    const int khalf = lane >> 5, mlane = lane & 31;
    const int which = n0 >= b.rope_d ? 1 : 0;        // q or k
    const int hd0 = (wn & 1) * 64;                   // this wave's first dimension of the head
    float ss[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        float s = 0.0f;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int q = 0; q < 16; ++q) s = fmaf(acc[nb][mb][q], acc[nb][mb][q], s);
        ss[mb] = s + __shfl_xor(s, 32, kWave);
    }
    __syncthreads();                                 // every wave is done with the last stage
    float* red = reinterpret_cast<float*>(smem);     // [2 wm][4 wn][128 rows], then the 128 weights
    if (khalf == 0) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) red[(wm * 4 + wn) * 128 + mb * 32 + mlane] = ss[mb];
    }
    const int tid = (wm * 4 + wn) * 64 + lane;
    if (tid < 128) red[1024 + tid] = bf_lo(reinterpret_cast<const uint16_t*>(b.rope_w[pi])[which * 128 + tid]);
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) ss[mb] += red[(wm * 4 + (wn ^ 1)) * 128 + mb * 32 + mlane];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int tok = b.rope_row0[pi] + min(m0 + wm * 128 + mb * 32 + mlane, M - 1);
        const float* crow = b.rope_cs + (size_t)tok * 128;
        // the row's 16 pairs: (cos, sin) of pairs p0, p0 + 1 in one 16-byte load per 4 values
        f32x4_v cs[2][4];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) cs[nb][i] = ldf4(crow + (hd0 + nb * 32 + 8 * i + 4 * khalf));
        const float rstd = __builtin_amdgcn_rsqf(ss[mb] * (1.0f / 128.0f) + b.rope_eps);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float* wp = red + 1024 + hd0 + nb * 32 + 8 * i + 4 * khalf;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const float c = cs[nb][i][2 * t], sn = cs[nb][i][2 * t + 1];
                    const float u0 = acc[nb][mb][4 * i + 2 * t] * rstd * wp[2 * t];
                    const float u1 = acc[nb][mb][4 * i + 2 * t + 1] * rstd * wp[2 * t + 1];
                    acc[nb][mb][4 * i + 2 * t] = u0 * c - u1 * sn;
                    acc[nb][mb][4 * i + 2 * t + 1] = u0 * sn + u1 * c;
                }
            }
        __builtin_amdgcn_sched_barrier(0);          // one row's table values live at a time
    }
}

// Returns -1, or (an owner whose piece jn did not arrive; its running sum is in its carry slot) the
// index jn of the next workgroup whose piece is still to be merged, with the missing piece's k-steps
// in [ckb, cke): the driver then runs that continuation as the workgroup's next item.
template <int MODE, int AT>
__device__ __forceinline__ int gemm_tile(const GemmBatch& b, char* smem, int L, int kb, int ke, int kind, int g,
                                         long S, long t_end, int jn0, int& ckb, int& cke) {
    constexpr int NW = 2 * WN;                     // waves per workgroup
    constexpr int NB = 4 / (WN / 2);               // 32-wide n-blocks per wave (4 or 2)
    constexpr int LPW = 32 / NW;                   // 1 KB load instructions per wave per operand
    constexpr int kStage = (BM + BN) * BK * 2;     // bytes of one A+B stage
    constexpr int kBOff = BM * BK * 2;             // B tile offset within a stage
    constexpr int MT = mfma_type<AT>();           // MFMA operand type
    typedef typename Frag<MT>::T FragT;

    // An owner's continuation takes its k-range from a flag word every lane read: make the range
    // wave-uniform so the k-loop runs on scalar control.
    kb = __builtin_amdgcn_readfirstlane(kb);
    ke = __builtin_amdgcn_readfirstlane(ke);
    int pi, tm, tn;
    tile_of(b, L, pi, tm, tn);
    const GemmProblem& P = b.p[pi];
    const int epi = MODE == MODE_MIXED ? P.epi : (MODE == MODE_SWIGLU ? EPI_SWIGLU
                                                  : (MODE == MODE_RES ? EPI_GATED_RES : EPI_STORE));
    const bool swiglu = epi == EPI_SWIGLU;
    const int m0 = tm * BM;
    const int n0 = swiglu ? tn * (BN / 2) : tn * BN;   // first output column
    const int M = P.M;

    // The thread index goes through an opaque zero: the per-lane address arithmetic below is then
    // recomputed for every tile of a persistent workgroup instead of being hoisted out of the
    // tile loop and held in registers across it.
    int zero;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
    const int tid = threadIdx.x + zero;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // ---- global -> LDS load plan: wave w, instruction i covers tile rows (w*LPW+i)*8 .. +7;
    //      lane l writes LDS bytes l*16 .. l*16+15 of that 1 KB block = row l/8, chunk l%8,
    //      which holds global chunk (l%8) ^ swz(row) of the row.
    const bf16_t* gA[LPW];
    const bf16_t* gB[LPW];
    // The same plan as a uniform tile base plus a 32-bit per-lane byte offset (the loads then take
    // the scalar-base addressing form, with no per-load 64-bit address arithmetic).  A wave's B
    // rows are all gate rows or all up rows of a SwiGLU tile.  Offsets stay below 2^32 because row
    // strides are below 2^22 elements (checked on the host).
    const char* tA = reinterpret_cast<const char*>(P.A) + (size_t)m0 * P.lda * 2;
    const bool wup = swiglu && wave * LPW * 8 >= BN / 2;
    const char* tB = reinterpret_cast<const char*>(P.B) + ((size_t)n0 + (wup ? P.up_off : 0)) * P.ldb * 2;
    uint32_t oA[LPW], oB[LPW];
    {
        const int lr = lane >> 3, lc = lane & 7;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int row = (wave * LPW + i) * 8 + lr;
            const int chunk = lc ^ swz(row);
            int am = m0 + row;
            am = am < M ? am : M - 1;
            gA[i] = reinterpret_cast<const bf16_t*>(P.A) + (size_t)am * P.lda + chunk * 8;
            long bn;
            if (swiglu) {
                const bool up = row >= BN / 2;
                bn = (long)n0 + (up ? row - BN / 2 : row);
                if (bn > P.N - 1) bn = P.N - 1;
                if (up) bn += P.up_off;
            } else {
                bn = n0 + row;
                if (bn > P.N - 1) bn = P.N - 1;
            }
            gB[i] = reinterpret_cast<const bf16_t*>(P.B) + (size_t)bn * P.ldb + chunk * 8;
            oA[i] = (uint32_t)(((long)(am - m0) * P.lda + chunk * 8) * 2);
            oB[i] = (uint32_t)(((bn - (wup ? P.up_off : 0) - n0) * P.ldb + chunk * 8) * 2);
        }
    }
    u32x4_v breg[LPW];
    auto issue_loads = [&](int buf, int k0) {
        if constexpr (AT == F16) {
#pragma unroll
            for (int i = 0; i < LPW; ++i) breg[i] = ld16(gB[i] + k0);  // issued first: waited on first
        }
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            __builtin_amdgcn_global_load_lds(gA[i] + k0, (lds_void*)(smem + buf * kStage + (wave * LPW + i) * 1024),
                                             16, 0, 0);
            if constexpr (AT != F16)
                __builtin_amdgcn_global_load_lds(gB[i] + k0,
                                                 (lds_void*)(smem + buf * kStage + kBOff + (wave * LPW + i) * 1024),
                                                 16, 0, 0);
        }
    };
    auto issue_load_pair = [&](int buf, int k0, int i) {
        __builtin_amdgcn_global_load_lds(tA + (long)k0 * 2 + oA[i],
                                         (lds_void*)(smem + buf * kStage + (wave * LPW + i) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(tB + (long)k0 * 2 + oB[i],
                                         (lds_void*)(smem + buf * kStage + kBOff + (wave * LPW + i) * 1024), 16, 0, 0);
    };
    auto store_b = [&](int buf) {
        if constexpr (AT == F16) {
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                u32x4_v w;
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = bf16x2_to_f16x2(breg[i][j]);
                *reinterpret_cast<u32x4_v*>(smem + buf * kStage + kBOff + (wave * LPW + i) * 1024 + lane * 16) = w;
            }
        }
    };

    // ---- fragment read offsets.  A fragment (m-block j): row wm*128 + j*32 + (lane & 31);
    //      B fragment (n-block j): a 32-row block of this wave's B rows (gate and up halves for
    //      SwiGLU tiles: the first NB/2 blocks gate, the last NB/2 the matching up rows).
    int a_row[4], b_row[NB];
#pragma unroll
    for (int j = 0; j < 4; ++j) a_row[j] = wm * 128 + j * 32 + (lane & 31);
    constexpr int WNR = BN / WN;                   // B rows per wave
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        if (swiglu) b_row[j] = (j < NB / 2 ? wn * (WNR / 2) + j * 32 : BN / 2 + wn * (WNR / 2) + (j - NB / 2) * 32)
                               + (lane & 31);
        else b_row[j] = wn * WNR + j * 32 + (lane & 31);
    }
    const int khalf = lane >> 5;

    f32x16_v acc[NB][4];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    // Fragments for k16 sub-step s of a staged tile (LDS byte offset `base` of its A tile).
    auto read_frags = [&](FragT* fa, FragT* fb, int base, int s) {
        const int c = 2 * s + khalf;
        const char* la = smem + base;
        const char* lb = la + kBOff;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            fa[j] = *reinterpret_cast<const FragT*>(la + a_row[j] * 128 + ((c ^ swz(a_row[j])) << 4));
#pragma unroll
        for (int j = 0; j < NB; ++j)
            fb[j] = *reinterpret_cast<const FragT*>(lb + b_row[j] * 128 + ((c ^ swz(b_row[j])) << 4));
    };

    FragT fa[2][4], fb[2][NB];
    // One k-step on the staged tile `buf`.  MORE: the next tile exists -- issue its loads
    // and (fp16) write its converted weight tile; the body is then one basic block, so the
    // scheduling groups below apply to all of it.
    auto kstep = [&]<bool MORE>(int k0, int it) {
        constexpr int kMFMA = 0x008, kVALU = 0x002, kDSR = 0x100, kDSW = 0x200, kVMEM = 0x020;
        constexpr int kReads = 4 + NB, kMfmas = 4 * NB;
        const int buf = it & 1;
        // Each k16 sub-step is its own scheduling region: its MFMAs, with the next sub-step's
        // fragment reads placed between the first of them (they then have the remaining MFMAs
        // of time to land), the next tile's global loads spread over sub-step 0, and (fp16
        // path) the next weight tile's conversion + LDS writes over sub-step 3.
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int cur = s & 1;
            if (s + 1 < BK / 16) read_frags(fa[cur ^ 1], fb[cur ^ 1], buf * kStage, s + 1);
            if constexpr (MORE) {
                if (s == 0) issue_loads(buf ^ 1, (k0 + it + 1) * BK);
                if constexpr (AT == F16) {
                    if (s == BK / 16 - 1) store_b(buf ^ 1);
                }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = mfma32<MT>(fb[cur][nb], fa[cur][mb], acc[nb][mb]);
            if (s + 1 < BK / 16) {
#pragma unroll
                for (int i = 0; i < kReads; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kMFMA, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kDSR, 1, 0);
                    if (MORE && s == 0 && i < LPW) __builtin_amdgcn_sched_group_barrier(kVMEM, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(kMFMA, kMfmas - kReads, 0);
            } else if (AT == F16 && MORE) {
#pragma unroll
                for (int i = 0; i < LPW; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kMFMA, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kVALU, 6, 0);
                    __builtin_amdgcn_sched_group_barrier(kMFMA, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kVALU, 6, 0);
                    __builtin_amdgcn_sched_group_barrier(kDSW, 1, 0);
                }
                if (kMfmas > 2 * LPW) __builtin_amdgcn_sched_group_barrier(kMFMA, kMfmas - 2 * LPW, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (MORE) read_frags(fa[0], fb[0], (buf ^ 1) * kStage, 0);
    };
    // Rotated pipeline for operands that both travel global -> LDS directly (AT != F16): the
    // barrier sits after sub-step 2, so the first fragment reads of the next staged tile and the
    // global loads of the tile after it are issued right behind the barrier and sub-step 3's
    // MFMAs (whose fragments are already in registers) cover their latency.  The loads of tile
    // it + 2 go into the stage tile it was read from: every wave finished reading it before the
    // barrier.  MORE: 2 = tiles it + 1 and it + 2 exist, 1 = only it + 1, 0 = last tile.
    auto kstep_rot = [&]<int MORE>(int k0, int it) {
        constexpr int kMFMA = 0x008, kDSR = 0x100;
        constexpr int kReads = 4 + NB, kMfmas = 4 * NB;
        const int buf = it & 1;
#pragma unroll
        for (int s = 0; s < BK / 16 - 1; ++s) {
            const int cur = s & 1;
            read_frags(fa[cur ^ 1], fb[cur ^ 1], buf * kStage, s + 1);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = mfma32<MT>(fb[cur][nb], fa[cur][mb], acc[nb][mb]);
#pragma unroll
            for (int i = 0; i < kReads; ++i) {
                __builtin_amdgcn_sched_group_barrier(kMFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kDSR, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kMFMA, kMfmas - kReads, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (MORE > 0) {
            // tile it + 1 has landed (own loads: waitcnt; every wave's: barrier) and no wave
            // reads stage `buf` any more
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            read_frags(fa[0], fb[0], (buf ^ 1) * kStage, 0);
        }
        // sub-step 3; the next tile's global loads go one A / B pair after each of the first LPW
        // MFMAs (fenced, so the issue of the loads and their address arithmetic overlaps MFMAs
        // instead of leaving the matrix pipe idle behind a burst of them)
#pragma unroll
        for (int q = 0; q < kMfmas; ++q) {
            const int nb = q / 4, mb = q % 4;
            acc[nb][mb] = mfma32<MT>(fb[1][nb], fa[1][mb], acc[nb][mb]);
            if constexpr (MORE > 1) {
                if (q < LPW) {
                    __builtin_amdgcn_sched_barrier(0);
                    issue_load_pair(buf, (k0 + it + 2) * BK, q);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // k-steps [k0, k1) of the tile, accumulated into acc
    // k-steps [k0, k1) of the tile, accumulated into acc
    auto kloop = [&](int k0, int k1) {
        const int nk = k1 - k0;
        issue_loads(0, k0 * BK);
        store_b(0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (AT != F16) {
            read_frags(fa[0], fb[0], 0, 0);
            if (nk > 1) issue_loads(1, (k0 + 1) * BK);
            int it = 0;
            for (; it < nk - 2; ++it) kstep_rot.template operator()<2>(k0, it);
            if (nk > 1) kstep_rot.template operator()<1>(k0, it++);
            kstep_rot.template operator()<0>(k0, it);
        } else {
            read_frags(fa[0], fb[0], 0, 0);
            for (int it = 0; it < nk - 1; ++it) kstep.template operator()<true>(k0, it);
            kstep.template operator()<false>(k0, nk - 1);
        }
    };

    // Partial tiles: lane l of wave w keeps float4 c of its accumulators at index
    // (w * NB*16 + c) * 64 + l of its workgroup's slot.
    constexpr int kF4 = NB * 16;                   // float4s of accumulators per lane
    kloop(kb, ke);

    const uint32_t slot_off = (uint32_t)((wave * kF4 * 64 + lane) * 16);     // float4 c at + c * 1024
    // adds the fp32 tile in a stream-K slot (partial or carry) to acc
    auto add_slot = [&](const float4* slot) {
        const __amdgpu_buffer_rsrc_t src = sk_slot(slot);
        // batches of 8 loads, all issued before the batch's adds (written load-then-add, the
        // scheduler placed each load just before its add and waited for it there: one round trip
        // past the L2 per float4); the k-loop's operand registers are free by now
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int hm = 0; hm < 2; ++hm) {
                float4 v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = sk_load(src, slot_off, (uint32_t)((nb * 4 + 2 * hm) * 4 + k) * 1024u);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int mb = 2 * hm + (k >> 2), q = k & 3;
                    acc[nb][mb][4 * q] += v[k].x;
                    acc[nb][mb][4 * q + 1] += v[k].y;
                    acc[nb][mb][4 * q + 2] += v[k].z;
                    acc[nb][mb][4 * q + 3] += v[k].w;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
    };
    // stores acc into a stream-K slot
    auto store_slot = [&](float4* slot) {
        const __amdgpu_buffer_rsrc_t dst = sk_slot(slot);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = (nb * 4 + mb) * 4 + q;
                    sk_store(dst, slot_off, (uint32_t)c * 1024u, acc[nb][mb][4 * q], acc[nb][mb][4 * q + 1],
                             acc[nb][mb][4 * q + 2], acc[nb][mb][4 * q + 3]);
                }
    };

    // The owner of a split tile has run its own k-steps (or, continuing, a missing piece's); it adds
    // the partials of the workgroups holding the rest of the tile, up to k-step t_end (stream-K
    // relative), which published them first thing in their shares.  When a piece's partial does
    // not arrive in time the owner claims the piece, parks its running sum in its carry slot and
    // returns; the driver runs the piece's k-steps as its next item, which resumes here.
    if (kind == TILE_OWNER || kind == TILE_OWNER_CONT) {
        const int G = b.sk_grid;
        int miss = -1;
        // jn = -1: the running sum parked in the carry slot (a continuation), then pieces from jn0
        for (int jn = kind == TILE_OWNER_CONT ? -1 : jn0; jn < G && (jn < 0 || sk_begin(S, jn, G) < t_end);
             jn = jn < 0 ? jn0 : jn + 1) {
            const float4* src = sk_carry(b, g);
            if (jn >= 0) {
                if (sk_begin(S, jn + 1, G) == sk_begin(S, jn, G)) continue;     // empty share
                if (!sk_take(sk_flag(b, jn), b.epoch, b.sk_spins)) {
                    miss = jn;
                    break;
                }
                src = sk_partial(b, jn);
            }
            add_slot(src);
        }
        if (miss >= 0) {
            store_slot(sk_carry(b, g));
            __builtin_amdgcn_s_waitcnt(0);
            const long t_first = t_end - b.k_steps;        // stream-K step of this tile's k-step 0
            ckb = (int)(sk_begin(S, miss, G) - t_first);
            cke = (int)(min(sk_begin(S, miss + 1, G), t_end) - t_first);
            return miss + 1;
        }
    }

    if (kind == TILE_PARTIAL) {
        store_slot(sk_partial(b, g));
        sk_raise(sk_flag(b, g), b.epoch, b.sk_spins);
        return -1;
    }

    // ---- epilogue.  acc[nb][mb][q]: row m = m0 + wm*128 + mb*32 + (lane & 31),
    //      B-row offset within the n-block: 8*(q>>2) + 4*khalf + (q&3).
    const int mlane = lane & 31;
    bool bad = false;              // an fp16 output out of fp16's range
    if (swiglu) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int m = m0 + wm * 128 + mb * 32 + mlane;
            if (m >= M) continue;
#pragma unroll
            for (int nb = 0; nb < NB / 2; ++nb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int col = n0 + wn * (WNR / 2) + nb * 32 + 8 * i + 4 * khalf;
                    if (col >= P.N) continue;
                    float f[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float g = acc[nb][mb][4 * i + j];
                        const float u = acc[nb + NB / 2][mb][4 * i + j];
                        f[j] = silu_acc(g) * u;
                    }
                    if (P.c_dtype == F16)
                        bad |= f16_out_of_range4(f);
                    store4_dt(P.C, (size_t)m * P.ldc + col, P.c_dtype, f);
                }
            }
        }
    } else {
        if constexpr (MODE == MODE_STORE) {
            // fused QK RMSNorm + RoPE on a q or k tile (two whole heads: rope_d is a multiple of 256)
            if (b.rope_cs && n0 < 2 * b.rope_d) qk_rope_tile(b, pi, smem, acc, m0, n0, M, wm, wn, lane);
        }
        // Store (and gated residual): the types are dispatched once, outside the row loop, and a
        // row's residual loads are all issued before its first store -- with a type switch or a
        // bounds test around each load, every load was followed by a wait at the branch's join,
        // one round trip per 4 outputs.  Loads clamp their row and column into the problem (N is
        // a multiple of 8); the stores test them.
        const bool res = epi == EPI_GATED_RES;
        auto rows = [&]<int RT, int CT>() {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int m = m0 + wm * 128 + mb * 32 + mlane;
                const char* rrow = reinterpret_cast<const char*>(P.R) + (size_t)min(m, M - 1) * P.ldr * ESize<RT>::v;
                char* crow = reinterpret_cast<char*>(P.C) + (size_t)m * P.ldc * ESize<CT>::v;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    float r[4][4];
                    f32x4_v gate[4];
                    if (res) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int col = min(n0 + wn * WNR + nb * 32 + 8 * i + 4 * khalf, P.N - 4);
                            gate[i] = ldf4(P.gate + col);
                            load4<RT>(rrow + (size_t)col * ESize<RT>::v, r[i]);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int col = n0 + wn * WNR + nb * 32 + 8 * i + 4 * khalf;
                        float o[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            o[j] = res ? fmaf(gate[i][j], acc[nb][mb][4 * i + j], r[i][j]) : acc[nb][mb][4 * i + j];
                        if (m < M && col < P.N) {
                            if constexpr (CT == F16) bad |= f16_out_of_range4(o);
                            store4<CT>(crow + (size_t)col * ESize<CT>::v, o);
                        }
                    }
                    // the next batch's loads stay below this one's stores (hoisted, they raised
                    // the register pressure past the file)
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        // gated residual outputs are F32 or BF16 (h, y), store outputs F32, F16 or BF16
        if (res) {
            if (P.r_dtype == BF16) {
                if (P.c_dtype == BF16) rows.template operator()<BF16, BF16>();
                else rows.template operator()<BF16, F32>();
            } else {
                if (P.c_dtype == BF16) rows.template operator()<F32, BF16>();
                else rows.template operator()<F32, F32>();
            }
        } else {
            if (P.c_dtype == F32) rows.template operator()<F32, F32>();
            else if (P.c_dtype == F16) rows.template operator()<F32, F16>();
            else rows.template operator()<F32, BF16>();
        }
    }
    raise_range_flag(b.range_flag, bad);
    return -1;
}

// Persistent stream-K driver (sk_grid > 0) or one tile per workgroup.  Workgroup g (XCD-remapped,
// so consecutive g share an XCD) runs tiles g, g + G, ... below dp_tiles, then its even share of
// the remaining tiles' k-steps in order: the end of a tile some earlier workgroup started
// (published as a partial), whole tiles, and the start of a tile later workgroups finish (it
// owns that one and adds their partials).  A tile's owner computes its piece last, after the
// workgroups holding the other pieces computed theirs first.
template <int MODE, int AT>
__device__ __forceinline__ void gemm_mfma_body(const GemmBatch& b) {
    __shared__ __attribute__((aligned(1024))) char smem[kGemmLds];
    const int g = xcd_remap(blockIdx.x, gridDim.x);
    const int G = b.sk_grid, I = b.k_steps;
    const long S = G ? (long)(b.total_tiles - b.dp_tiles) * I : 0;     // stream-K k-steps
    const long e = G ? sk_begin(S, g + 1, G) : 0;
    long it = G ? sk_begin(S, g, G) : 0;
    int cont = -1, ckb = 0, cke = 0, cL = 0;     // an owner's continuation (gemm_tile's return)
    long ct_end = 0;
    // one work item per pass, so the tile code is generated once
    for (int w = 0;; ++w) {
        int L, kb = 0, ke = I, kind = TILE_FULL, jn0 = g + 1;
        long t_end = 0;
        if (cont >= 0) {
            L = cL; kb = ckb; ke = cke; kind = TILE_OWNER_CONT; t_end = ct_end; jn0 = cont;
        } else if (G == 0) {
            if (w > 0) break;
            L = g;
        } else if ((long)g + (long)w * G < b.dp_tiles) {
            L = g + w * G;
        } else {
            if (it >= e) break;
            const int t = (int)(it / I);
            kb = (int)(it - (long)t * I);
            ke = (int)min((long)I, e - (long)t * I);
            kind = kb > 0 ? TILE_PARTIAL : (ke == I ? TILE_FULL : TILE_OWNER);
            L = b.dp_tiles + t;
            t_end = (long)(t + 1) * I;
            it = (long)t * I + ke;
        }
        if (w > 0) __syncthreads();                 // LDS stages are reused by the next tile
        cont = gemm_tile<MODE, AT>(b, smem, L, kb, ke, kind, g, S, t_end, jn0, ckb, cke);
        cL = L;
        ct_end = t_end;
    }
}

template <int MODE, int AT>
__global__ __launch_bounds__(512, 1) void gemm_mfma_w8(GemmBatch b) { gemm_mfma_body<MODE, AT>(b); }

// ------------------------------------------------------------------------------------------
// fp32 GEMM: 64 x 64 block tile, K step 16, 256 threads each owning a 4 x 4 output patch.
// SwiGLU problems load a second B tile (the up rows) and keep a second accumulator.
// ------------------------------------------------------------------------------------------
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <bool SWIGLU>
__device__ __forceinline__ void gemm_f32_tile(const GemmProblem& P, int tm, int tn) {
    __shared__ float sA[FBK][FBM + 4];
    __shared__ float sB[FBK][FBN + 4];
    __shared__ float sU[SWIGLU ? FBK : 1][FBN + 4];
    const int tid = threadIdx.x;
    const int m0 = tm * FBM, n0 = tn * FBN;
    const int lr = tid >> 2, lk = (tid & 3) * 4;          // loader: row, k offset
    const int ty = tid >> 4, tx = tid & 15;               // compute: 4 rows, 4 cols
    float acc[4][4] = {}, accu[4][4] = {};
    const int am = min(m0 + lr, P.M - 1);
    const int bn = min(n0 + lr, P.N - 1);
    const float* Ap = reinterpret_cast<const float*>(P.A) + (size_t)am * P.lda;
    const float* Bp = reinterpret_cast<const float*>(P.B) + (size_t)bn * P.ldb;
    const float* Up = reinterpret_cast<const float*>(P.B) + (size_t)(P.up_off + bn) * P.ldb;
    for (int k0 = 0; k0 < P.K; k0 += FBK) {
        const f32x4_v a = ldf4(Ap + k0 + lk), bb = ldf4(Bp + k0 + lk);
        f32x4_v uu = {0, 0, 0, 0};
        if (SWIGLU) uu = ldf4(Up + k0 + lk);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            sA[lk + t][lr] = a[t];
            sB[lk + t][lr] = bb[t];
            if (SWIGLU) sU[lk + t][lr] = uu[t];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < FBK; ++kk) {
            float av[4], bv[4], uv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = sA[kk][ty * 4 + i];
                bv[i] = sB[kk][tx * 4 + i];
                if (SWIGLU) uv[i] = sU[kk][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
                    if (SWIGLU) accu[i][j] = fmaf(av[i], uv[j], accu[i][j]);
                }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= P.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= P.N) continue;
            float o = acc[i][j];
            if (SWIGLU) o = (o / (1.0f + expf(-o))) * accu[i][j];
            if (P.epi == EPI_GATED_RES) {
                const float r = reinterpret_cast<const float*>(P.R)[(size_t)m * P.ldr + n];
                o = fmaf(P.gate[n], o, r);
            }
            reinterpret_cast<float*>(P.C)[(size_t)m * P.ldc + n] = o;
        }
    }
}

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmBatch b) {
    const int L = blockIdx.x;
    const int pi = (b.n > 1 && L >= b.p[1].tile_begin) ? 1 : 0;
    const GemmProblem& P = b.p[pi];
    const int t = L - P.tile_begin;
    const int tm = t / P.tiles_n, tn = t % P.tiles_n;
    if (P.epi == EPI_SWIGLU) gemm_f32_tile<true>(P, tm, tn);
    else gemm_f32_tile<false>(P, tm, tn);
}

template <int AT>
static void launch_mfma(GemmBatch& b, hipStream_t s, bool all_store, bool all_res, bool all_swiglu) {
    const dim3 grid(b.sk_grid ? b.sk_grid : b.total_tiles), block(512);
    if (all_store) hipLaunchKernelGGL((gemm_mfma_w8<MODE_STORE, AT>), grid, block, 0, s, b);
    else if (all_res) hipLaunchKernelGGL((gemm_mfma_w8<MODE_RES, AT>), grid, block, 0, s, b);
    else if (all_swiglu) hipLaunchKernelGGL((gemm_mfma_w8<MODE_SWIGLU, AT>), grid, block, 0, s, b);
    else hipLaunchKernelGGL((gemm_mfma_w8<MODE_MIXED, AT>), grid, block, 0, s, b);
}

// Compute units of the current device (the stream-K grid: one 128 KB-LDS workgroup per CU, all
// resident at once); 0 if unknown.
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) n = 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

size_t gemm_sk_scratch_bytes() {
    const int G = device_cu_count();
    return G > 0 ? (size_t)G * (2 * (size_t)kPartialF4 * 16 + 8) : 0;
}

// Launch tags for the stream-K flags: nonzero, unique per launch in this process and started from a
// time-derived value, so flags left in a reused workspace never match a new launch.  An owner
// clears each flag it consumed, so replays of one launch (one tag) work too.
static std::atomic<unsigned> g_epoch{
    (unsigned)std::chrono::steady_clock::now().time_since_epoch().count() | 1u};
unsigned next_launch_tag() {
    unsigned e;
    do e = g_epoch.fetch_add(1, std::memory_order_relaxed) & ~kSkAbandoned; while (e == 0);
    return e;
}

static thread_local int tl_sk_spins = kSkSpinsDefault;
int sk_spin_limit() { return tl_sk_spins; }
void set_sk_spin_limit(int spins) { tl_sk_spins = spins < 0 ? kSkSpinsDefault : spins; }

hipError_t launch_gemm(GemmBatch& b, hipStream_t s) {
    int total = 0;
    bool all_swiglu = true, all_res = true, all_store = true;
    const bool mfma = b.a_dtype != F32;
    for (int i = 0; i < b.n; ++i) {
        GemmProblem& P = b.p[i];
        const bool sw = P.epi == EPI_SWIGLU;
        all_swiglu &= sw;
        all_res &= P.epi == EPI_GATED_RES;
        all_store &= P.epi == EPI_STORE;
        if (mfma) {
            P.tiles_m = (P.M + BM - 1) / BM;
            P.tiles_n = sw ? (P.N + BN / 2 - 1) / (BN / 2) : (P.N + BN - 1) / BN;
        } else {
            P.tiles_m = (P.M + FBM - 1) / FBM;
            P.tiles_n = (P.N + FBN - 1) / FBN;
        }
        if (P.M == 0) P.tiles_m = 0;
        // the MFMA epilogue handles gated-residual outputs of F32 or BF16 over BF16 or F32 residuals
        if (mfma && P.epi == EPI_GATED_RES && P.M > 0 &&
            ((P.c_dtype != F32 && P.c_dtype != BF16) || (P.r_dtype != F32 && P.r_dtype != BF16)))
            return hipErrorInvalidValue;
        // the MFMA kernel addresses a tile's rows by 32-bit byte offsets from the tile's first row
        if (mfma && P.M > 0 && (P.lda >= kGemmMaxLd || P.ldb >= kGemmMaxLd)) return hipErrorInvalidValue;
        P.tile_begin = total;
        total += P.tiles_m * P.tiles_n;
    }
    b.total_tiles = total;
    if (total == 0) return hipSuccess;
    // Stream-K when at least two full rounds of tiles exist and the last round would leave at
    // least three quarters of the CUs idle (and every problem has the same K).  Split k-ranges
    // cost L2 reuse (co-resident workgroups then read different k-slices of shared A and B
    // panels), so on the block's shapes a partly full last round is cheaper run as it is: at 512
    // text + 4096 image tokens this picks FFN-in (1296 tiles on 256 CUs), not QKV (648) or the
    // d-output GEMMs (216).
    b.sk_grid = 0;
    b.dp_tiles = 0;
    b.k_steps = 0;
    bool same_k = true;
    for (int i = 0; i < b.n; ++i) {
        if (b.p[i].M == 0) continue;
        if (b.k_steps == 0) b.k_steps = b.p[i].K / BK;
        else same_k &= b.p[i].K / BK == b.k_steps;
    }
    const int G = device_cu_count();
    // Fewer tiles than half the CUs (512 + 1024 tokens: the 72 tiles of the d-output GEMMs) split
    // every tile's k-steps over all CUs when each workgroup still gets 12 or more k-steps (the
    // fp32 partials' hand-over past the L2s costs about as much as a few k-steps).  A single
    // partly filled round (216 tiles at 512 + 4096 tokens) stays unsplit: there the split put
    // co-resident workgroups at different k-offsets and ran 114 -> 147 us (out-proj).
    if (mfma && b.sk_scratch && same_k && G > 0 &&
        ((total >= 2 * G && total % G != 0 && 4 * (total % G) <= G) ||
         (2 * total <= G && (long)total * b.k_steps >= 12L * G))) {
        const int D = total / G;
        b.sk_grid = G;
        b.dp_tiles = D >= 1 ? (D - 1) * G : 0;
        b.epoch = next_launch_tag();
        b.sk_spins = sk_spin_limit();
    }
    if (b.a_dtype == F16 && b.b_f16) launch_mfma<F16W>(b, s, all_store, all_res, all_swiglu);
    else if (b.a_dtype == F16) launch_mfma<F16>(b, s, all_store, all_res, all_swiglu);
    else if (b.a_dtype == BF16) launch_mfma<BF16>(b, s, all_store, all_res, all_swiglu);
    else hipLaunchKernelGGL(gemm_f32_kernel, dim3(total), dim3(256), 0, s, b);
    return hipGetLastError();
}

}  // namespace dit
