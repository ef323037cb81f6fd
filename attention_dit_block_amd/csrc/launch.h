// Host-side launchers of the gfx950 kernels (internal to the library).
// Every launcher assumes its arguments were validated by the C ABI layer and launches exactly
// one kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

enum DType { F32 = 0, BF16 = 1, F16 = 2 };
// Bits of a call's range-flag word (device memory; the entry points keep it in their workspace).
// Kernels that round fp32 results to fp16 OR in kRangeF16 when a value is outside fp16's finite
// range (|x| > 65504) or NaN, so it would reach the next step as inf or NaN.
constexpr unsigned kRangeF16 = 1u;
// Output type of the modulate kernel only: OCP e4m3 codes with a per-row fp32 scale.
constexpr int FP8_ROWS = 3;

// ---- AdaLN GEMV: out_p[r] = sum_k W_p[r, k] * SiLU(cond[k]) ------------------
struct GemvProblem {
    const void* w;      // [rows, d_cond]
    float* out;         // [rows]
    int rows;
};
struct GemvBatch {
    GemvProblem p[2];
    int n;
    const void* cond;   // [d_cond]
    int d_cond;
    int dtype;          // dtype of w and cond (F32 or BF16)
    unsigned* clear_flag;   // range-flag word to reset to 0 (the first kernel of a call), or null
};
hipError_t launch_adaln_gemv(const GemvBatch& b, hipStream_t s);

// ---- modulate: out = (1 + scale) * RMSNorm(x) + shift, per row ---------------
struct ModProblem {
    const void* x; long ld_x; int x_dtype;    // F32 or BF16
    void* out; long ld_out;                   // out_dtype of the batch
    const float* shift; const float* scale;   // [d] fp32
    int rows;
    float* out_scale;                         // FP8_ROWS: [rows] per-row scales
};
struct RopeTable {
    double omega_d[64];     // frequency of pair p
    int8_t axis[64];        // position axis of pair p
};
struct ModBatch {
    ModProblem p[2];
    int n;
    int d;
    float eps;
    int out_dtype;      // F32, BF16, F16, or FP8_ROWS: e4m3 codes (bytes, row stride ld_out) quantised per
                        // row as launch_quantize_fp8 does, from the fp32 results
    unsigned* range_flag;   // or null: kRangeF16 when an F16 output is out of range
    unsigned* clear; int clear_n;   // or null: words the kernel sets to 0 (a later kernel's maxima)
    // or null: the kernel also writes the (cos, sin) table of the 64 rotation angles of rope_n
    // tokens, [rope_n][64][2] fp32, with the QK RMSNorm + RoPE pass's angle arithmetic (one angle
    // per thread of the grid, which has at least 64 threads per modulated row; rope_n must not
    // exceed the rows)
    float* rope_cs; const int32_t* rope_pos; int rope_n, rope_n_axes;
    RopeTable rope_tab;
};
hipError_t launch_modulate(const ModBatch& b, hipStream_t s);

// ---- QK RMSNorm + RoPE, in place -----------------------------------------------
struct QkRopeArgs {
    void* q; long ld_q;
    void* k; long ld_k;
    // e4m3 output (qkv8 non-null): q, k stay as they are; the kernel writes codes into qkv8 rows
    // (stride ld8 bytes; q in columns 0 .. d-1, k in d .. 2d-1, v in 2d .. 3d-1, d = n_heads * 128):
    // q per token and head (scales sq [n_tok, n_heads]), k per head with the static scale of the
    // k-norm weights (sk [n_heads]), v (read from v) per head from the maxima vmax (sv [n_heads]);
    // sk and sv are written by workgroup 0.  n_heads <= 256.
    uint8_t* qkv8; long ld8;
    float* sq; float* sk; float* sv;
    const void* v; long ld_v;
    const unsigned* vmax;
    int n_tok, n_heads;
    const void* qk_w0;      // [2 (q, k)][128] for rows n < n_first
    const void* qk_w1;      // [2 (q, k)][128] for rows n >= n_first
    int n_first;
    float eps;
    const int32_t* pos; int n_axes;
    RopeTable tab;
    int dtype;              // q / k: F32, BF16 or F16
    int w_dtype;            // QK-norm weights: F32, BF16 or F16
};
hipError_t launch_qk_rmsnorm_rope(const QkRopeArgs& a, hipStream_t s);

// ---- grouped GEMM  C = epilogue(A . B^T) -----------------------------------------
enum Epilogue {
    EPI_STORE = 0,        // C (c_dtype) = acc
    EPI_GATED_RES = 1,    // C (c_dtype) = R (r_dtype) + gate[col] * acc
    EPI_SWIGLU = 2        // C (c_dtype) = SiLU(acc_gate) * acc_up; B rows [n] gate, [up_off + n] up
};
struct GemmProblem {
    const void* A; long lda;        // [M, K], a_dtype of the batch
    const void* B; long ldb;        // [N_b, K] weights ([out, in]): BF16 (F32 for an F32 batch)
    void* C; long ldc; int c_dtype;
    const void* R; long ldr; int r_dtype;
    const float* gate;              // [N]
    long up_off;                    // SwiGLU: row offset of the up half in B
    int M, N, K;                    // N = output columns
    int epi;
    int tiles_m, tiles_n, tile_begin;   // filled by the launcher
};
struct GemmBatch {
    GemmProblem p[2];
    int n;
    int a_dtype;        // F32 (fp32 path, fp32 weights), BF16 (bf16 weights) or F16 (bf16 weights,
                        // converted to fp16 while they are staged)
    bool b_f16;         // F16 activations only: the weights are fp16 copies, staged as they are
    int group_m;        // tile raster: groups of group_m M-tiles, N-major inside a group (0: 4)
    int total_tiles;    // filled by the launcher
    // Stream-K scratch (16-B-aligned device memory of gemm_sk_scratch_bytes(), or null: one
    // workgroup per tile).  The launcher fills the rest: a persistent grid of sk_grid
    // workgroups runs tiles [0, dp_tiles) whole and splits the k-steps of the others evenly.
    void* sk_scratch;
    int sk_grid, dp_tiles, k_steps;
    unsigned epoch;
    int sk_spins;       // bound on an owner's wait for a piece (then it computes the piece itself)
    unsigned* range_flag;   // or null: kRangeF16 when an F16 output is out of range
    // QK RMSNorm + 4-axis RoPE applied to the accumulators of EPI_STORE tiles before they are
    // stored (MFMA batches, rope_cs non-null): output columns [0, rope_d) of each problem are q,
    // [rope_d, 2 rope_d) k, 128 per head (rope_d a multiple of 256), normalised with the
    // problem's bf16 weights rope_w[p] ([2 (q, k)][128]) and rotated by the (cos, sin) pairs of
    // token rope_row0[p] + row in rope_cs ([n_tok][64 pairs][2], written by the modulation).
    const float* rope_cs; int rope_d; float rope_eps;
    const void* rope_w[2]; int rope_row0[2];
};
// Row strides (lda, ldb) of the 16-bit GEMMs are below this many elements (launch_gemm returns
// hipErrorInvalidValue otherwise; the entry points reject such strides first).
constexpr long kGemmMaxLd = 1L << 22;
hipError_t launch_gemm(GemmBatch& b, hipStream_t s);
// Bytes of stream-K scratch launch_gemm uses on the current device (0 if it cannot tell).
size_t gemm_sk_scratch_bytes();

// ---- joint attention ---------------------------------------------------------------
struct AttnArgs {
    const void* q; long ld_q;
    const void* k; long ld_k;
    const void* v; long ld_v;
    void* o; long ld_o;
    int n_tok, n_heads;
    float scale;
    int dtype;          // F32, BF16 or F16
    // Stream-K scratch (16-B-aligned device memory of attention_sk_scratch_bytes(), or null:
    // one workgroup per (head, query tile) unit).  The launcher fills the rest.
    void* sk_scratch;
    int sk_grid, sk_segs, units, k_tiles;
    unsigned epoch;
    int sk_spins;       // bound on an owner's wait for a piece (then it computes the piece itself)
};
hipError_t launch_attention(AttnArgs& a, hipStream_t s);
size_t attention_sk_scratch_bytes();

// ---- joint attention on e4m3 operands ----------------------------------------------------
struct AttnFp8Args {
    const void* q; long ld_q;           // e4m3 codes; strides in bytes (multiples of 16)
    const float* q_scale;               // [n_tok, n_heads]
    const void* k; long ld_k;
    const float* k_scale;               // [n_heads]
    const void* v; long ld_v;
    const float* v_scale;               // [n_heads]
    void* o; long ld_o;                 // o_dtype elements
    int o_dtype;                        // F32, BF16 or F16
    int n_tok, n_heads;
    float scale;
    // Key-split scratch (16-B-aligned device memory of attention_sk_scratch_bytes(), or null: one
    // workgroup per (head, query tile) unit).  The launcher fills the rest.
    void* sk_scratch;
    int sk_grid, sk_segs, units, k_tiles;
    unsigned epoch;
    int sk_spins;
};
hipError_t launch_attention_fp8(AttnFp8Args& a, hipStream_t s);

// ---- calibration: a loop of fp16 MFMAs, 4 waves x 4 chains x iters per workgroup ----------
hipError_t launch_mfma_loop(int workgroups, int iters, float* out, hipStream_t s);
hipError_t launch_gemm_kloop_probe(int mode, int workgroups, int ksteps, const void* win, float* out, hipStream_t s);
hipError_t launch_attention_step_probe(int mode, int workgroups, int tiles, float c2, float* out, hipStream_t s);
// ---- calibration: streaming read (mode 0, one float per thread into sink) or copy (mode 1) ----
hipError_t launch_stream_probe(const void* src, void* dst, size_t bytes, int mode, int workgroups, float* sink,
                               hipStream_t s);

// ---- windowed (neighborhood) attention over a [T, H, W] token grid --------------------------
struct WinAttnArgs {
    const void* q; long ld_q;
    const void* k; long ld_k;
    const void* v; long ld_v;
    void* o; long ld_o;
    int T, H, W;            // grid; token (t, h, w) is row (t * H + h) * W + w
    int kT, kH, kW;         // effective window per axis: min(requested, extent)
    int rT, rH, rW;         // requested (odd) window per axis, for the window start
    int n_heads;
    float scale;
    int dtype;              // F32, BF16 or F16
    int tiles_h, tiles_w;   // filled by the launcher
};
hipError_t launch_window_attention(WinAttnArgs& a, hipStream_t s);
// Largest effective window along W the 16-bit kernel handles, and the most window keys the fp32
// kernel handles.
constexpr int kWinMaxKW = 49;
constexpr int kWinMaxKeysF32 = 4096;

// ---- fp8 (OCP e4m3) quantisation and GEMM ---------------------------------------------------
// q [rows, cols] e4m3 codes, scales [rows] fp32: s = max|x_row| / 448 (1 for a zero row),
// q = e4m3(x / s) rounded to nearest even.  x: F32, BF16 or F16; cols % 8 == 0.
hipError_t launch_quantize_fp8(const void* x, int x_dtype, long ld_x, int rows, int cols, uint8_t* q, long ld_q,
                               float* scales, hipStream_t s);
struct Fp8GemmProblem {
    const uint8_t* a; long lda; const float* sa;   // [M, K] codes, [M] scales
    const uint8_t* b; long ldb; const float* sb;   // [N_b, K] codes, [N_b] scales
    void* c; long ldc; int c_dtype;                // [M, N]: epilogue(sa[m] sb[n] sum_k a b)
    const void* r; long ldr; int r_dtype;          // EPI_GATED_RES: residual (F32 or BF16)
    const float* gate;                             // EPI_GATED_RES: [N]
    long up_off;                                   // EPI_SWIGLU: row offset of the up half in b and sb
    int M, N, K, epi;                              // K % 128 == 0, N % 4 == 0
    int tiles_m, tiles_n, tile_begin;              // filled by the launcher
};
struct Fp8GemmBatch {
    Fp8GemmProblem p[2];
    int n;              // every problem has p[0].epi
    int total_tiles;    // filled by the launcher
    unsigned* range_flag;   // or null: kRangeF16 when an F16 output is out of range
    // EPI_STORE only, or null: for output columns from vmax_col0 on (a multiple of 128), the largest
    // |stored value| of each 128-column head, as fp32 bits, raised by atomic max (every problem of
    // the batch into the same words; the caller zeroes them first)
    unsigned* vmax; int vmax_col0;
};
hipError_t launch_gemm_fp8(Fp8GemmBatch& g, hipStream_t s);

// ---- 2-D convolution (NHWC), implicit GEMM ----------------------------------------------------
struct ConvArgs {
    const void* x;          // [B, T, H, W, Cin], BF16
    const void* w;          // [Cout, KT, KH, KW, Cin], BF16
    const float* bias;      // [Cout] or null
    void* y; int y_dtype;   // [B, T, H, W, Cout]
    int B, H, W, Cin, Cout, KH, KW;     // stride 1, zero padding (K - 1) / 2 in h and w
    int T, KT;              // frames per clip and temporal taps: frames t-KT+1 .. t (zeros before 0);
                            // T = KT = 1: the 2-D convolution
    int tiles_m, tiles_n;   // filled by the launcher
};
hipError_t launch_conv2d(ConvArgs& a, hipStream_t s);

// ---- layers either side of the block stack ---------------------------------------------
// emb [dim] fp32 = [cos(s f_j), sin(s f_j)], s = time_factor * t[0], f_j = max_period^(-j / (dim/2))
hipError_t launch_freq_embed(const float* t, double time_factor, double max_period, int dim, float* emb,
                             hipStream_t s);
// out [rows] fp32 (+)= W [rows, K] (w_dtype F32 or BF16) . act(v), act = SiLU if silu_in
hipError_t launch_vec_gemv(const void* w, int w_dtype, int rows, int K, const float* v, bool silu_in, float* out,
                           bool accumulate, hipStream_t s);
hipError_t launch_cast(const float* in, void* out, int n, int dtype, hipStream_t s);
// out[i] = fp16(in[i]) for bf16 in (16-byte aligned in and out)
hipError_t launch_bf16_to_f16(const void* in, void* out, size_t n, hipStream_t s);
// out = (1 + scale) * LayerNorm(x) + shift per row (x: F32 or BF16)
hipError_t launch_layernorm_modulate(const void* x, int x_dtype, long ld_x, void* out, int out_dtype, long ld_out,
                                     const float* shift, const float* scale, int rows, int d, float eps,
                                     hipStream_t s);

// Compute units of the current device (0 if unknown), and nonzero launch tags unique in the
// process (below 2^31), for the stream-K grids.
int device_cu_count();
unsigned next_launch_tag();
// The calling thread's bound on a stream-K owner's wait for a piece, in polls of the flag
// (default kSkSpinsDefault; 0: owners compute every piece whose partial is not already there).
constexpr int kSkSpinsDefault = 1 << 22;
int sk_spin_limit();
void set_sk_spin_limit(int spins);

}  // namespace dit
