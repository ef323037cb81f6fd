/*
 * dit.h -- C ABI of the MI355X (gfx950) forward pass of a FLUX-style joint
 * text+image DiT transformer block.
 *
 * The block (antirez/iris.c issue #15, "CUDA codepath !"): the transformer of
 * the FLUX Klein image model, whose operations are the QKV projections, the
 * FFN and the attention scores (matrix products) plus RMSNorm, RoPE, AdaLN
 * modulation, softmax and activations (ServeurpersoCom's reply on the
 * cuBLAS / custom-kernel split); its RoPE has 4 axes of [32, 32, 32, 32] dims
 * with separate text and image positions (the GGML update, item 3); and it is
 * "AdaLN + custom RoPE + joint attention" (the GGML update's bottom line).
 * The remaining conventions are FLUX's and are stated per call below.
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE pointers unless marked (host).  The caller allocates
 *    and frees every buffer; the library keeps no device memory and no caches.
 *  - Every call enqueues its kernels on `stream` (a hipStream_t; NULL = the
 *    default stream), returns without synchronising, allocates nothing and
 *    never writes an input buffer.
 *  - Matrices are row-major.  Linear weights are [out, in], so y = x W^T.
 *    `ld*` arguments are row strides in ELEMENTS.
 *  - Element types: DIT_BF16 and DIT_F16 (16-bit storage, fp32 accumulation)
 *    and DIT_F32 (fp32 storage and arithmetic, no reduced-precision matrix
 *    math).  A bf16 model keeps its weights and block input in bf16; the
 *    activations handed between the block's steps may be carried in fp16
 *    (act_dtype), whose 10-bit mantissa keeps the block output within 2e-2
 *    (max |err| / RMS) of exact arithmetic where bf16's 7 bits do not.
 *  - Alignment: every pointer 16-byte aligned, every row stride a multiple of
 *    16 bytes.
 *  - Errors: arguments are validated on the host before any launch.  On a
 *    failed check the call returns a dit_status code, sets the thread-local
 *    message returned by dit_last_error() and launches nothing.  A HIP launch
 *    error after validation returns DIT_ERR_HIP.  No call aborts or throws.
 *  - Threading: reentrant; the only state is thread-local (error text,
 *    launch counter, kernel timing).
 */
#ifndef DIT_H
#define DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIT_ABI_VERSION 1

enum dit_dtype { DIT_F32 = 0, DIT_BF16 = 1, DIT_F16 = 2 };

enum dit_status {
    DIT_OK = 0,
    DIT_ERR_INVALID_ARG = 1,   /* null / misaligned pointer, bad size or stride */
    DIT_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. head_dim != 128) */
    DIT_ERR_WORKSPACE = 3,     /* workspace smaller than dit_block_workspace_size() */
    DIT_ERR_HIP = 4            /* a HIP runtime call failed */
};

/*
 * AdaLN modulation (the thread's "AdaLN modulation" kernel).
 *
 *   mod_out = W_mod . SiLU(cond)                       [n_chunks * d] fp32
 *   x_out   = (1 + mod[scale_chunk]) * RMSNorm(x) + mod[shift_chunk]
 *
 * RMSNorm(x) = x / sqrt(mean_j x_j^2 + eps) over the d features of a row
 * (no learnable weight).  Chunk c of mod_out is mod_out[c*d .. c*d + d - 1];
 * the FLUX order is shift, scale, gate (twice for a double-stream block).
 *
 *  dtype     storage type of cond and w_mod: DIT_BF16 or DIT_F32
 *  cond      [d_cond]
 *  w_mod     [n_chunks * d, d_cond]
 *  mod_out   [n_chunks * d] fp32
 *  x         optional, [n_tok rows, stride ld_x] of x_dtype (DIT_BF16 or
 *            DIT_F32).  NULL: only mod_out is computed.
 *  x_out     [n_tok rows, stride ld_out] of out_dtype (DIT_BF16, DIT_F16 or
 *            DIT_F32; DIT_F32 for an fp32 call); must not overlap x.
 * Limits: 8 <= d <= 8192, d % 8 == 0, 8 <= d_cond <= 16384, d_cond % 8 == 0, n_tok >= 0.
 */
int dit_adaln_modulate(int dtype, void* stream,
                       const void* cond, int d_cond,
                       const void* w_mod, int n_chunks, int d,
                       float* mod_out,
                       const void* x, int x_dtype, int n_tok, long ld_x,
                       int shift_chunk, int scale_chunk, float eps,
                       void* x_out, int out_dtype, long ld_out);

/*
 * Per-head QK RMSNorm followed by 4-axis RoPE, in place
 * (the thread's "RMSNorm" and "RoPE" kernels; RoPE as in the GGML update,
 * item 3).
 *
 * For every token n and head h, with u = q[n, h*128 .. h*128+127]:
 *   u <- u / sqrt(mean(u^2) + eps) * w_q          (w_k for k)
 *   then every interleaved pair (u[2p], u[2p+1]) is rotated by +phi:
 *   (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi),
 *   phi = pos[n, ax] * theta^(-2j / axes_dim[ax]) for pair j of axis ax,
 *   axis ax owning dims [sum(axes_dim[:ax]), + axes_dim[ax]).
 *
 *  dtype     element type of q and k (DIT_BF16, DIT_F16 or DIT_F32)
 *  q, k      [n_tok rows, stride ld_q / ld_k], n_heads*head_dim columns each
 *            (may be column views of one qkv buffer)
 *  qk_w      [2 sets][2 (q, k)][head_dim] of w_dtype: rows n < n_first use
 *            set 0 (text), the others set 1 (image).  If n_first >= n_tok
 *            only set 0 is read.
 *  pos       int32 [n_tok, n_axes]
 *  axes_dim  (host) [n_axes], each even, summing to head_dim
 * Limits: head_dim == 128, 1 <= n_axes <= 4, n_heads >= 1, n_tok >= 0
 * (n_tok == 0: nothing is read or written).
 */
int dit_qk_rmsnorm_rope(int dtype, void* stream,
                        void* q, long ld_q, void* k, long ld_k,
                        int n_tok, int n_heads, int head_dim,
                        const void* qk_w, int w_dtype, int n_first, float eps,
                        const int32_t* pos, int n_axes, const int* axes_dim, float theta);

/*
 * Joint softmax attention over all n_tok tokens (text and image in one
 * softmax, no mask, not causal) -- the thread's "attention scores" product
 * and "softmax" kernel, here fused (flash style: the scores are never
 * stored).
 *
 *   O_h = softmax(Q_h K_h^T * softmax_scale) V_h       for every head h
 *
 *  dtype     element type of q, k, v and o (DIT_BF16, DIT_F16 or DIT_F32)
 *  q, k, v   [n_tok rows, stride ld_q/ld_k/ld_v]; head h = columns
 *            h*head_dim .. h*head_dim + head_dim - 1
 *  o         [n_tok rows, stride ld_o] of dtype; must not overlap q, k, v
 *  softmax_scale  usually 1/sqrt(head_dim)
 * Scores, softmax and accumulation are fp32; the 16-bit paths pass the
 * probabilities to the PV product within 2^-11 (fp16) or 2^-16 (bf16, two
 * terms) of their fp32 values.
 * Limits: head_dim == 128, n_heads >= 1, n_tok >= 0 (n_tok == 0: nothing is
 * read or written).
 */
int dit_joint_attention(int dtype, void* stream,
                        const void* q, long ld_q, const void* k, long ld_k,
                        const void* v, long ld_v,
                        void* o, long ld_o, int n_tok, int n_heads, int head_dim,
                        float softmax_scale);

/* Shapes and constants of one block. */
typedef struct dit_block_config {
    int dtype;          /* weights and cond: DIT_BF16 or DIT_F32 */
    int act_dtype;      /* activations between the steps (a, qkv, O, b, f): DIT_F16 or
                           DIT_BF16 for bf16 weights, DIT_F32 for fp32 weights */
    int x_dtype;        /* block input x (residual stream): DIT_BF16 or DIT_F32 */
    int y_dtype;        /* block output y: DIT_F32 or DIT_BF16 */
    int d;              /* hidden size = n_heads * head_dim */
    int n_heads;
    int head_dim;       /* must be 128 */
    int ffn_inner;      /* F, SwiGLU inner width; multiple of 128, at most 2^20 */
    int d_cond;         /* conditioning vector length; multiple of 8 */
    int n_txt;          /* text tokens (first in the joint sequence) */
    int n_img;          /* image tokens */
    float eps;          /* pre-norm RMSNorm epsilon */
    float eps_qk;       /* QK-norm epsilon */
    float theta;        /* RoPE base (1e4 for FLUX) */
    int n_axes;         /* RoPE axes (4) */
    int axes_dim[4];    /* dims per axis ({32,32,32,32}) */
    int gemm_w_dtype;   /* storage of the matrix-product weights (w_qkv, w_o, w_ffn_in,
                           w_ffn_out; w_1, w_2): 0 = dtype; DIT_F16 (dtype DIT_BF16 with
                           DIT_F16 activations only) = fp16 copies of the bf16 weights made
                           once by dit_convert_bf16_to_f16, which the GEMMs stage without
                           converting (results identical to the bf16 weights); w_mod,
                           qk_norm_w and cond stay of dtype */
} dit_block_config;

/* Weights of one stream of a double-stream block ([out, in], dtype). */
typedef struct dit_stream_weights {
    const void* w_mod;      /* [6d, d_cond]: shift1, scale1, gate1, shift2, scale2, gate2 */
    const void* w_qkv;      /* [3d, d]: rows q | k | v, head-major inside each */
    const void* qk_norm_w;  /* [2][head_dim]: q weight, k weight */
    const void* w_o;        /* [d, d] */
    const void* w_ffn_in;   /* [2F, d]: rows 0..F-1 gate (SiLU), F..2F-1 up */
    const void* w_ffn_out;  /* [d, F] */
} dit_stream_weights;

/* Weights of a single-stream block (fused parallel attention + SwiGLU MLP). */
typedef struct dit_single_weights {
    const void* w_mod;      /* [3d, d_cond]: shift, scale, gate */
    const void* w_1;        /* [3d + 2F, d]: rows q | k | v | gate | up */
    const void* qk_norm_w;  /* [2][head_dim]: q weight, k weight */
    const void* w_2;        /* [d, d + F]: input columns [O | f] */
} dit_single_weights;

/* Workspace bytes needed by dit_block_forward (single_stream = 0) or
 * dit_single_block_forward (single_stream = 1).  (host) cfg.  Returns 0 for
 * an invalid config (see dit_last_error()). */
size_t dit_block_workspace_size(const dit_block_config* cfg, int single_stream);

/*
 * Double-stream block forward (text and image streams with their own weights,
 * one joint attention):
 *   m_s = W_mod,s SiLU(c);  a_s = (1+scale1) RMSNorm(x_s) + shift1
 *   [q|k|v]_s = a_s W_qkv,s^T;  q,k <- RoPE(RMSNorm_head(.) * w_{q,k},s)
 *   O = joint attention over [text; image];  h_s = x_s + gate1 (O_s W_o,s^T)
 *   b_s = (1+scale2) RMSNorm(h_s) + shift2;  [g|u] = b_s W_in,s^T
 *   y_s = h_s + gate2 ((SiLU(g) * u) W_down,s^T)
 * Storage: the AdaLN vectors and h are fp32; a, qkv, O, b and f are
 * act_dtype; x is x_dtype and y is y_dtype.  With bf16 weights and d a
 * multiple of 256 the QK RMSNorm + RoPE is applied to the q and k products'
 * fp32 values before they are stored (otherwise to the stored act_dtype
 * values, by a pass of its own).
 *
 *  cfg, txt, img (host)
 *  cond      [d_cond] of dtype (shared by both streams)
 *  pos       int32 [n_txt + n_img, n_axes], text tokens first
 *  x_txt     [n_txt, d], x_img [n_img, d] of x_dtype (contiguous rows)
 *  y_txt     [n_txt, d], y_img [n_img, d] of y_dtype; y may alias x when
 *            x_dtype == y_dtype, otherwise must not overlap it
 *  workspace >= dit_block_workspace_size(cfg, 0) bytes, scratch (never
 *            zeroed, contents undefined afterwards); must not overlap any
 *            other argument.  Calls sharing a workspace must be ordered on
 *            one stream.  Its first 4 bytes are the call's range-flag word
 *            (dit_workspace_flags): the call resets it in its first kernel and
 *            sets DIT_RANGE_F16 when an fp16 activation (act_dtype DIT_F16)
 *            leaves fp16's finite range, so the output is not to be trusted.
 */
int dit_block_forward(const dit_block_config* cfg,
                      const dit_stream_weights* txt, const dit_stream_weights* img,
                      const void* cond, const int32_t* pos,
                      const void* x_txt, const void* x_img, void* y_txt, void* y_img,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * Single-stream block forward over the concatenated sequence x = [text; image]:
 *   m = W_mod SiLU(c);  a = (1+scale) RMSNorm(x) + shift
 *   [q|k|v|g|u] = a W_1^T;  q,k <- RoPE(RMSNorm_head(.) * w_{q,k})
 *   O = joint attention;  y = x + gate ([O | SiLU(g) * u] W_2^T)
 *  x, y      [n_txt + n_img, d] of x_dtype / y_dtype; aliasing as above
 *  Other arguments as for dit_block_forward (one qk_norm_w set).
 */
int dit_single_block_forward(const dit_block_config* cfg, const dit_single_weights* w,
                             const void* cond, const int32_t* pos,
                             const void* x, void* y,
                             void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes needed by dit_step_forward with n_double / n_single blocks
 * (the larger of the two block kinds' needs).  (host) cfg.  Returns 0 for an
 * invalid config or negative counts. */
size_t dit_step_workspace_size(const dit_block_config* cfg, int n_double, int n_single);

/*
 * The block stack of one denoising step: n_double double-stream blocks, then
 * n_single single-stream blocks over [text; image], all with one conditioning
 * vector (the transformer of the FLUX-style model the "CUDA codepath !" thread
 * runs, antirez/iris.c issue #15).  Every launch goes to `stream` and nothing
 * synchronises or allocates, so the whole step can be captured into one graph
 * and replayed (the reusable-graph approach of the fak GPU page, "GPU -- the
 * in-kernel forward pass, on the GPU", section 3b).
 *
 *  cfg (host): x_dtype is the type of x_txt / x_img; y_dtype is ignored (the
 *            stream y is fp32).  act_dtype as for the blocks.
 *  txt, img  (host) arrays of n_double stream weights (block order)
 *  single    (host) array of n_single single-block weights
 *  x_txt, x_img  the stack's input, [n_txt, d] and [n_img, d] of x_dtype.  With
 *            n_double = 0, x_img must directly follow x_txt.
 *  y         fp32 [n_txt + n_img, d], text rows first: the first block writes it
 *            from x, every later block updates it in place; it holds the stack's
 *            output at the end.  Must not overlap x.
 *  workspace >= dit_step_workspace_size(cfg, n_double, n_single) bytes, as for
 *            the blocks.
 * All arguments of all blocks are validated before the first launch; an error
 * launches nothing.  9 launches per double-stream block (8 when its QK RMSNorm
 * + RoPE runs in the QKV product's epilogue: bf16 weights, d a multiple of
 * 256), 6 per single-stream block.
 */
int dit_step_forward(const dit_block_config* cfg, int n_double,
                     const dit_stream_weights* txt, const dit_stream_weights* img,
                     int n_single, const dit_single_weights* single,
                     const void* cond, const int32_t* pos,
                     const void* x_txt, const void* x_img, float* y,
                     void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes of dit_step_forward_shared_mod: dit_step_workspace_size
 * rounded up to 256 bytes, plus 15 * d fp32 AdaLN values. */
size_t dit_step_shared_mod_workspace_size(const dit_block_config* cfg, int n_double, int n_single);

/*
 * dit_step_forward with shared modulation: one set of AdaLN weights serves
 * every double-stream block (one matrix per stream) and another every
 * single-stream block, so the step computes its AdaLN vectors once -- one
 * GEMV launch per block kind instead of one per block (the "one GEMV per
 * step" variant of the denoising step of a FLUX-style model, the FLUX Klein
 * transformer the "CUDA codepath !" thread runs).  The per-block w_mod fields
 * are not read and may be NULL.
 *  w_mod_txt, w_mod_img  [6d, d_cond] of dtype (needed when n_double > 0)
 *  w_mod_single          [3d, d_cond] of dtype (needed when n_single > 0)
 *  workspace >= dit_step_shared_mod_workspace_size(cfg, n_double, n_single)
 * Other arguments and guarantees as for dit_step_forward; 8 launches per
 * double-stream block (7 with the QK RMSNorm + RoPE in the QKV product) and 5
 * per single-stream block, plus 1 per block kind.
 * With every block's w_mod equal to the shared matrix the result is
 * bit-identical to dit_step_forward's.
 */
int dit_step_forward_shared_mod(const dit_block_config* cfg, int n_double,
                                const dit_stream_weights* txt, const dit_stream_weights* img,
                                int n_single, const dit_single_weights* single,
                                const void* w_mod_txt, const void* w_mod_img, const void* w_mod_single,
                                const void* cond, const int32_t* pos,
                                const void* x_txt, const void* x_img, float* y,
                                void* workspace, size_t ws_bytes, void* stream);

/*
 * The layers either side of the block stack.  The pages name the step's
 * transformer but print none of them; they follow the FLUX model (no biases,
 * like the block).
 */

/* Workspace bytes of dit_timestep_embedding (fp32 scratch: freq_dim + 2 d
 * values, each part 256-byte aligned); 0 for invalid sizes. */
size_t dit_timestep_embedding_workspace_size(int freq_dim, int d);

/*
 * Conditioning vector from the timestep (and optional guidance) value:
 *   emb(v) = [cos(s f_0) .. cos(s f_{h-1}), sin(s f_0) .. sin(s f_{h-1})],
 *            s = time_factor * v, h = freq_dim / 2, f_j = max_period^(-j/h)
 *   cond   = W_t_out SiLU(W_t_in emb(t))  [+ W_g_out SiLU(W_g_in emb(g))]
 * summed in fp32 and rounded once to dtype.  FLUX: freq_dim 256,
 * max_period 1e4, time_factor 1000.
 *  dtype     weights and cond_out: DIT_BF16 or DIT_F32
 *  t         fp32 [1] on the device (a graph replay picks up a new value)
 *  g         fp32 [1] on the device, or NULL (no guidance term; w_g_* unused)
 *  w_t_in, w_g_in    [d, freq_dim];  w_t_out, w_g_out  [d, d]
 *  cond_out  [d] of dtype (the cond argument of the block calls)
 *  workspace >= dit_timestep_embedding_workspace_size(freq_dim, d) bytes
 * Limits: freq_dim and d multiples of 8 in [8, 16384]; max_period > 1.
 * 4 launches (7 with guidance).
 */
int dit_timestep_embedding(int dtype, void* stream, const float* t, const float* g,
                           const void* w_t_in, const void* w_t_out,
                           const void* w_g_in, const void* w_g_out,
                           int freq_dim, int d, float max_period, float time_factor,
                           void* cond_out, void* workspace, size_t ws_bytes);

/*
 * dit_timestep_embedding for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * kernels and result, with the scratch in a static device array of the library
 * (DIT_TEMB_STATIC_SCRATCH bytes per GPU, held until the process ends) instead of a
 * caller workspace.  The call allocates nothing.
 * Limit: dit_timestep_embedding_workspace_size(freq_dim, d) <= DIT_TEMB_STATIC_SCRATCH
 * (e.g. freq_dim 256 with d up to 8064); larger sizes return DIT_ERR_UNSUPPORTED.
 * Every call on one GPU shares that GPU's array: calls that can overlap on one GPU
 * (different streams without ordering, different threads) race and must not be
 * issued; calls ordered on one stream are fine.  Other arguments as above.
 */
#define DIT_TEMB_STATIC_SCRATCH 65536
int dit_timestep_embedding_noalloc(int dtype, void* stream, const float* t, const float* g,
                                   const void* w_t_in, const void* w_t_out,
                                   const void* w_g_in, const void* w_g_out,
                                   int freq_dim, int d, float max_period, float time_factor,
                                   void* cond_out);

/*
 * y = x W^T on the block's GEMM kernel: the patch embedding of the image
 * latents ([n_img, 64] -> [n_img, d] for 16 latent channels in 2x2 patches),
 * the text embedding, or any other projection without bias.
 *  dtype     of w [n, k]: DIT_BF16 (x DIT_BF16 or DIT_F16, fp32 accumulation)
 *            or DIT_F32 (x and y DIT_F32, fp32 arithmetic)
 *  x         [m, k] of x_dtype, row stride ld_x;  y [m, n] of y_dtype, ld_y
 * Limits: n a multiple of 8; k a multiple of 64 (bf16) or 16 (fp32); bf16:
 * k and ld_x below 2^22 (DIT_ERR_UNSUPPORTED otherwise); y must not overlap
 * x or w.  One launch.
 */
int dit_linear(int dtype, void* stream, const void* x, int x_dtype, long ld_x,
               const void* w, int m, int n, int k, void* y, int y_dtype, long ld_y);

/* Workspace bytes of dit_final_layer: 2 d fp32 values + n_tok rows of d
 * act_dtype values (each part 256-byte aligned). */
size_t dit_final_layer_workspace_size(int n_tok, int d, int act_dtype);

/*
 * Last layer of the model over the image tokens:
 *   [shift, scale] = W_mod SiLU(cond)                         (2 d, fp32)
 *   a = (1 + scale) LayerNorm(x) + shift,  LayerNorm(x) = (x - mean) / sqrt(var + eps)
 *       over the d features of a row (population variance, no affine)
 *   y = a W_out^T
 *  dtype     of cond, w_mod [2d, d_cond] and w_out [p, d]: DIT_BF16 or DIT_F32
 *  act_dtype storage of a (DIT_F16 or DIT_BF16 for bf16 weights, DIT_F32)
 *  x         [n_tok, d] of x_dtype (DIT_F32 or DIT_BF16), contiguous rows --
 *            e.g. the image rows of dit_step_forward's y
 *  y         [n_tok, p] of y_dtype, contiguous rows (p = 64 for FLUX's 2x2
 *            patches of 16 channels); must not overlap x
 * Limits: d a multiple of 64 in [64, 8192]; p a multiple of 8.  3 launches.
 */
int dit_final_layer(int dtype, int act_dtype, void* stream, const void* x, int x_dtype,
                    int n_tok, int d, const void* cond, int d_cond, const void* w_mod,
                    const void* w_out, int p, float eps, void* y, int y_dtype,
                    void* workspace, size_t ws_bytes);

/*
 * Windowed (neighborhood) attention over a [T, H, W] token grid (the
 * neighborhood-attention kernel of the diffusion-VAE decoder page; LTX-2.5's
 * decoder uses a [11, 11, 11] window).  Token (t, h, w) is row
 * (t * H + h) * W + w of q, k, v and o.  Per head, the query at (t, h, w)
 * attends to the keys of its window: along each axis the min(kernel, extent)
 * consecutive positions starting at clamp(i - kernel / 2, 0, extent - size) --
 * centred where it fits, shifted inwards at an edge, and the whole axis when
 * the window is wider than the grid.
 *   o = softmax(q K_win^T * softmax_scale) V_win
 *  dtype     DIT_BF16 or DIT_F16 (fp32 accumulation; MFMA) or DIT_F32
 *  q, k, v, o  [T*H*W, n_heads * head_dim] views with row strides ld_*
 *  grid, kernel  (host) int[3]: extents T, H, W and the requested window, each
 *            window size a positive odd number
 * Limits: head_dim 128; at most 2^24 tokens; 16-bit: softmax_scale > 0 and at
 * most 49 positions of window along W; fp32: at most 4096 keys per window.
 * o must not overlap q, k or v.  One launch.
 */
int dit_neighborhood_attention(int dtype, void* stream,
                               const void* q, long ld_q, const void* k, long ld_k,
                               const void* v, long ld_v, void* o, long ld_o,
                               const int* grid, const int* kernel,
                               int n_heads, int head_dim, float softmax_scale);

/*
 * fp8 (OCP e4m3) variant of the matrix products: 8-bit floats with 1 sign, 4
 * exponent (bias 7) and 3 mantissa bits, largest finite 448, one fp32 scale
 * per row of each operand -- the speed-for-accuracy trade the thread weighs
 * ("slight (invisible) loss of accuracy"), on MI355X's fp8 MFMA (twice the
 * dense bf16 peak).
 *
 * dit_quantize_fp8: per row r of x [rows, cols] (x_dtype DIT_F32, DIT_BF16 or
 *   DIT_F16, row stride ld_x): scales[r] = max_j |x[r, j]| / 448 (1 for an
 *   all-zero row) and q[r, j] = e4m3(x[r, j] / scales[r]), rounded to
 *   nearest even; both divisions correctly rounded in fp32.  q is bytes with
 *   row stride ld_q (>= cols, multiple of 16); cols a multiple of 8.
 * dit_linear_fp8: y[i, j] = sx[i] sw[j] sum_k dec(xq[i, k]) dec(wq[j, k]),
 *   fp32 accumulation, y of y_dtype (DIT_F32, DIT_BF16 or DIT_F16, stride
 *   ld_y).  xq [m, k], wq [n, k] e4m3 codes with byte strides ld_x, ld_w
 *   (multiples of 16); sx [m], sw [n] fp32.  k a multiple of 128, n a
 *   multiple of 8.  One launch each.
 */
int dit_quantize_fp8(int x_dtype, void* stream, const void* x, long ld_x, int rows, int cols,
                     void* q, long ld_q, float* scales);
int dit_linear_fp8(void* stream, const void* xq, long ld_x, const float* sx,
                   const void* wq, long ld_w, const float* sw, int m, int n, int k,
                   void* y, int y_dtype, long ld_y);

/*
 * Joint attention with e4m3 operands: dit_joint_attention's softmax attention
 * with both products (the scores and the PV product) on fp8 MFMA.
 *
 *   O_h = softmax(diag(sq_h) dec(Q_h) dec(K_h)^T sk_h * softmax_scale)
 *         dec(V_h) sv_h                                      for every head h
 *
 *  q8, k8, v8  e4m3 codes [n_tok rows, byte strides ld_q/ld_k/ld_v]; head h
 *              = columns h*128 .. h*128 + 127.  Strides multiples of 16 and
 *              below 2^25, base pointers 16-byte aligned.
 *  q_scale     fp32 [n_tok, n_heads] (sq_h = column h): one scale per token
 *              and head, as dit_quantize_fp8 writes for the rows of one head
 *  k_scale, v_scale  fp32 [n_heads]: one scale per head (sk_h, sv_h)
 *  o           [n_tok rows, stride ld_o elements] of o_dtype (DIT_F32,
 *              DIT_BF16 or DIT_F16); must not overlap the inputs
 * Scores and softmax are fp32; the probabilities enter the PV product rounded
 * to e4m3 (each within 2^-4 of its value relative to the tile's running max,
 * or 2^-10 absolutely below e4m3's normal range); the normaliser is the
 * fp32 sum of the unrounded probabilities.  Codes 0x7f / 0xff (NaN) and
 * non-finite scales give non-finite outputs.
 * Limits: head_dim == 128, n_heads >= 1, n_tok >= 0 (n_tok == 0: nothing is
 * read or written), n_tok * n_heads <= 2^30.  One launch, one workgroup per
 * (head, 256 queries).
 */
int dit_joint_attention_fp8(void* stream,
                            const void* q8, long ld_q, const float* q_scale,
                            const void* k8, long ld_k, const float* k_scale,
                            const void* v8, long ld_v, const float* v_scale,
                            void* o, int o_dtype, long ld_o,
                            int n_tok, int n_heads, int head_dim, float softmax_scale);

/*
 * Calibration for measurements (not part of the block): `workgroups`
 * workgroups of 4 waves each run iters x 4 independent
 * v_mfma_f32_32x32x16_f16 (32768 flop each) with no memory traffic, then
 * write one float per thread to out [workgroups * 256].  Its rate is the
 * matrix cores' sustained fp16 throughput at the device's present clock.
 */
int dit_mfma_loop(void* stream, int workgroups, int iters, float* out);

/*
 * Calibration for measurements (not part of the block): a grid-stride stream
 * over `bytes` (a positive multiple of 16384) of src with 16-byte nontemporal
 * accesses, `workgroups` workgroups of 256 threads.  mode 0 reads src and
 * writes one float per thread to sink [workgroups * 256] (the HBM read
 * ceiling); mode 1 copies src to dst (read + write ceiling), dst not
 * overlapping src.  src, dst 16-byte aligned.
 */
int dit_stream_probe(void* stream, int mode, const void* src, void* dst, size_t bytes, int workgroups,
                     float* sink);

/*
 * Calibration for measurements (not part of the block): the inner loop of the
 * block's GEMM kernel on LDS-resident operands.  `workgroups` workgroups of 8
 * waves (128 KB of LDS each, one per CU) run `ksteps` k-steps of the 256 x 256
 * x 64 fp16 tile: 128 v_mfma_f32_32x32x16_f16 per wave per k-step
 * (2 * 256 * 256 * 64 flop per workgroup), fragments read from two staged
 * tiles laid out and swizzled as the GEMM lays them out.  mode bit 0: the
 * ping-pong schedule (the two waves of a SIMD alternate fragment-read and MFMA
 * phases, a barrier per phase, MFMA phases at raised wave priority) instead of
 * the GEMM's interleaved one; bit 1: also load each k-step's 64 KB global ->
 * LDS from `window` (at least 4 MiB, 16-byte aligned, filled with the fp16
 * value 2^-6 = 0x2400 so the staged values stay 2^-6; read only; ignored
 * without bit 1).  Every staged element is 2^-6, so each thread writes
 * out[w * 512 + t] = 2 * ksteps (the sum of its 128 accumulators); out holds
 * workgroups * 512 floats.  Bit 2: the LDS tiles start as hashed fp16 values
 * of random sign and magnitude in [2^-6, 2^-2) instead (operands whose bits
 * switch as real data do; the device holds a lower clock on them), and out is
 * the sums they give.  Bit 3 (not with bit 1): the fragments are read once and
 * the k-steps run their MFMAs from registers, without LDS reads.
 */
int dit_gemm_kloop_probe(void* stream, int mode, int workgroups, int ksteps, const void* window, size_t window_bytes,
                         float* out);

/*
 * Calibration for measurements (not part of the block): the joint-attention
 * kernel's pipeline step on LDS-resident K and V.  `workgroups` workgroups of
 * 8 waves (32 queries each, 64 KB of LDS) run `tiles` 64-key tiles at head
 * dimension 128: per wave and tile 16 score MFMAs, 32 exponentials of
 * fma(s, c2, -1) with their sums and fp16 packing, a rarely taken branch and
 * 16 PV MFMAs (4 * 256 * 64 * 128 flop per workgroup and tile).  mode bit 0
 * clear: the kernel's order (next tile's scores beside this tile's softmax,
 * then PV, a barrier per tile); set: the two waves of a SIMD half a tile apart
 * (MFMA phase at raised priority, softmax phase), a barrier per phase.  Staged
 * values are 2^-6; with c2 = 0 every probability is 1/2 and each thread writes
 * out[w * 512 + t] = 48 * tiles (bit 0 clear) or 48 * tiles + 16 (set).  Bit
 * 1: K, V and Q start as hashed fp16 values of random sign and magnitude in
 * [2^-6, 2^-2) instead (see dit_gemm_kloop_probe).
 */
int dit_attention_step_probe(void* stream, int mode, int workgroups, int tiles, float c2, float* out);

/*
 * fp8 double-stream block: dit_block_forward with its four weight products
 * (QKV, out-projection, FFN-in, FFN-down) on e4m3 codes.  Before each product
 * the block quantises the product's activations per row by dit_quantize_fp8's
 * rule (a and b from their fp32 values, inside the modulation kernel; O and f
 * from their act_dtype values); the
 * weights come quantised per output row (w[j, :] = s[j] * dec(codes[j, :]), as
 * dit_quantize_fp8 writes them from the 16-bit weights).  The attention runs
 * as dit_joint_attention_fp8 on e4m3 q, k, v written by the QK-norm + RoPE
 * kernel: q per token and head by dit_quantize_fp8's rule, k per head with the
 * static scale max|w_k| * sqrt(128) / 448 (max over both streams' k-norm
 * weights: a normed, rotated element never exceeds sqrt(128) * max|w_k|), v
 * per head with s = max|v| / 448 over all tokens (the QKV epilogue raises the
 * maxima).  The AdaLN GEMV, the norms, RoPE and the epilogues (gated residual,
 * SwiGLU) are those of the 16-bit block, so the extra error is the e4m3
 * rounding of both operands of each product (up to 2^-4 relative per element)
 * and of the attention's probabilities.
 *  cfg       dtype DIT_BF16; act_dtype DIT_F16 or DIT_BF16
 *  txt, img  (host) fp8 weights of each stream (below); every pointer 16-byte
 *            aligned
 *  workspace >= dit_block_fp8_workspace_size(cfg) bytes (the 16-bit block's
 *            plus n * 3d attention code bytes, (n + 3) * n_heads fp32 words,
 *            n * max(d, F) product code bytes and n fp32 scales)
 * Other arguments, aliasing rules and errors as for dit_block_forward.
 * Launches (11): GEMV, modulate x (to e4m3), QKV, QK-norm + RoPE (to e4m3),
 * attention (e4m3), quantise O, out-projection, modulate h (to e4m3), FFN-in,
 * quantise f, FFN-down.
 */
typedef struct dit_stream_weights_fp8 {
    const void* w_mod;          /* [6d, d_cond] of dtype (shift1, scale1, gate1, shift2, scale2, gate2) */
    const void* qk_norm_w;      /* [2][head_dim] of dtype */
    const void* w_qkv;          /* [3d, d] e4m3 codes (row stride d) */
    const float* s_qkv;         /* [3d] per-row scales */
    const void* w_o;            /* [d, d] codes */
    const float* s_o;           /* [d] */
    const void* w_ffn_in;       /* [2F, d] codes: rows 0..F-1 gate, F..2F-1 up */
    const float* s_ffn_in;      /* [2F] */
    const void* w_ffn_out;      /* [d, F] codes (row stride F) */
    const float* s_ffn_out;     /* [d] */
} dit_stream_weights_fp8;

/* fp8 weights of a single-stream block: w_1 codes [3d + 2F, d] (rows q | k | v | gate | up) with
 * [3d + 2F] row scales, w_2 codes [d, d + F] with [d] row scales; w_mod and qk_norm_w of dtype. */
typedef struct dit_single_weights_fp8 {
    const void* w_mod;          /* [3d, d_cond] of dtype: shift, scale, gate */
    const void* qk_norm_w;      /* [2][head_dim] of dtype */
    const void* w_1;            /* [3d + 2F, d] e4m3 codes */
    const float* s_1;           /* [3d + 2F] */
    const void* w_2;            /* [d, d + F] e4m3 codes (row stride d + F) */
    const float* s_2;           /* [d] */
} dit_single_weights_fp8;

/* Workspace bytes of dit_single_block_forward_fp8; 0 for an invalid config. */
size_t dit_single_block_fp8_workspace_size(const dit_block_config* cfg);

/*
 * fp8 single-stream block: dit_single_block_forward with its two weight products on e4m3 codes:
 * a is quantised per row inside the modulation kernel, [O | f] per row (width d + F) by a
 * separate pass; W_1 and W_2 come quantised per output row.  Arguments, aliasing and errors as for
 * dit_single_block_forward; cfg as for dit_block_forward_fp8; the attention on e4m3 q, k, v as in
 * dit_block_forward_fp8 (k scale from the block's one k-norm weight).  Launches (8): GEMV,
 * modulate x (to e4m3), linear1 q|k|v, linear1 gate|up (SwiGLU), QK-norm + RoPE (to e4m3),
 * attention (e4m3), quantise [O | f], linear2.
 */
int dit_single_block_forward_fp8(const dit_block_config* cfg, const dit_single_weights_fp8* w,
                                 const void* cond, const int32_t* pos, const void* x, void* y,
                                 void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes of dit_block_forward_fp8; 0 for an invalid config. */
size_t dit_block_fp8_workspace_size(const dit_block_config* cfg);

int dit_block_forward_fp8(const dit_block_config* cfg,
                          const dit_stream_weights_fp8* txt, const dit_stream_weights_fp8* img,
                          const void* cond, const int32_t* pos,
                          const void* x_txt, const void* x_img, void* y_txt, void* y_img,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * 2-D convolution of the diffusion-VAE decoder (the pipeline's second stage,
 * whose convolutions the decoder page measures), as an implicit GEMM on MFMA:
 * no column buffer is built.
 *   y[b, h, w, co] = bias[co] + sum_{i, j, ci} x[b, h + i - kh/2, w + j - kw/2, ci]
 *                                              * weight[co, i, j, ci]
 * stride 1, zeros outside the image (the output has the input's size).
 *  dtype     of x and weight: DIT_BF16 (fp32 accumulation)
 *  x         [batch, height, width, c_in] (NHWC), contiguous
 *  weight    [c_out, kh, kw, c_in], contiguous;  bias fp32 [c_out] or NULL
 *  y         [batch, height, width, c_out] of y_dtype (DIT_BF16 or DIT_F32);
 *            must not overlap x, weight or bias
 * Limits: c_in a multiple of 8 (a multiple of 64 wastes no matrix work), c_out >= 1
 * (a multiple of 4 stores four channels at a time), kh and kw odd <= 7.  One launch.
 */
int dit_conv2d(int dtype, void* stream, const void* x, int batch, int height, int width,
               int c_in, const void* weight, int c_out, int kh, int kw, const float* bias,
               void* y, int y_dtype);

/*
 * Causal 3-D convolution over video frames (the layers of a video VAE's decoder, whose
 * convolutions the decoder page measures per latent frame), as the same implicit GEMM:
 *   y[b, t, h, w, co] = bias[co] + sum_{s, i, j, ci} x[b, t + s - (kt-1), h + i - kh/2, w + j - kw/2, ci]
 *                                                    * weight[co, s, i, j, ci]
 * zeros before the first frame of each clip and outside the image, so output frame t depends on
 * frames t-kt+1 .. t only; stride 1, output the input's size.
 *  x         [batch, frames, height, width, c_in] (channels last), contiguous
 *  weight    [c_out, kt, kh, kw, c_in], contiguous;  bias fp32 [c_out] or NULL
 *  y         [batch, frames, height, width, c_out] of y_dtype; must not overlap the inputs
 * Limits as for dit_conv2d, kt from 1 to 7 (kt = frames = 1 is dit_conv2d).  One launch.
 */
int dit_conv3d_causal(int dtype, void* stream, const void* x, int batch, int frames, int height,
                      int width, int c_in, const void* weight, int c_out, int kt, int kh, int kw,
                      const float* bias, void* y, int y_dtype);

/*
 * Weight format conversion: dst[i] = fp16(src[i]) for n bf16 values (exact for
 * |x| >= 2^-14 and zero; smaller magnitudes round to nearest even among fp16
 * subnormals, as the GEMMs' own staging conversion does).  src and dst 16-byte
 * aligned, not overlapping.  One launch on stream.  For gemm_w_dtype = DIT_F16.
 */
int dit_convert_bf16_to_f16(void* stream, const void* src, void* dst, size_t n);

/* Thread-local text of the last error of this thread (never NULL). */
const char* dit_last_error(void);

/* Thread-local count of kernels this thread has launched successfully (a test
 * hook: a parity test checks that the GPU path really ran). */
uint64_t dit_launch_count(void);

/* DIT_ABI_VERSION of the built library. */
int dit_abi_version(void);

/*
 * Range flags of the last block / step call that used `workspace` (the word at
 * its first 4 bytes): waits for the work queued on `stream`, then copies the
 * word to *flags (host).  The one call of the library that synchronises.
 *   DIT_RANGE_F16: an fp32 result rounded to an fp16 activation (a, qkv, b, f,
 *   and the fp8 blocks' fp16 products; act_dtype DIT_F16) was NaN or larger than
 *   65504 in magnitude, so it became inf or NaN.  q and k after QK-norm + RoPE
 *   are not checked: each is a unit-RMS 128-vector times the QK-norm weight, so
 *   its magnitude is at most sqrt(128) max|w_qk|, and they stay finite for QK-norm
 *   weights below 5792 in magnitude (a precondition of DIT_F16 activations).
 *   Attention's output is a convex combination of v rows and cannot leave the
 *   range either.  fp16 activations keep bf16 models' block outputs closer to
 *   exact arithmetic but have a narrower range than bf16; a model whose
 *   activations leave it needs act_dtype DIT_BF16.
 * Reentrant; returns DIT_ERR_HIP if the copy or the wait fails.
 */
#define DIT_RANGE_F16 1u
int dit_workspace_flags(const void* workspace, void* stream, uint32_t* flags);

/*
 * Test hook of the split-work hand-over.  When a launch splits its last round of
 * work units over a persistent grid of one workgroup per compute unit (the GEMMs'
 * k-steps, attention's key tiles), the workgroup owning a unit adds the partial
 * results the other workgroups publish for their pieces of it.  It polls a
 * piece's flag at most `polls` times; then it computes that piece itself (the
 * result equals the split one up to the summation order), so no piece is ever
 * dropped, whether or not every workgroup of the grid is resident.  Default
 * 2^22 polls (a value < 0 restores it).  0 turns the hand-over off: no
 * partial is published and every owner computes all the pieces of its unit
 * itself (for tests of that path).  Thread-local: applies to the calling
 * thread's later calls.
 */
void dit_set_split_wait_limit(int polls);

/*
 * Kernel timing for measurement tools.  dit_timing_begin(capacity) makes the
 * calling thread bracket each of its next `capacity` launches with a pair of
 * HIP events recorded on the launch stream (the events are created here, not
 * per launch).  dit_timing_end() stops recording.  dit_timing_read(i, ...)
 * waits for the recorded events and reports, for the i-th distinct kernel
 * seen, its name, its number of launches and the sum of their durations in
 * milliseconds; it returns the number of distinct kernels, or -1 on error.
 * name_buf (host) receives a NUL-terminated name of at most name_len bytes.
 */
int dit_timing_begin(int capacity);
int dit_timing_end(void);
int dit_timing_read(int i, char* name_buf, int name_len, int* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* DIT_H */
