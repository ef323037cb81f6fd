// C ABI of the DiT block library (declared in include/dit.h): argument validation on the host,
// workspace planning and the launch sequence of each entry point.  Validation happens before
// any HIP call, so an invalid call launches nothing and needs no GPU.  The pattern of a flat C
// ABI that carries device pointers and shapes and re-validates them at the boundary follows the
// fak GPU backend page ("GPU -- the in-kernel forward pass, on the GPU", section 2).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/dit.h"
#include "launch.h"

using namespace dit;

namespace {

// ---- thread-local state -----------------------------------------------------------------
struct TimingState {
    bool on = false;
    int capacity = 0, used = 0;
    std::vector<hipEvent_t> ev;         // 2 per slot
    std::vector<const char*> name;
};
thread_local char tl_err[512] = "";
thread_local uint64_t tl_launches = 0;
thread_local TimingState tl_timing;

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(tl_err, sizeof(tl_err), fmt, ap);
    va_end(ap);
    return code;
}
void clear_err() { tl_err[0] = 0; }

template <typename F>
int launch(const char* name, hipStream_t s, F&& fn) {
    TimingState& T = tl_timing;
    const bool timed = T.on && T.used < T.capacity;
    if (timed && hipEventRecord(T.ev[2 * T.used], s) != hipSuccess)
        return fail(DIT_ERR_HIP, "hipEventRecord failed before %s", name);
    const hipError_t e = fn();
    if (e != hipSuccess) return fail(DIT_ERR_HIP, "launch of %s failed: %s", name, hipGetErrorString(e));
    if (timed) {
        if (hipEventRecord(T.ev[2 * T.used + 1], s) != hipSuccess)
            return fail(DIT_ERR_HIP, "hipEventRecord failed after %s", name);
        T.name[T.used++] = name;
    }
    ++tl_launches;
    return DIT_OK;
}
#define DIT_TRY(x)                     \
    do {                               \
        const int _rc = (x);           \
        if (_rc != DIT_OK) return _rc; \
    } while (0)

// ---- validation helpers ------------------------------------------------------------------------
size_t esize(int dt) { return dt == DIT_F32 ? 4 : 2; }
bool valid_dtype(int dt) { return dt == DIT_BF16 || dt == DIT_F32 || dt == DIT_F16; }
bool valid_wdtype(int dt) { return dt == DIT_BF16 || dt == DIT_F32; }   // weights, cond, x
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptr(const void* p, const char* what) {
    if (!p) return fail(DIT_ERR_INVALID_ARG, "%s is NULL", what);
    if (!aligned16(p)) return fail(DIT_ERR_INVALID_ARG, "%s is not 16-byte aligned", what);
    return DIT_OK;
}
int check_ld(long ld, long width, int dt, const char* what) {
    if (ld < width) return fail(DIT_ERR_INVALID_ARG, "%s = %ld is smaller than the row width %ld", what, ld, width);
    if ((ld * (long)esize(dt)) % 16 != 0)
        return fail(DIT_ERR_INVALID_ARG, "%s = %ld: row stride is not a multiple of 16 bytes", what, ld);
    return DIT_OK;
}
// Byte range [lo, hi) of a strided matrix.
struct Range { uintptr_t lo, hi; };
Range range_of(const void* p, long rows, long ld, long width, int dt) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    if (rows <= 0) return {lo, lo};
    return {lo, lo + (uintptr_t)(((rows - 1) * ld + width) * (long)esize(dt))};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

int build_rope_table(int head_dim, int n_axes, const int* axes_dim, float theta, RopeTable& t) {
    if (!axes_dim) return fail(DIT_ERR_INVALID_ARG, "axes_dim is NULL");
    if (n_axes < 1 || n_axes > 4) return fail(DIT_ERR_UNSUPPORTED, "n_axes = %d (1..4 supported)", n_axes);
    if (!(theta > 0.0f) || !std::isfinite(theta)) return fail(DIT_ERR_INVALID_ARG, "theta must be positive");
    int sum = 0, p = 0;
    for (int a = 0; a < n_axes; ++a) {
        const int dim = axes_dim[a];
        if (dim <= 0 || dim % 2) return fail(DIT_ERR_INVALID_ARG, "axes_dim[%d] = %d must be even and positive", a, dim);
        sum += dim;
        if (sum > head_dim) break;
        for (int j = 0; j < dim / 2; ++j, ++p) {
            const double om = std::pow((double)theta, -2.0 * j / dim);
            t.omega_d[p] = om;
            t.axis[p] = (int8_t)a;
        }
    }
    if (sum != head_dim) return fail(DIT_ERR_INVALID_ARG, "axes_dim sum to %d, head_dim is %d", sum, head_dim);
    return DIT_OK;
}

int validate_config(const dit_block_config* c) {
    if (!c) return fail(DIT_ERR_INVALID_ARG, "cfg is NULL");
    if (!valid_wdtype(c->dtype) || !valid_wdtype(c->x_dtype) || !valid_wdtype(c->y_dtype) ||
        !valid_dtype(c->act_dtype))
        return fail(DIT_ERR_INVALID_ARG, "dtype / x_dtype / y_dtype must be DIT_F32 or DIT_BF16, act_dtype one of "
                                         "DIT_F32, DIT_BF16, DIT_F16");
    if (c->dtype == DIT_F32 && (c->x_dtype != DIT_F32 || c->y_dtype != DIT_F32 || c->act_dtype != DIT_F32))
        return fail(DIT_ERR_UNSUPPORTED, "an fp32 block needs fp32 activations, x and y");
    if (c->dtype == DIT_BF16 && c->act_dtype == DIT_F32)
        return fail(DIT_ERR_UNSUPPORTED, "bf16 weights need DIT_F16 or DIT_BF16 activations");
    if (c->gemm_w_dtype != 0 && c->gemm_w_dtype != c->dtype &&
        !(c->gemm_w_dtype == DIT_F16 && c->dtype == DIT_BF16 && c->act_dtype == DIT_F16))
        return fail(DIT_ERR_UNSUPPORTED, "gemm_w_dtype must be 0, dtype, or DIT_F16 for a bf16 block with DIT_F16 "
                                         "activations");
    if (c->head_dim != 128) return fail(DIT_ERR_UNSUPPORTED, "head_dim = %d (only 128 is supported)", c->head_dim);
    if (c->n_heads < 1 || c->d != c->n_heads * c->head_dim)
        return fail(DIT_ERR_INVALID_ARG, "d = %d must equal n_heads * head_dim = %d * %d", c->d, c->n_heads, c->head_dim);
    if (c->d > 8192) return fail(DIT_ERR_UNSUPPORTED, "d = %d (at most 8192)", c->d);
    if (c->ffn_inner < 128 || c->ffn_inner % 128)
        return fail(DIT_ERR_INVALID_ARG, "ffn_inner = %d must be a positive multiple of 128", c->ffn_inner);
    if (c->ffn_inner > (1 << 20)) return fail(DIT_ERR_UNSUPPORTED, "ffn_inner = %d (at most 2^20)", c->ffn_inner);
    if (c->d_cond < 8 || c->d_cond % 8 || c->d_cond > 16384)
        return fail(DIT_ERR_INVALID_ARG, "d_cond = %d must be a multiple of 8 in [8, 16384]", c->d_cond);
    if (c->n_txt < 0 || c->n_img < 0 || c->n_txt + c->n_img < 1)
        return fail(DIT_ERR_INVALID_ARG, "n_txt = %d, n_img = %d: need n_txt, n_img >= 0 and at least one token",
                    c->n_txt, c->n_img);
    if (!(c->eps >= 0.0f) || !(c->eps_qk >= 0.0f)) return fail(DIT_ERR_INVALID_ARG, "eps must be >= 0");
    RopeTable t;
    return build_rope_table(c->head_dim, c->n_axes, c->axes_dim, c->theta, t);
}

// Workspace plan: 256-byte aligned sub-buffers.
struct WsPlan {
    size_t flags, mod, act, qkv, o, h, f, of, cs, cs_bytes, sk, sk_bytes, ask, ask_bytes, a8, a8s, q8, sq, total;
};
size_t up256(size_t x) { return (x + 255) & ~size_t(255); }
WsPlan plan_workspace(const dit_block_config* c, int single, bool fp8 = false) {
    const size_t n = (size_t)c->n_txt + c->n_img, d = c->d, F = c->ffn_inner, es = esize(c->act_dtype);
    WsPlan p{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += up256(bytes); return o; };
    p.flags = take(4);          // the call's range-flag word, first in every plan (offset 0)
    if (!single) {
        p.mod = take(2 * 6 * d * 4);
        p.act = take(n * d * es);
        p.qkv = take(n * 3 * d * es);
        p.o = take(n * d * es);
        p.h = take(n * d * 4);
        p.f = take(n * F * es);
        // the rotation angles' (cos, sin) per token for the QKV product's fused QK RMSNorm + RoPE
        // (16-bit path, every 256-column tile two whole heads)
        p.cs_bytes = !fp8 && c->dtype == DIT_BF16 && d % 256 == 0 ? n * 64 * 2 * 4 : 0;
        p.cs = take(p.cs_bytes);
    } else {
        p.mod = take(3 * d * 4);
        p.act = take(n * d * es);
        p.qkv = take(n * 3 * d * es);
        p.of = take(n * (d + F) * es);
    }
    // the GEMMs' stream-K scratch (16-bit paths), shared by the block's GEMMs in stream order
    p.sk_bytes = c->dtype == DIT_BF16 ? gemm_sk_scratch_bytes() : 0;
    p.sk = take(p.sk_bytes);
    // attention's stream-K scratch (16-bit paths)
    p.ask_bytes = c->dtype == DIT_BF16 ? attention_sk_scratch_bytes() : 0;
    p.ask = take(p.ask_bytes);
    // fp8: the attention's e4m3 operands [n, 3d] (q | k | v codes) and their scales (q per token
    // and head, k and v per head) with the per-head |v| maxima; then the codes and per-row scales
    // of the current product's activations
    if (fp8) {
        const size_t H = c->n_heads;
        p.a8 = take(n * 3 * d);
        p.a8s = take((n * H + 3 * H) * 4);
        p.q8 = take(n * (single ? d + F : std::max(d, F)));
        p.sq = take(n * 4);
    }
    p.total = off;
    return p;
}

}  // namespace

// =========================================================================================
extern "C" {

const char* dit_last_error(void) { return tl_err; }
uint64_t dit_launch_count(void) { return tl_launches; }

void dit_set_split_wait_limit(int polls) { set_sk_spin_limit(polls); }

int dit_workspace_flags(const void* workspace, void* stream, uint32_t* flags) {
    clear_err();
    if (!flags) return fail(DIT_ERR_INVALID_ARG, "flags is NULL");
    DIT_TRY(check_ptr(workspace, "workspace"));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint32_t v = 0;
    hipError_t e = hipMemcpyAsync(&v, workspace, sizeof v, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(DIT_ERR_HIP, "reading the flag word failed: %s", hipGetErrorString(e));
    *flags = v;
    return DIT_OK;
}
int dit_abi_version(void) { return DIT_ABI_VERSION; }

int dit_adaln_modulate(int dtype, void* stream, const void* cond, int d_cond, const void* w_mod, int n_chunks,
                       int d, float* mod_out, const void* x, int x_dtype, int n_tok, long ld_x, int shift_chunk,
                       int scale_chunk, float eps, void* x_out, int out_dtype, long ld_out) {
    clear_err();
    if (!valid_wdtype(dtype)) return fail(DIT_ERR_INVALID_ARG, "dtype %d (DIT_BF16 or DIT_F32)", dtype);
    DIT_TRY(check_ptr(cond, "cond"));
    DIT_TRY(check_ptr(w_mod, "w_mod"));
    DIT_TRY(check_ptr(mod_out, "mod_out"));
    if (d < 8 || d % 8 || d > 8192) return fail(DIT_ERR_INVALID_ARG, "d = %d must be a multiple of 8 in [8, 8192]", d);
    if (d_cond < 8 || d_cond % 8 || d_cond > 16384)
        return fail(DIT_ERR_INVALID_ARG, "d_cond = %d must be a multiple of 8 in [8, 16384]", d_cond);
    if (n_chunks < 1) return fail(DIT_ERR_INVALID_ARG, "n_chunks = %d", n_chunks);
    if ((long)n_chunks * d > (1L << 30)) return fail(DIT_ERR_UNSUPPORTED, "n_chunks * d too large");
    if (x) {
        if (!valid_wdtype(x_dtype)) return fail(DIT_ERR_INVALID_ARG, "x_dtype %d (DIT_BF16 or DIT_F32)", x_dtype);
        if (!valid_dtype(out_dtype)) return fail(DIT_ERR_INVALID_ARG, "out_dtype %d", out_dtype);
        if (dtype == DIT_F32 && (x_dtype != DIT_F32 || out_dtype != DIT_F32))
            return fail(DIT_ERR_UNSUPPORTED, "an fp32 call needs fp32 x and x_out");
        if (n_tok < 0) return fail(DIT_ERR_INVALID_ARG, "n_tok = %d", n_tok);
        if (shift_chunk < 0 || shift_chunk >= n_chunks || scale_chunk < 0 || scale_chunk >= n_chunks)
            return fail(DIT_ERR_INVALID_ARG, "shift_chunk / scale_chunk out of [0, n_chunks)");
        if (!(eps >= 0.0f)) return fail(DIT_ERR_INVALID_ARG, "eps must be >= 0");
        DIT_TRY(check_ptr(x, "x"));
        DIT_TRY(check_ptr(x_out, "x_out"));
        DIT_TRY(check_ld(ld_x, d, x_dtype, "ld_x"));
        DIT_TRY(check_ld(ld_out, d, out_dtype, "ld_out"));
        if (overlap(range_of(x, n_tok, ld_x, d, x_dtype), range_of(x_out, n_tok, ld_out, d, out_dtype)))
            return fail(DIT_ERR_INVALID_ARG, "x_out overlaps x");
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    GemvBatch g{};
    g.p[0] = {w_mod, mod_out, n_chunks * d};
    g.n = 1;
    g.cond = cond;
    g.d_cond = d_cond;
    g.dtype = dtype;
    DIT_TRY(launch("adaln_gemv", s, [&] { return launch_adaln_gemv(g, s); }));
    if (x && n_tok > 0) {
        ModBatch m{};
        m.p[0] = {x, ld_x, x_dtype, x_out, ld_out, mod_out + (size_t)shift_chunk * d,
                  mod_out + (size_t)scale_chunk * d, n_tok};
        m.n = 1;
        m.d = d;
        m.eps = eps;
        m.out_dtype = out_dtype;
        DIT_TRY(launch("modulate", s, [&] { return launch_modulate(m, s); }));
    }
    return DIT_OK;
}

int dit_qk_rmsnorm_rope(int dtype, void* stream, void* q, long ld_q, void* k, long ld_k, int n_tok, int n_heads,
                        int head_dim, const void* qk_w, int w_dtype, int n_first, float eps, const int32_t* pos,
                        int n_axes, const int* axes_dim, float theta) {
    clear_err();
    if (!valid_dtype(dtype)) return fail(DIT_ERR_INVALID_ARG, "dtype %d", dtype);
    if (!valid_dtype(w_dtype)) return fail(DIT_ERR_INVALID_ARG, "w_dtype %d", w_dtype);
    if (head_dim != 128) return fail(DIT_ERR_UNSUPPORTED, "head_dim = %d (only 128 is supported)", head_dim);
    if (n_heads < 1) return fail(DIT_ERR_INVALID_ARG, "n_heads = %d", n_heads);
    if (n_tok < 0) return fail(DIT_ERR_INVALID_ARG, "n_tok = %d", n_tok);
    if (!(eps >= 0.0f)) return fail(DIT_ERR_INVALID_ARG, "eps must be >= 0");
    QkRopeArgs a{};
    DIT_TRY(build_rope_table(head_dim, n_axes, axes_dim, theta, a.tab));
    if (n_tok == 0) return DIT_OK;          // nothing is read or written
    DIT_TRY(check_ptr(q, "q"));
    DIT_TRY(check_ptr(k, "k"));
    DIT_TRY(check_ptr(qk_w, "qk_w"));
    DIT_TRY(check_ptr(pos, "pos"));
    const long width = (long)n_heads * head_dim;
    DIT_TRY(check_ld(ld_q, width, dtype, "ld_q"));
    DIT_TRY(check_ld(ld_k, width, dtype, "ld_k"));
    if (overlap(range_of(q, n_tok, ld_q, width, dtype), range_of(k, n_tok, ld_k, width, dtype))) {
        // q and k may be column views of one buffer: they must not share an element.
        const uintptr_t qa = reinterpret_cast<uintptr_t>(q), ka = reinterpret_cast<uintptr_t>(k);
        const uintptr_t dist = qa > ka ? qa - ka : ka - qa;
        if (ld_q != ld_k || dist < (uintptr_t)width * esize(dtype) ||
            dist + (uintptr_t)width * esize(dtype) > (uintptr_t)ld_q * esize(dtype))
            return fail(DIT_ERR_INVALID_ARG, "q and k overlap");
    }
    if (n_tok == 0) return DIT_OK;
    a.q = q; a.ld_q = ld_q; a.k = k; a.ld_k = ld_k;
    a.n_tok = n_tok; a.n_heads = n_heads; a.n_first = n_first; a.eps = eps;
    a.qk_w0 = qk_w;
    a.qk_w1 = reinterpret_cast<const char*>(qk_w) + (n_first < n_tok ? 2 * (size_t)head_dim * esize(w_dtype) : 0);
    a.w_dtype = w_dtype;
    a.pos = pos; a.n_axes = n_axes; a.dtype = dtype;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch("qk_rmsnorm_rope", s, [&] { return launch_qk_rmsnorm_rope(a, s); });
}

int dit_joint_attention(int dtype, void* stream, const void* q, long ld_q, const void* k, long ld_k, const void* v,
                        long ld_v, void* o, long ld_o, int n_tok, int n_heads, int head_dim, float softmax_scale) {
    clear_err();
    if (!valid_dtype(dtype)) return fail(DIT_ERR_INVALID_ARG, "dtype %d", dtype);
    if (head_dim != 128) return fail(DIT_ERR_UNSUPPORTED, "head_dim = %d (only 128 is supported)", head_dim);
    if (n_heads < 1) return fail(DIT_ERR_INVALID_ARG, "n_heads = %d", n_heads);
    if (n_tok < 0) return fail(DIT_ERR_INVALID_ARG, "n_tok = %d", n_tok);
    if (!std::isfinite(softmax_scale)) return fail(DIT_ERR_INVALID_ARG, "softmax_scale is not finite");
    if (n_tok == 0) return DIT_OK;          // nothing is read or written
    DIT_TRY(check_ptr(q, "q"));
    DIT_TRY(check_ptr(k, "k"));
    DIT_TRY(check_ptr(v, "v"));
    DIT_TRY(check_ptr(o, "o"));
    const long width = (long)n_heads * head_dim;
    DIT_TRY(check_ld(ld_q, width, dtype, "ld_q"));
    DIT_TRY(check_ld(ld_k, width, dtype, "ld_k"));
    DIT_TRY(check_ld(ld_v, width, dtype, "ld_v"));
    DIT_TRY(check_ld(ld_o, width, dtype, "ld_o"));
    const Range ro = range_of(o, n_tok, ld_o, width, dtype);
    if (overlap(ro, range_of(q, n_tok, ld_q, width, dtype)) || overlap(ro, range_of(k, n_tok, ld_k, width, dtype)) ||
        overlap(ro, range_of(v, n_tok, ld_v, width, dtype)))
        return fail(DIT_ERR_INVALID_ARG, "o overlaps q, k or v");
    if ((long)n_tok * n_heads > (1L << 30)) return fail(DIT_ERR_UNSUPPORTED, "n_tok * n_heads too large");
    if (n_tok == 0) return DIT_OK;
    AttnArgs a{q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_tok, n_heads, softmax_scale, dtype};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch("joint_attention", s, [&] { return launch_attention(a, s); });
}

size_t dit_block_workspace_size(const dit_block_config* cfg, int single_stream) {
    clear_err();
    if (validate_config(cfg) != DIT_OK) return 0;
    return plan_workspace(cfg, single_stream ? 1 : 0).total;
}

// need_mod = false: w_mod is not used (the shared-modulation step) and may be NULL
static int check_stream_weights(const dit_stream_weights* w, const char* s, bool need_mod = true) {
    if (!w) return fail(DIT_ERR_INVALID_ARG, "%s weights are NULL", s);
    const void* p[6] = {w->w_mod, w->w_qkv, w->qk_norm_w, w->w_o, w->w_ffn_in, w->w_ffn_out};
    const char* n[6] = {"w_mod", "w_qkv", "qk_norm_w", "w_o", "w_ffn_in", "w_ffn_out"};
    for (int i = need_mod ? 0 : 1; i < 6; ++i) {
        if (!p[i]) return fail(DIT_ERR_INVALID_ARG, "%s.%s is NULL", s, n[i]);
        if (!aligned16(p[i])) return fail(DIT_ERR_INVALID_ARG, "%s.%s is not 16-byte aligned", s, n[i]);
    }
    return DIT_OK;
}

static int check_stream_weights_fp8(const dit_stream_weights_fp8* w, const char* s) {
    if (!w) return fail(DIT_ERR_INVALID_ARG, "%s weights are NULL", s);
    const void* p[10] = {w->w_mod, w->qk_norm_w, w->w_qkv, w->s_qkv, w->w_o, w->s_o, w->w_ffn_in, w->s_ffn_in,
                         w->w_ffn_out, w->s_ffn_out};
    const char* n[10] = {"w_mod", "qk_norm_w", "w_qkv", "s_qkv", "w_o", "s_o", "w_ffn_in", "s_ffn_in", "w_ffn_out",
                         "s_ffn_out"};
    for (int i = 0; i < 10; ++i) {
        if (!p[i]) return fail(DIT_ERR_INVALID_ARG, "%s.%s is NULL", s, n[i]);
        if (!aligned16(p[i])) return fail(DIT_ERR_INVALID_ARG, "%s.%s is not 16-byte aligned", s, n[i]);
    }
    return DIT_OK;
}

static int validate_fp8_config(const dit_block_config* c) {
    DIT_TRY(validate_config(c));
    if (c->dtype != DIT_BF16 || (c->act_dtype != DIT_F16 && c->act_dtype != DIT_BF16))
        return fail(DIT_ERR_UNSUPPORTED, "the fp8 block needs dtype DIT_BF16 and DIT_F16 or DIT_BF16 activations");
    return DIT_OK;
}

// mod_pre: the [2][6d] fp32 AdaLN vectors (text, image) computed by the caller, or NULL (the block
// computes them from its own w_mod; cond is then required).  t8 / i8: fp8 weights (the four
// products run on e4m3 codes; txt / img are then NULL).
static int block_forward_impl(const dit_block_config* cfg, const dit_stream_weights* txt,
                              const dit_stream_weights* img, const void* cond, const int32_t* pos, const void* x_txt,
                              const void* x_img, void* y_txt, void* y_img, void* workspace, size_t ws_bytes,
                              void* stream, const float* mod_pre, const dit_stream_weights_fp8* t8 = nullptr,
                              const dit_stream_weights_fp8* i8 = nullptr, bool clear_flags = true) {
    clear_err();
    const bool fp8 = t8 != nullptr;
    DIT_TRY(fp8 ? validate_fp8_config(cfg) : validate_config(cfg));
    const dit_block_config& c = *cfg;
    const int nt = c.n_txt, ni = c.n_img, n = nt + ni, d = c.d, F = c.ffn_inner;
    if (fp8) {
        DIT_TRY(check_stream_weights_fp8(t8, "txt"));
        DIT_TRY(check_stream_weights_fp8(i8, "img"));
    } else {
        DIT_TRY(check_stream_weights(txt, "txt", !mod_pre));
        DIT_TRY(check_stream_weights(img, "img", !mod_pre));
    }
    const void* wmod_t = fp8 ? t8->w_mod : txt->w_mod;
    const void* wmod_i = fp8 ? i8->w_mod : img->w_mod;
    const void* qkw_t = fp8 ? t8->qk_norm_w : txt->qk_norm_w;
    const void* qkw_i = fp8 ? i8->qk_norm_w : img->qk_norm_w;
    if (!mod_pre) DIT_TRY(check_ptr(cond, "cond"));
    DIT_TRY(check_ptr(pos, "pos"));
    if (nt > 0) { DIT_TRY(check_ptr(x_txt, "x_txt")); DIT_TRY(check_ptr(y_txt, "y_txt")); }
    if (ni > 0) { DIT_TRY(check_ptr(x_img, "x_img")); DIT_TRY(check_ptr(y_img, "y_img")); }
    DIT_TRY(check_ptr(workspace, "workspace"));
    const WsPlan W = plan_workspace(cfg, 0, fp8);
    if (ws_bytes < W.total)
        return fail(DIT_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, W.total);
    // y may alias x (same dtype); otherwise no overlap; nothing may overlap the workspace.
    const Range rws{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + W.total};
    const Range rxt = range_of(x_txt, nt, d, d, c.x_dtype), rxi = range_of(x_img, ni, d, d, c.x_dtype);
    const Range ryt = range_of(y_txt, nt, d, d, c.y_dtype), ryi = range_of(y_img, ni, d, d, c.y_dtype);
    if (overlap(rws, rxt) || overlap(rws, rxi) || overlap(rws, ryt) || overlap(rws, ryi))
        return fail(DIT_ERR_INVALID_ARG, "workspace overlaps an input or output");
    if (overlap(ryt, ryi)) return fail(DIT_ERR_INVALID_ARG, "y_txt overlaps y_img");
    const bool same = c.x_dtype == c.y_dtype;
    if ((overlap(ryt, rxt) && !(same && ryt.lo == rxt.lo)) || (overlap(ryi, rxi) && !(same && ryi.lo == rxi.lo)) ||
        overlap(ryt, rxi) || overlap(ryi, rxt))
        return fail(DIT_ERR_INVALID_ARG, "y overlaps x other than as an exact alias of the same dtype");

    char* ws = reinterpret_cast<char*>(workspace);
    float* mod_t = mod_pre ? const_cast<float*>(mod_pre) : reinterpret_cast<float*>(ws + W.mod);
    float* mod_i = mod_t + 6 * (size_t)d;
    char* act = ws + W.act;
    char* qkv = ws + W.qkv;
    char* ob = ws + W.o;
    float* h = reinterpret_cast<float*>(ws + W.h);
    char* f = ws + W.f;
    unsigned* flag = reinterpret_cast<unsigned*>(ws + W.flags);
    const size_t es = esize(c.act_dtype);     // activation element size
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    // 1. AdaLN vectors of both streams (this first kernel also resets the range-flag word)
    if (!mod_pre) {
        GemvBatch g{};
        g.p[0] = {wmod_t, mod_t, 6 * d};
        g.p[1] = {wmod_i, mod_i, 6 * d};
        g.n = 2;
        g.cond = cond;
        g.d_cond = c.d_cond;
        g.dtype = c.dtype;
        g.clear_flag = clear_flags ? flag : nullptr;
        DIT_TRY(launch("adaln_gemv", s, [&] { return launch_adaln_gemv(g, s); }));
    }

    // 2. a = (1 + scale1) RMSNorm(x) + shift1   (text rows, then image rows)
    ModBatch m{};
    int nm = 0;
    if (nt) m.p[nm++] = {x_txt, d, c.x_dtype, act, d, mod_t + 0 * d, mod_t + 1 * (size_t)d, nt};
    if (ni) m.p[nm++] = {x_img, d, c.x_dtype, act + (size_t)nt * d * es, d, mod_i + 0 * d, mod_i + 1 * (size_t)d, ni};
    m.n = nm; m.d = d; m.eps = c.eps; m.out_dtype = c.act_dtype; m.range_flag = flag;
    // 16-bit path with whole heads per 256-column tile: QK RMSNorm + RoPE in the QKV product's
    // epilogue, from a table of the angles' (cos, sin) that this modulation writes as well
    const bool fuse_rope = !fp8 && W.cs_bytes > 0;
    float* rope_cs = fuse_rope ? reinterpret_cast<float*>(ws + W.cs) : nullptr;
    if (fuse_rope) {
        DIT_TRY(build_rope_table(c.head_dim, c.n_axes, c.axes_dim, c.theta, m.rope_tab));
        m.rope_cs = rope_cs; m.rope_pos = pos; m.rope_n = n; m.rope_n_axes = c.n_axes;
    }
    // fp8 products: a goes straight to e4m3 codes with per-row scales
    uint8_t* q8 = fp8 ? reinterpret_cast<uint8_t*>(ws + W.q8) : nullptr;
    float* sq = fp8 ? reinterpret_cast<float*>(ws + W.sq) : nullptr;
    // fp8 attention operands: codes, scales, and the per-head |v| maxima (zeroed by the modulation)
    uint8_t* a8 = fp8 ? reinterpret_cast<uint8_t*>(ws + W.a8) : nullptr;
    float* a8_sq = fp8 ? reinterpret_cast<float*>(ws + W.a8s) : nullptr;
    float* a8_sk = fp8 ? a8_sq + (size_t)n * c.n_heads : nullptr;
    float* a8_sv = fp8 ? a8_sk + c.n_heads : nullptr;
    unsigned* a8_vmax = fp8 ? reinterpret_cast<unsigned*>(a8_sv + c.n_heads) : nullptr;
    auto to_fp8 = [&](ModBatch& mb) {
        int r0 = 0;
        for (int i = 0; i < mb.n; ++i) {
            mb.p[i].out = q8 + (size_t)r0 * d;
            mb.p[i].out_scale = sq + r0;
            r0 += mb.p[i].rows;
        }
        mb.out_dtype = FP8_ROWS;
    };
    if (fp8) {
        to_fp8(m);
        m.clear = a8_vmax; m.clear_n = c.n_heads;
    }
    DIT_TRY(launch(fp8 ? "modulate_x_fp8" : "modulate_x", s, [&] { return launch_modulate(m, s); }));

    // fp8 products: quantise the activations [n, k] (row stride k) per row (a and b come quantised
    // from the modulate kernel), then one grouped e4m3 GEMM over the text rows and the image rows.
    auto quantize = [&](const char* name, const void* src, int k) {
        return launch(name, s, [&] { return launch_quantize_fp8(src, c.act_dtype, k, n, k, q8, k, sq, s); });
    };
    // problem of `rows` rows starting at row r0 of the quantised activations (row stride k)
    auto fp8_problem = [&](int r0, int rows, int k, const void* wq, const float* sw, void* out, long ldc, int c_dtype,
                           int N, int epi) {
        Fp8GemmProblem P{};
        P.a = q8 + (size_t)r0 * k; P.lda = k; P.sa = sq + r0;
        P.b = reinterpret_cast<const uint8_t*>(wq); P.ldb = k; P.sb = sw;
        P.c = out; P.ldc = ldc; P.c_dtype = c_dtype;
        P.M = rows; P.N = N; P.K = k; P.epi = epi;
        return P;
    };

    // 3. qkv = a W_qkv^T (with QK RMSNorm + RoPE in its epilogue when fuse_rope)
    if (fp8) {
        Fp8GemmBatch b{};
        if (nt) b.p[b.n++] = fp8_problem(0, nt, d, t8->w_qkv, t8->s_qkv, qkv, 3L * d, c.act_dtype, 3 * d, EPI_STORE);
        if (ni) b.p[b.n++] = fp8_problem(nt, ni, d, i8->w_qkv, i8->s_qkv, qkv + (size_t)nt * 3 * d * es, 3L * d,
                                         c.act_dtype, 3 * d, EPI_STORE);
        b.range_flag = flag;
        b.vmax = a8_vmax; b.vmax_col0 = 2 * d;
        DIT_TRY(launch("gemm_fp8_qkv", s, [&] { return launch_gemm_fp8(b, s); }));
    } else {
    GemmBatch gq{};
    gq.range_flag = flag;
    gq.sk_scratch = W.sk_bytes ? ws + W.sk : nullptr;
    gq.a_dtype = c.act_dtype;
    gq.b_f16 = c.gemm_w_dtype == DIT_F16;
    {
        int k = 0;
        if (nt) gq.p[k++] = {act, d, txt->w_qkv, d, qkv, 3L * d, c.act_dtype, nullptr, 0, 0, nullptr, 0, nt, 3 * d, d, EPI_STORE};
        if (ni) gq.p[k++] = {act + (size_t)nt * d * es, d, img->w_qkv, d, qkv + (size_t)nt * 3 * d * es, 3L * d, c.act_dtype,
                             nullptr, 0, 0, nullptr, 0, ni, 3 * d, d, EPI_STORE};
        gq.n = k;
    }
    if (fuse_rope) {
        gq.rope_cs = rope_cs; gq.rope_d = d; gq.rope_eps = c.eps_qk;
        int k = 0;
        if (nt) { gq.rope_w[k] = qkw_t; gq.rope_row0[k++] = 0; }
        if (ni) { gq.rope_w[k] = qkw_i; gq.rope_row0[k++] = nt; }
    }
    DIT_TRY(launch("gemm_qkv", s, [&] { return launch_gemm(gq, s); }));
    }

    // 4. QK RMSNorm + RoPE in place (text rows use the text weights), unless fused above
    QkRopeArgs r{};
    DIT_TRY(build_rope_table(c.head_dim, c.n_axes, c.axes_dim, c.theta, r.tab));
    r.q = qkv; r.ld_q = 3L * d; r.k = qkv + (size_t)d * es; r.ld_k = 3L * d;
    r.n_tok = n; r.n_heads = c.n_heads; r.qk_w0 = qkw_t; r.qk_w1 = qkw_i; r.n_first = nt;
    r.eps = c.eps_qk; r.pos = pos; r.n_axes = c.n_axes; r.dtype = c.act_dtype; r.w_dtype = c.dtype;
    if (fp8) {
        // e4m3 q, k, v for the attention (q, k in qkv stay unrotated)
        r.qkv8 = a8; r.ld8 = 3L * d; r.sq = a8_sq; r.sk = a8_sk; r.sv = a8_sv;
        r.v = qkv + (size_t)2 * d * es; r.ld_v = 3L * d; r.vmax = a8_vmax;
    }
    if (!fuse_rope)
        DIT_TRY(launch(fp8 ? "qk_rmsnorm_rope_fp8" : "qk_rmsnorm_rope", s, [&] { return launch_qk_rmsnorm_rope(r, s); }));

    // 5. O = joint attention over all n tokens
    if (fp8) {
        AttnFp8Args af{a8, 3L * d, a8_sq, a8 + d, 3L * d, a8_sk, a8 + 2 * (size_t)d, 3L * d, a8_sv, ob, d,
                       c.act_dtype, n, c.n_heads, 1.0f / std::sqrt((float)c.head_dim)};
        af.sk_scratch = W.ask_bytes ? ws + W.ask : nullptr;
        DIT_TRY(launch("joint_attention_fp8", s, [&] { return launch_attention_fp8(af, s); }));
    } else {
        AttnArgs at{qkv, 3L * d, qkv + (size_t)d * es, 3L * d, qkv + (size_t)2 * d * es, 3L * d, ob, d, n, c.n_heads,
                    1.0f / std::sqrt((float)c.head_dim), c.act_dtype};
        at.sk_scratch = W.ask_bytes ? ws + W.ask : nullptr;
        DIT_TRY(launch("joint_attention", s, [&] { return launch_attention(at, s); }));
    }

    // 6. h = x + gate1 * (O W_o^T)   (fp32)
    if (fp8) {
        DIT_TRY(quantize("quantize_o", ob, d));
        Fp8GemmBatch b{};
        if (nt) {
            b.p[b.n] = fp8_problem(0, nt, d, t8->w_o, t8->s_o, h, d, DIT_F32, d, EPI_GATED_RES);
            b.p[b.n].r = x_txt; b.p[b.n].ldr = d; b.p[b.n].r_dtype = c.x_dtype; b.p[b.n++].gate = mod_t + 2 * (size_t)d;
        }
        if (ni) {
            b.p[b.n] = fp8_problem(nt, ni, d, i8->w_o, i8->s_o, h + (size_t)nt * d, d, DIT_F32, d, EPI_GATED_RES);
            b.p[b.n].r = x_img; b.p[b.n].ldr = d; b.p[b.n].r_dtype = c.x_dtype; b.p[b.n++].gate = mod_i + 2 * (size_t)d;
        }
        DIT_TRY(launch("gemm_fp8_out_proj", s, [&] { return launch_gemm_fp8(b, s); }));
    } else {
    GemmBatch go{};
    go.sk_scratch = W.sk_bytes ? ws + W.sk : nullptr;
    go.a_dtype = c.act_dtype;
    go.b_f16 = c.gemm_w_dtype == DIT_F16;
    {
        int k = 0;
        if (nt) go.p[k++] = {ob, d, txt->w_o, d, h, d, DIT_F32, x_txt, d, c.x_dtype, mod_t + 2 * (size_t)d, 0, nt, d, d,
                             EPI_GATED_RES};
        if (ni) go.p[k++] = {ob + (size_t)nt * d * es, d, img->w_o, d, h + (size_t)nt * d, d, DIT_F32, x_img, d,
                             c.x_dtype, mod_i + 2 * (size_t)d, 0, ni, d, d, EPI_GATED_RES};
        go.n = k;
    }
    DIT_TRY(launch("gemm_out_proj", s, [&] { return launch_gemm(go, s); }));
    }

    // 7. b = (1 + scale2) RMSNorm(h) + shift2
    ModBatch m2{};
    nm = 0;
    if (nt) m2.p[nm++] = {h, d, DIT_F32, act, d, mod_t + 3 * (size_t)d, mod_t + 4 * (size_t)d, nt};
    if (ni) m2.p[nm++] = {h + (size_t)nt * d, d, DIT_F32, act + (size_t)nt * d * es, d, mod_i + 3 * (size_t)d,
                          mod_i + 4 * (size_t)d, ni};
    m2.n = nm; m2.d = d; m2.eps = c.eps; m2.out_dtype = c.act_dtype; m2.range_flag = flag;
    if (fp8) to_fp8(m2);
    DIT_TRY(launch(fp8 ? "modulate_h_fp8" : "modulate_h", s, [&] { return launch_modulate(m2, s); }));

    // 8. f = SiLU(b W_gate^T) * (b W_up^T)
    if (fp8) {
        Fp8GemmBatch b{};
        if (nt) {
            b.p[b.n] = fp8_problem(0, nt, d, t8->w_ffn_in, t8->s_ffn_in, f, F, c.act_dtype, F, EPI_SWIGLU);
            b.p[b.n++].up_off = F;
        }
        if (ni) {
            b.p[b.n] = fp8_problem(nt, ni, d, i8->w_ffn_in, i8->s_ffn_in, f + (size_t)nt * F * es, F, c.act_dtype, F,
                                   EPI_SWIGLU);
            b.p[b.n++].up_off = F;
        }
        b.range_flag = flag;
        DIT_TRY(launch("gemm_fp8_ffn_in_swiglu", s, [&] { return launch_gemm_fp8(b, s); }));
    } else {
    GemmBatch gf{};
    gf.range_flag = flag;
    gf.sk_scratch = W.sk_bytes ? ws + W.sk : nullptr;
    gf.a_dtype = c.act_dtype;
    gf.b_f16 = c.gemm_w_dtype == DIT_F16;
    {
        int k = 0;
        if (nt) gf.p[k++] = {act, d, txt->w_ffn_in, d, f, F, c.act_dtype, nullptr, 0, 0, nullptr, F, nt, F, d, EPI_SWIGLU};
        if (ni) gf.p[k++] = {act + (size_t)nt * d * es, d, img->w_ffn_in, d, f + (size_t)nt * F * es, F, c.act_dtype, nullptr,
                             0, 0, nullptr, F, ni, F, d, EPI_SWIGLU};
        gf.n = k;
    }
    DIT_TRY(launch("gemm_ffn_in_swiglu", s, [&] { return launch_gemm(gf, s); }));
    }

    // 9. y = h + gate2 * (f W_down^T)
    if (fp8) {
        DIT_TRY(quantize("quantize_f", f, F));
        Fp8GemmBatch b{};
        if (nt) {
            b.p[b.n] = fp8_problem(0, nt, F, t8->w_ffn_out, t8->s_ffn_out, y_txt, d, c.y_dtype, d, EPI_GATED_RES);
            b.p[b.n].r = h; b.p[b.n].ldr = d; b.p[b.n].r_dtype = DIT_F32; b.p[b.n++].gate = mod_t + 5 * (size_t)d;
        }
        if (ni) {
            b.p[b.n] = fp8_problem(nt, ni, F, i8->w_ffn_out, i8->s_ffn_out, y_img, d, c.y_dtype, d, EPI_GATED_RES);
            b.p[b.n].r = h + (size_t)nt * d; b.p[b.n].ldr = d; b.p[b.n].r_dtype = DIT_F32;
            b.p[b.n++].gate = mod_i + 5 * (size_t)d;
        }
        DIT_TRY(launch("gemm_fp8_ffn_down", s, [&] { return launch_gemm_fp8(b, s); }));
        return DIT_OK;
    }
    GemmBatch gd{};
    gd.sk_scratch = W.sk_bytes ? ws + W.sk : nullptr;
    gd.a_dtype = c.act_dtype;
    gd.b_f16 = c.gemm_w_dtype == DIT_F16;
    {
        int k = 0;
        if (nt) gd.p[k++] = {f, F, txt->w_ffn_out, F, y_txt, d, c.y_dtype, h, d, DIT_F32, mod_t + 5 * (size_t)d, 0, nt, d,
                             F, EPI_GATED_RES};
        if (ni) gd.p[k++] = {f + (size_t)nt * F * es, F, img->w_ffn_out, F, y_img, d, c.y_dtype, h + (size_t)nt * d, d,
                             DIT_F32, mod_i + 5 * (size_t)d, 0, ni, d, F, EPI_GATED_RES};
        gd.n = k;
    }
    DIT_TRY(launch("gemm_ffn_down", s, [&] { return launch_gemm(gd, s); }));
    return DIT_OK;
}

int dit_block_forward(const dit_block_config* cfg, const dit_stream_weights* txt, const dit_stream_weights* img,
                      const void* cond, const int32_t* pos, const void* x_txt, const void* x_img, void* y_txt,
                      void* y_img, void* workspace, size_t ws_bytes, void* stream) {
    return block_forward_impl(cfg, txt, img, cond, pos, x_txt, x_img, y_txt, y_img, workspace, ws_bytes, stream,
                              nullptr);
}

size_t dit_block_fp8_workspace_size(const dit_block_config* cfg) {
    clear_err();
    if (validate_fp8_config(cfg) != DIT_OK) return 0;
    return plan_workspace(cfg, 0, true).total;
}

int dit_block_forward_fp8(const dit_block_config* cfg, const dit_stream_weights_fp8* txt,
                          const dit_stream_weights_fp8* img, const void* cond, const int32_t* pos, const void* x_txt,
                          const void* x_img, void* y_txt, void* y_img, void* workspace, size_t ws_bytes,
                          void* stream) {
    if (!txt || !img) {
        clear_err();
        return fail(DIT_ERR_INVALID_ARG, "fp8 weights are NULL");
    }
    return block_forward_impl(cfg, nullptr, nullptr, cond, pos, x_txt, x_img, y_txt, y_img, workspace, ws_bytes,
                              stream, nullptr, txt, img);
}

// mod_pre: the [3d] fp32 AdaLN vectors computed by the caller, or NULL (from w->w_mod and cond).
static int single_block_impl(const dit_block_config* cfg, const dit_single_weights* w, const void* cond,
                             const int32_t* pos, const void* x, void* y, void* workspace, size_t ws_bytes,
                             void* stream, const float* mod_pre, const dit_single_weights_fp8* w8 = nullptr,
                             bool clear_flags = true) {
    clear_err();
    const bool fp8 = w8 != nullptr;
    DIT_TRY(fp8 ? validate_fp8_config(cfg) : validate_config(cfg));
    const dit_block_config& c = *cfg;
    const int n = c.n_txt + c.n_img, d = c.d, F = c.ffn_inner;
    if (!w && !w8) return fail(DIT_ERR_INVALID_ARG, "weights are NULL");
    const void* w_mod = fp8 ? w8->w_mod : w->w_mod;
    const void* w_1 = fp8 ? w8->w_1 : w->w_1;
    const void* w_2 = fp8 ? w8->w_2 : w->w_2;
    const void* qk_norm_w = fp8 ? w8->qk_norm_w : w->qk_norm_w;
    if (!mod_pre) DIT_TRY(check_ptr(w_mod, "w_mod"));
    DIT_TRY(check_ptr(w_1, "w_1"));
    DIT_TRY(check_ptr(qk_norm_w, "qk_norm_w"));
    DIT_TRY(check_ptr(w_2, "w_2"));
    if (fp8) {
        DIT_TRY(check_ptr(w8->s_1, "s_1"));
        DIT_TRY(check_ptr(w8->s_2, "s_2"));
    }
    if (!mod_pre) DIT_TRY(check_ptr(cond, "cond"));
    DIT_TRY(check_ptr(pos, "pos"));
    DIT_TRY(check_ptr(x, "x"));
    DIT_TRY(check_ptr(y, "y"));
    DIT_TRY(check_ptr(workspace, "workspace"));
    const WsPlan W = plan_workspace(cfg, 1, fp8);
    if (ws_bytes < W.total)
        return fail(DIT_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, W.total);
    const Range rws{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + W.total};
    const Range rx = range_of(x, n, d, d, c.x_dtype), ry = range_of(y, n, d, d, c.y_dtype);
    if (overlap(rws, rx) || overlap(rws, ry)) return fail(DIT_ERR_INVALID_ARG, "workspace overlaps x or y");
    if (overlap(rx, ry) && !(c.x_dtype == c.y_dtype && rx.lo == ry.lo))
        return fail(DIT_ERR_INVALID_ARG, "y overlaps x other than as an exact alias of the same dtype");

    char* ws = reinterpret_cast<char*>(workspace);
    float* mod = mod_pre ? const_cast<float*>(mod_pre) : reinterpret_cast<float*>(ws + W.mod);
    char* act = ws + W.act;
    char* qkv = ws + W.qkv;
    char* of = ws + W.of;
    uint8_t* q8 = fp8 ? reinterpret_cast<uint8_t*>(ws + W.q8) : nullptr;
    float* sq = fp8 ? reinterpret_cast<float*>(ws + W.sq) : nullptr;
    // fp8 attention operands: codes, scales, and the per-head |v| maxima (zeroed by the modulation)
    uint8_t* a8 = fp8 ? reinterpret_cast<uint8_t*>(ws + W.a8) : nullptr;
    float* a8_sq = fp8 ? reinterpret_cast<float*>(ws + W.a8s) : nullptr;
    float* a8_sk = fp8 ? a8_sq + (size_t)n * c.n_heads : nullptr;
    float* a8_sv = fp8 ? a8_sk + c.n_heads : nullptr;
    unsigned* a8_vmax = fp8 ? reinterpret_cast<unsigned*>(a8_sv + c.n_heads) : nullptr;
    unsigned* flag = reinterpret_cast<unsigned*>(ws + W.flags);
    const size_t es = esize(c.act_dtype);     // activation element size
    const long ldof = (long)d + F;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    if (!mod_pre) {
        GemvBatch g{};
        g.p[0] = {w_mod, mod, 3 * d};
        g.n = 1; g.cond = cond; g.d_cond = c.d_cond; g.dtype = c.dtype;
        g.clear_flag = clear_flags ? flag : nullptr;
        DIT_TRY(launch("adaln_gemv", s, [&] { return launch_adaln_gemv(g, s); }));
    }

    ModBatch m{};
    m.p[0] = {x, d, c.x_dtype, act, d, mod, mod + d, n};
    m.n = 1; m.d = d; m.eps = c.eps; m.out_dtype = c.act_dtype; m.range_flag = flag;
    if (fp8) {
        // a goes straight to e4m3 codes with per-row scales
        m.p[0].out = q8; m.p[0].out_scale = sq; m.out_dtype = FP8_ROWS;
        m.clear = a8_vmax; m.clear_n = c.n_heads;
    }
    DIT_TRY(launch(fp8 ? "modulate_x_fp8" : "modulate_x", s, [&] { return launch_modulate(m, s); }));

    // [q|k|v] = a W_1[0:3d]^T  and  f = SiLU(a W_1[3d:3d+F]^T) * (a W_1[3d+F:]^T), written next to O
    if (fp8) {
        auto prob = [&](const void* wq, const float* sw, void* out, long ldc, int N, int epi) {
            Fp8GemmProblem P{};
            P.a = q8; P.lda = d; P.sa = sq;
            P.b = reinterpret_cast<const uint8_t*>(wq); P.ldb = d; P.sb = sw;
            P.c = out; P.ldc = ldc; P.c_dtype = c.act_dtype;
            P.M = n; P.N = N; P.K = d; P.epi = epi;
            return P;
        };
        Fp8GemmBatch bq{}, bg{};
        bq.p[0] = prob(w_1, w8->s_1, qkv, 3L * d, 3 * d, EPI_STORE);
        bq.n = 1;
        bg.p[0] = prob(reinterpret_cast<const uint8_t*>(w_1) + (size_t)3 * d * d, w8->s_1 + 3 * (size_t)d,
                       of + (size_t)d * es, ldof, F, EPI_SWIGLU);
        bg.p[0].up_off = F;
        bg.n = 1;
        bq.range_flag = bg.range_flag = flag;
        bq.vmax = a8_vmax; bq.vmax_col0 = 2 * d;
        DIT_TRY(launch("gemm_fp8_linear1_qkv", s, [&] { return launch_gemm_fp8(bq, s); }));
        DIT_TRY(launch("gemm_fp8_linear1_gu", s, [&] { return launch_gemm_fp8(bg, s); }));
    } else {
        GemmBatch g1{};
        g1.range_flag = flag;
        g1.sk_scratch = W.sk_bytes ? ws + W.sk : nullptr;
        g1.a_dtype = c.act_dtype;
        g1.b_f16 = c.gemm_w_dtype == DIT_F16;
        g1.p[0] = {act, d, w_1, d, qkv, 3L * d, c.act_dtype, nullptr, 0, 0, nullptr, 0, n, 3 * d, d, EPI_STORE};
        g1.p[1] = {act, d, reinterpret_cast<const char*>(w_1) + (size_t)3 * d * d * esize(c.dtype), d,
                   of + (size_t)d * es, ldof, c.act_dtype, nullptr, 0, 0, nullptr, F, n, F, d, EPI_SWIGLU};
        g1.n = 2;
        DIT_TRY(launch("gemm_linear1", s, [&] { return launch_gemm(g1, s); }));
    }

    QkRopeArgs r{};
    DIT_TRY(build_rope_table(c.head_dim, c.n_axes, c.axes_dim, c.theta, r.tab));
    r.q = qkv; r.ld_q = 3L * d; r.k = qkv + (size_t)d * es; r.ld_k = 3L * d;
    r.n_tok = n; r.n_heads = c.n_heads; r.qk_w0 = qk_norm_w; r.qk_w1 = qk_norm_w; r.n_first = n;
    r.eps = c.eps_qk;
    r.pos = pos; r.n_axes = c.n_axes; r.dtype = c.act_dtype; r.w_dtype = c.dtype;
    if (fp8) {
        r.qkv8 = a8; r.ld8 = 3L * d; r.sq = a8_sq; r.sk = a8_sk; r.sv = a8_sv;
        r.v = qkv + (size_t)2 * d * es; r.ld_v = 3L * d; r.vmax = a8_vmax;
    }
    DIT_TRY(launch(fp8 ? "qk_rmsnorm_rope_fp8" : "qk_rmsnorm_rope", s, [&] { return launch_qk_rmsnorm_rope(r, s); }));

    if (fp8) {
        AttnFp8Args af{a8, 3L * d, a8_sq, a8 + d, 3L * d, a8_sk, a8 + 2 * (size_t)d, 3L * d, a8_sv, of, ldof,
                       c.act_dtype, n, c.n_heads, 1.0f / std::sqrt((float)c.head_dim)};
        af.sk_scratch = W.ask_bytes ? ws + W.ask : nullptr;
        DIT_TRY(launch("joint_attention_fp8", s, [&] { return launch_attention_fp8(af, s); }));
    } else {
        AttnArgs at{qkv, 3L * d, qkv + (size_t)d * es, 3L * d, qkv + (size_t)2 * d * es, 3L * d, of, ldof, n,
                    c.n_heads, 1.0f / std::sqrt((float)c.head_dim), c.act_dtype};
        at.sk_scratch = W.ask_bytes ? ws + W.ask : nullptr;
        DIT_TRY(launch("joint_attention", s, [&] { return launch_attention(at, s); }));
    }

    if (fp8) {
        DIT_TRY(launch("quantize_of", s, [&] {
            return launch_quantize_fp8(of, c.act_dtype, ldof, n, d + F, q8, ldof, sq, s);
        }));
        Fp8GemmBatch b2{};
        Fp8GemmProblem& P = b2.p[0];
        P.a = q8; P.lda = ldof; P.sa = sq;
        P.b = reinterpret_cast<const uint8_t*>(w_2); P.ldb = ldof; P.sb = w8->s_2;
        P.c = y; P.ldc = d; P.c_dtype = c.y_dtype;
        P.r = x; P.ldr = d; P.r_dtype = c.x_dtype; P.gate = mod + 2 * (size_t)d;
        P.M = n; P.N = d; P.K = d + F; P.epi = EPI_GATED_RES;
        b2.n = 1;
        DIT_TRY(launch("gemm_fp8_linear2", s, [&] { return launch_gemm_fp8(b2, s); }));
        return DIT_OK;
    }
    GemmBatch g2{};
    g2.sk_scratch = W.sk_bytes ? ws + W.sk : nullptr;
    g2.a_dtype = c.act_dtype;
    g2.b_f16 = c.gemm_w_dtype == DIT_F16;
    g2.p[0] = {of, ldof, w_2, ldof, y, d, c.y_dtype, x, d, c.x_dtype, mod + 2 * (size_t)d, 0, n, d, d + F,
               EPI_GATED_RES};
    g2.n = 1;
    DIT_TRY(launch("gemm_linear2", s, [&] { return launch_gemm(g2, s); }));
    return DIT_OK;
}

int dit_single_block_forward(const dit_block_config* cfg, const dit_single_weights* w, const void* cond,
                             const int32_t* pos, const void* x, void* y, void* workspace, size_t ws_bytes,
                             void* stream) {
    return single_block_impl(cfg, w, cond, pos, x, y, workspace, ws_bytes, stream, nullptr);
}

size_t dit_single_block_fp8_workspace_size(const dit_block_config* cfg) {
    clear_err();
    if (validate_fp8_config(cfg) != DIT_OK) return 0;
    return plan_workspace(cfg, 1, true).total;
}

int dit_single_block_forward_fp8(const dit_block_config* cfg, const dit_single_weights_fp8* w, const void* cond,
                                 const int32_t* pos, const void* x, void* y, void* workspace, size_t ws_bytes,
                                 void* stream) {
    if (!w) {
        clear_err();
        return fail(DIT_ERR_INVALID_ARG, "fp8 weights are NULL");
    }
    return single_block_impl(cfg, nullptr, cond, pos, x, y, workspace, ws_bytes, stream, nullptr, w);
}

// ---- kernel timing --------------------------------------------------------------------------
int dit_timing_begin(int capacity) {
    clear_err();
    TimingState& T = tl_timing;
    if (capacity < 1 || capacity > (1 << 20)) return fail(DIT_ERR_INVALID_ARG, "capacity = %d", capacity);
    for (hipEvent_t e : T.ev) (void)hipEventDestroy(e);
    T.ev.assign(2 * (size_t)capacity, nullptr);
    T.name.assign(capacity, nullptr);
    for (auto& e : T.ev)
        if (hipEventCreate(&e) != hipSuccess) return fail(DIT_ERR_HIP, "hipEventCreate failed");
    T.capacity = capacity;
    T.used = 0;
    T.on = true;
    return DIT_OK;
}

int dit_timing_end(void) {
    tl_timing.on = false;
    return DIT_OK;
}

int dit_timing_read(int i, char* name_buf, int name_len, int* launches, double* total_ms) {
    clear_err();
    TimingState& T = tl_timing;
    std::vector<const char*> names;
    std::vector<double> sums;
    std::vector<int> counts;
    for (int u = 0; u < T.used; ++u) {
        if (hipEventSynchronize(T.ev[2 * u + 1]) != hipSuccess) {
            fail(DIT_ERR_HIP, "hipEventSynchronize failed");
            return -1;
        }
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, T.ev[2 * u], T.ev[2 * u + 1]) != hipSuccess) {
            fail(DIT_ERR_HIP, "hipEventElapsedTime failed");
            return -1;
        }
        size_t k = 0;
        while (k < names.size() && std::strcmp(names[k], T.name[u]) != 0) ++k;
        if (k == names.size()) { names.push_back(T.name[u]); sums.push_back(0.0); counts.push_back(0); }
        sums[k] += ms;
        counts[k] += 1;
    }
    if (i >= 0 && i < (int)names.size()) {
        if (name_buf && name_len > 0) {
            std::strncpy(name_buf, names[i], (size_t)name_len - 1);
            name_buf[name_len - 1] = 0;
        }
        if (launches) *launches = counts[i];
        if (total_ms) *total_ms = sums[i];
    }
    return (int)names.size();
}

}  // extern "C"

// =========================================================================================
// The block stack of one denoising step.
// =========================================================================================
static size_t step_ws(const dit_block_config* cfg, int n_double, int n_single) {
    size_t need = 0;
    if (n_double > 0) need = plan_workspace(cfg, 0).total;
    if (n_single > 0) need = std::max(need, plan_workspace(cfg, 1).total);
    return need;
}
// The shared-modulation step appends the step's AdaLN vectors: [2][6d] (double) then [3d] (single).
static size_t shared_mod_bytes(const dit_block_config* cfg) { return up256((size_t)15 * cfg->d * 4); }

size_t dit_step_workspace_size(const dit_block_config* cfg, int n_double, int n_single) {
    clear_err();
    if (validate_config(cfg) != DIT_OK || n_double < 0 || n_single < 0) return 0;
    return step_ws(cfg, n_double, n_single);
}

size_t dit_step_shared_mod_workspace_size(const dit_block_config* cfg, int n_double, int n_single) {
    clear_err();
    if (validate_config(cfg) != DIT_OK || n_double < 0 || n_single < 0) return 0;
    return up256(step_ws(cfg, n_double, n_single)) + shared_mod_bytes(cfg);
}

// shared: NULL (every block computes its AdaLN vectors from its own w_mod), or the three shared
// modulation matrices {text [6d, d_cond], image [6d, d_cond], single [3d, d_cond]}.
static int step_forward_impl(const dit_block_config* cfg, int n_double, const dit_stream_weights* txt,
                             const dit_stream_weights* img, int n_single, const dit_single_weights* single,
                             const void* const* shared, const void* cond, const int32_t* pos, const void* x_txt,
                             const void* x_img, float* y, void* workspace, size_t ws_bytes, void* stream) {
    clear_err();
    DIT_TRY(validate_config(cfg));
    const dit_block_config& c = *cfg;
    if (n_double < 0 || n_single < 0 || n_double + n_single == 0)
        return fail(DIT_ERR_INVALID_ARG, "n_double = %d, n_single = %d: need >= 0 and at least one block", n_double,
                    n_single);
    if (n_double > 0 && (!txt || !img)) return fail(DIT_ERR_INVALID_ARG, "txt / img weight arrays are NULL");
    if (n_single > 0 && !single) return fail(DIT_ERR_INVALID_ARG, "single weight array is NULL");
    // everything is checked before the first launch
    char what[48];
    for (int b = 0; b < n_double; ++b) {
        snprintf(what, sizeof what, "txt[%d]", b);
        DIT_TRY(check_stream_weights(&txt[b], what, !shared));
        snprintf(what, sizeof what, "img[%d]", b);
        DIT_TRY(check_stream_weights(&img[b], what, !shared));
    }
    for (int b = 0; b < n_single; ++b) {
        const dit_single_weights& w = single[b];
        const void* p[4] = {w.w_mod, w.w_1, w.qk_norm_w, w.w_2};
        const char* nm[4] = {"w_mod", "w_1", "qk_norm_w", "w_2"};
        for (int i = shared ? 1 : 0; i < 4; ++i) {
            snprintf(what, sizeof what, "single[%d].%s", b, nm[i]);
            DIT_TRY(check_ptr(p[i], what));
        }
    }
    if (shared) {
        if (n_double > 0) {
            DIT_TRY(check_ptr(shared[0], "w_mod_txt"));
            DIT_TRY(check_ptr(shared[1], "w_mod_img"));
        }
        if (n_single > 0) DIT_TRY(check_ptr(shared[2], "w_mod_single"));
    }
    DIT_TRY(check_ptr(cond, "cond"));
    DIT_TRY(check_ptr(pos, "pos"));
    DIT_TRY(check_ptr(y, "y"));
    if (c.n_txt > 0) DIT_TRY(check_ptr(x_txt, "x_txt"));
    if (c.n_img > 0) DIT_TRY(check_ptr(x_img, "x_img"));
    DIT_TRY(check_ptr(workspace, "workspace"));
    const size_t blocks_need = step_ws(cfg, n_double, n_single);
    const size_t need = shared ? up256(blocks_need) + shared_mod_bytes(cfg) : blocks_need;
    if (ws_bytes < need) return fail(DIT_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
    const size_t nt = c.n_txt, ni = c.n_img, d = c.d, es = esize(c.x_dtype);
    if (n_double == 0 && nt > 0 && ni > 0 &&
        reinterpret_cast<const char*>(x_img) != reinterpret_cast<const char*>(x_txt) + nt * d * es)
        return fail(DIT_ERR_INVALID_ARG, "with no double-stream block, x_img must directly follow x_txt");
    const Range ry = range_of(y, (int)(nt + ni), (int)d, (long)d, DIT_F32);
    const Range rws{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
    const Range rxt = range_of(x_txt, (int)nt, (int)d, (long)d, c.x_dtype);
    const Range rxi = range_of(x_img, (int)ni, (int)d, (long)d, c.x_dtype);
    if (overlap(rws, ry) || overlap(rws, rxt) || overlap(rws, rxi))
        return fail(DIT_ERR_INVALID_ARG, "workspace overlaps an input or y");
    if (overlap(ry, rxt) || overlap(ry, rxi)) return fail(DIT_ERR_INVALID_ARG, "y overlaps x_txt / x_img");

    // shared modulation: one AdaLN GEMV launch per block kind for the whole step.  The step's first
    // kernel resets the range-flag word (the blocks' kernels then only raise it).
    float* mod_d = nullptr;
    float* mod_s = nullptr;
    unsigned* flag = reinterpret_cast<unsigned*>(workspace);
    bool cleared = false;
    if (shared) {
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        mod_d = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + up256(blocks_need));
        mod_s = mod_d + 12 * d;
        if (n_double > 0) {
            GemvBatch g{};
            g.p[0] = {shared[0], mod_d, (int)(6 * d)};
            g.p[1] = {shared[1], mod_d + 6 * d, (int)(6 * d)};
            g.n = 2; g.cond = cond; g.d_cond = c.d_cond; g.dtype = c.dtype;
            g.clear_flag = cleared ? nullptr : flag;
            cleared = true;
            DIT_TRY(launch("adaln_gemv", s, [&] { return launch_adaln_gemv(g, s); }));
        }
        if (n_single > 0) {
            GemvBatch g{};
            g.p[0] = {shared[2], mod_s, (int)(3 * d)};
            g.n = 1; g.cond = cond; g.d_cond = c.d_cond; g.dtype = c.dtype;
            g.clear_flag = cleared ? nullptr : flag;
            cleared = true;
            DIT_TRY(launch("adaln_gemv", s, [&] { return launch_adaln_gemv(g, s); }));
        }
    }

    // the first block reads x (cfg->x_dtype) and writes the fp32 stream y; the others update y in place
    dit_block_config c_first = c, c_rest = c;
    c_first.y_dtype = DIT_F32;
    c_rest.y_dtype = DIT_F32;
    c_rest.x_dtype = DIT_F32;
    float* y_txt = y;
    float* y_img = y + nt * d;
    for (int b = 0; b < n_double; ++b) {
        const dit_block_config* cb = b == 0 ? &c_first : &c_rest;
        DIT_TRY(block_forward_impl(cb, &txt[b], &img[b], cond, pos, b == 0 ? x_txt : y_txt, b == 0 ? x_img : y_img,
                                   y_txt, y_img, workspace, blocks_need, stream, mod_d, nullptr, nullptr, !cleared));
        cleared = true;
    }
    for (int b = 0; b < n_single; ++b) {
        const bool first = n_double == 0 && b == 0;
        DIT_TRY(single_block_impl(first ? &c_first : &c_rest, &single[b], cond, pos, first ? x_txt : y, y, workspace,
                                  blocks_need, stream, mod_s, nullptr, !cleared));
        cleared = true;
    }
    return DIT_OK;
}

int dit_step_forward(const dit_block_config* cfg, int n_double, const dit_stream_weights* txt,
                     const dit_stream_weights* img, int n_single, const dit_single_weights* single,
                     const void* cond, const int32_t* pos, const void* x_txt, const void* x_img, float* y,
                     void* workspace, size_t ws_bytes, void* stream) {
    return step_forward_impl(cfg, n_double, txt, img, n_single, single, nullptr, cond, pos, x_txt, x_img, y,
                             workspace, ws_bytes, stream);
}

int dit_step_forward_shared_mod(const dit_block_config* cfg, int n_double, const dit_stream_weights* txt,
                                const dit_stream_weights* img, int n_single, const dit_single_weights* single,
                                const void* w_mod_txt, const void* w_mod_img, const void* w_mod_single,
                                const void* cond, const int32_t* pos, const void* x_txt, const void* x_img, float* y,
                                void* workspace, size_t ws_bytes, void* stream) {
    const void* shared[3] = {w_mod_txt, w_mod_img, w_mod_single};
    return step_forward_impl(cfg, n_double, txt, img, n_single, single, shared, cond, pos, x_txt, x_img, y,
                             workspace, ws_bytes, stream);
}

// =========================================================================================
// The layers either side of the block stack.
// =========================================================================================
static size_t temb_ws(int freq_dim, int d) { return up256((size_t)freq_dim * 4) + 2 * up256((size_t)d * 4); }

size_t dit_timestep_embedding_workspace_size(int freq_dim, int d) {
    clear_err();
    if (freq_dim < 8 || freq_dim % 8 || d < 8 || d % 8) {
        fail(DIT_ERR_INVALID_ARG, "freq_dim = %d, d = %d: need multiples of 8, at least 8", freq_dim, d);
        return 0;
    }
    return temb_ws(freq_dim, d);
}

// Checks of the timestep embedding's arguments other than its scratch.
static int check_temb(int dtype, const float* t, const float* g, const void* w_t_in, const void* w_t_out,
                      const void* w_g_in, const void* w_g_out, int freq_dim, int d, float max_period,
                      float time_factor, const void* cond_out) {
    if (!valid_wdtype(dtype)) return fail(DIT_ERR_INVALID_ARG, "dtype must be DIT_BF16 or DIT_F32");
    if (freq_dim < 8 || freq_dim % 8 || freq_dim > 16384)
        return fail(DIT_ERR_INVALID_ARG, "freq_dim = %d must be a multiple of 8 in [8, 16384]", freq_dim);
    if (d < 8 || d % 8 || d > 16384) return fail(DIT_ERR_INVALID_ARG, "d = %d must be a multiple of 8 in [8, 16384]", d);
    if (!(max_period > 1.0f) || !std::isfinite(max_period)) return fail(DIT_ERR_INVALID_ARG, "max_period must be > 1");
    if (!std::isfinite(time_factor)) return fail(DIT_ERR_INVALID_ARG, "time_factor must be finite");
    if (!t) return fail(DIT_ERR_INVALID_ARG, "t is NULL");
    DIT_TRY(check_ptr(w_t_in, "w_t_in"));
    DIT_TRY(check_ptr(w_t_out, "w_t_out"));
    if (g) {
        DIT_TRY(check_ptr(w_g_in, "w_g_in"));
        DIT_TRY(check_ptr(w_g_out, "w_g_out"));
    }
    return check_ptr(cond_out, "cond_out");
}

// The launch sequence on scratch `ws` of temb_ws(freq_dim, d) bytes (arguments checked).
static int temb_launch(int dtype, hipStream_t s, const float* t, const float* g, const void* w_t_in,
                       const void* w_t_out, const void* w_g_in, const void* w_g_out, int freq_dim, int d,
                       float max_period, float time_factor, void* cond_out, char* ws) {
    float* emb = reinterpret_cast<float*>(ws);
    float* hid = reinterpret_cast<float*>(ws + up256((size_t)freq_dim * 4));
    float* acc = reinterpret_cast<float*>(ws + up256((size_t)freq_dim * 4) + up256((size_t)d * 4));
    // c = W_out . SiLU(W_in . emb(value)), summed over the timestep and (optionally) the guidance
    for (int pass = 0; pass < (g ? 2 : 1); ++pass) {
        const float* val = pass ? g : t;
        const void* wi = pass ? w_g_in : w_t_in;
        const void* wo = pass ? w_g_out : w_t_out;
        DIT_TRY(launch("timestep_freq", s, [&] { return launch_freq_embed(val, time_factor, max_period, freq_dim, emb, s); }));
        DIT_TRY(launch("embed_gemv_in", s, [&] { return launch_vec_gemv(wi, dtype, d, freq_dim, emb, false, hid, false, s); }));
        DIT_TRY(launch("embed_gemv_out", s, [&] { return launch_vec_gemv(wo, dtype, d, d, hid, true, acc, pass > 0, s); }));
    }
    return launch("cast", s, [&] { return launch_cast(acc, cond_out, d, dtype, s); });
}

int dit_timestep_embedding(int dtype, void* stream, const float* t, const float* g, const void* w_t_in,
                           const void* w_t_out, const void* w_g_in, const void* w_g_out, int freq_dim, int d,
                           float max_period, float time_factor, void* cond_out, void* workspace, size_t ws_bytes) {
    clear_err();
    DIT_TRY(check_temb(dtype, t, g, w_t_in, w_t_out, w_g_in, w_g_out, freq_dim, d, max_period, time_factor, cond_out));
    DIT_TRY(check_ptr(workspace, "workspace"));
    const size_t need = temb_ws(freq_dim, d);
    if (ws_bytes < need) return fail(DIT_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
    const Range rws{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
    if (overlap(rws, range_of(cond_out, 1, d, d, dtype))) return fail(DIT_ERR_INVALID_ARG, "cond_out overlaps the workspace");
    return temb_launch(dtype, reinterpret_cast<hipStream_t>(stream), t, g, w_t_in, w_t_out, w_g_in, w_g_out, freq_dim,
                       d, max_period, time_factor, cond_out, reinterpret_cast<char*>(workspace));
}

// ---- the allocation-free variant: its scratch is a file-scope device array --------------------
// Each GPU holds its own copy of `scratch` (DIT_TEMB_STATIC_SCRATCH bytes) until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: its device address on the
// current device comes from hipGetSymbolAddress, once per device, and only that address is handed
// to kernels.
static __device__ __align__(256) char scratch[DIT_TEMB_STATIC_SCRATCH];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (nullptr + error message on failure).
void* static_scratch(int& err) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        err = fail(DIT_ERR_HIP, "hipGetDevice failed or device %d out of range", dev);
        return nullptr;
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            err = fail(DIT_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}
}  // namespace

int dit_timestep_embedding_noalloc(int dtype, void* stream, const float* t, const float* g, const void* w_t_in,
                                   const void* w_t_out, const void* w_g_in, const void* w_g_out, int freq_dim, int d,
                                   float max_period, float time_factor, void* cond_out) {
    clear_err();
    DIT_TRY(check_temb(dtype, t, g, w_t_in, w_t_out, w_g_in, w_g_out, freq_dim, d, max_period, time_factor, cond_out));
    const size_t need = temb_ws(freq_dim, d);
    if (need > (size_t)DIT_TEMB_STATIC_SCRATCH)
        return fail(DIT_ERR_UNSUPPORTED, "freq_dim = %d, d = %d need %zu bytes of scratch; the static scratch holds %d",
                    freq_dim, d, need, DIT_TEMB_STATIC_SCRATCH);
    int err = DIT_OK;
    void* ws = static_scratch(err);
    if (!ws) return err;
    return temb_launch(dtype, reinterpret_cast<hipStream_t>(stream), t, g, w_t_in, w_t_out, w_g_in, w_g_out, freq_dim,
                       d, max_period, time_factor, cond_out, reinterpret_cast<char*>(ws));
}

int dit_linear(int dtype, void* stream, const void* x, int x_dtype, long ld_x, const void* w, int m, int n, int k,
               void* y, int y_dtype, long ld_y) {
    clear_err();
    if (!valid_wdtype(dtype)) return fail(DIT_ERR_INVALID_ARG, "dtype must be DIT_BF16 or DIT_F32");
    if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype))
        return fail(DIT_ERR_INVALID_ARG, "x_dtype / y_dtype must be DIT_F32, DIT_BF16 or DIT_F16");
    if (dtype == DIT_F32 && (x_dtype != DIT_F32 || y_dtype != DIT_F32))
        return fail(DIT_ERR_UNSUPPORTED, "fp32 weights need fp32 x and y");
    if (dtype == DIT_BF16 && x_dtype == DIT_F32)
        return fail(DIT_ERR_UNSUPPORTED, "bf16 weights need DIT_BF16 or DIT_F16 x");
    if (m < 0 || n < 8 || n % 8 || k < 16)
        return fail(DIT_ERR_INVALID_ARG, "m = %d, n = %d, k = %d: need m >= 0, n a multiple of 8", m, n, k);
    if (dtype == DIT_BF16 ? k % 64 : k % 16)
        return fail(DIT_ERR_UNSUPPORTED, "k = %d must be a multiple of %d", k, dtype == DIT_BF16 ? 64 : 16);
    if ((long)m * n > (1L << 31) || (long)n * k > (1L << 31)) return fail(DIT_ERR_UNSUPPORTED, "matrix too large");
    if (dtype != DIT_F32 && (k >= kGemmMaxLd || ld_x >= kGemmMaxLd))
        return fail(DIT_ERR_UNSUPPORTED, "k = %d, ld_x = %ld: row strides of 2^22 elements or more", k, ld_x);
    DIT_TRY(check_ptr(w, "w"));
    if (m == 0) return DIT_OK;
    DIT_TRY(check_ptr(x, "x"));
    DIT_TRY(check_ptr(y, "y"));
    DIT_TRY(check_ld(ld_x, k, x_dtype, "ld_x"));
    DIT_TRY(check_ld(ld_y, n, y_dtype, "ld_y"));
    const Range ry = range_of(y, m, ld_y, n, y_dtype);
    if (overlap(ry, range_of(x, m, ld_x, k, x_dtype)) || overlap(ry, range_of(w, n, k, k, dtype)))
        return fail(DIT_ERR_INVALID_ARG, "y overlaps x or w");
    GemmBatch b{};
    b.a_dtype = dtype == DIT_F32 ? DIT_F32 : x_dtype;
    b.p[0] = {x, ld_x, w, k, y, ld_y, y_dtype, nullptr, 0, 0, nullptr, 0, m, n, k, EPI_STORE};
    b.n = 1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch("gemm_linear", s, [&] { return launch_gemm(b, s); });
}

static size_t final_ws(int n_tok, int d, int act_dtype) {
    return up256((size_t)2 * d * 4) + up256((size_t)n_tok * d * esize(act_dtype));
}

size_t dit_final_layer_workspace_size(int n_tok, int d, int act_dtype) {
    clear_err();
    if (n_tok < 0 || d < 8 || !valid_dtype(act_dtype)) {
        fail(DIT_ERR_INVALID_ARG, "n_tok = %d, d = %d, act_dtype = %d", n_tok, d, act_dtype);
        return 0;
    }
    return final_ws(n_tok, d, act_dtype);
}

int dit_final_layer(int dtype, int act_dtype, void* stream, const void* x, int x_dtype, int n_tok, int d,
                    const void* cond, int d_cond, const void* w_mod, const void* w_out, int p, float eps, void* y,
                    int y_dtype, void* workspace, size_t ws_bytes) {
    clear_err();
    if (!valid_wdtype(dtype) || !valid_wdtype(x_dtype) || !valid_dtype(act_dtype) || !valid_dtype(y_dtype))
        return fail(DIT_ERR_INVALID_ARG, "dtype / x_dtype must be DIT_F32 or DIT_BF16, act_dtype / y_dtype one of "
                                         "DIT_F32, DIT_BF16, DIT_F16");
    if (dtype == DIT_F32 && (x_dtype != DIT_F32 || act_dtype != DIT_F32 || y_dtype != DIT_F32))
        return fail(DIT_ERR_UNSUPPORTED, "fp32 weights need fp32 x, activations and y");
    if (dtype == DIT_BF16 && act_dtype == DIT_F32)
        return fail(DIT_ERR_UNSUPPORTED, "bf16 weights need DIT_F16 or DIT_BF16 activations");
    if (n_tok < 0) return fail(DIT_ERR_INVALID_ARG, "n_tok = %d", n_tok);
    if (d < 64 || d % 64 || d > 8192) return fail(DIT_ERR_UNSUPPORTED, "d = %d must be a multiple of 64 in [64, 8192]", d);
    if (d_cond < 8 || d_cond % 8 || d_cond > 16384)
        return fail(DIT_ERR_INVALID_ARG, "d_cond = %d must be a multiple of 8 in [8, 16384]", d_cond);
    if (p < 8 || p % 8) return fail(DIT_ERR_INVALID_ARG, "p = %d must be a positive multiple of 8", p);
    if (!(eps >= 0.0f)) return fail(DIT_ERR_INVALID_ARG, "eps must be >= 0");
    DIT_TRY(check_ptr(cond, "cond"));
    DIT_TRY(check_ptr(w_mod, "w_mod"));
    DIT_TRY(check_ptr(w_out, "w_out"));
    DIT_TRY(check_ptr(workspace, "workspace"));
    const size_t need = final_ws(n_tok, d, act_dtype);
    if (ws_bytes < need) return fail(DIT_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
    if (n_tok > 0) {
        DIT_TRY(check_ptr(x, "x"));
        DIT_TRY(check_ptr(y, "y"));
    }
    const Range rws{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
    const Range rx = range_of(x, n_tok, d, d, x_dtype), ry = range_of(y, n_tok, p, p, y_dtype);
    if (overlap(rws, rx) || overlap(rws, ry)) return fail(DIT_ERR_INVALID_ARG, "workspace overlaps x or y");
    if (overlap(rx, ry)) return fail(DIT_ERR_INVALID_ARG, "y overlaps x");
    char* ws = reinterpret_cast<char*>(workspace);
    float* mod = reinterpret_cast<float*>(ws);
    char* act = ws + up256((size_t)2 * d * 4);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // [shift, scale] = W_mod . SiLU(c)
    GemvBatch g{};
    g.p[0] = {w_mod, mod, 2 * d};
    g.n = 1; g.cond = cond; g.d_cond = d_cond; g.dtype = dtype;
    DIT_TRY(launch("adaln_gemv", s, [&] { return launch_adaln_gemv(g, s); }));
    if (n_tok == 0) return DIT_OK;
    DIT_TRY(launch("layernorm_modulate", s, [&] {
        return launch_layernorm_modulate(x, x_dtype, d, act, act_dtype, d, mod, mod + d, n_tok, d, eps, s);
    }));
    GemmBatch b{};
    b.a_dtype = act_dtype;
    b.p[0] = {act, d, w_out, d, y, p, y_dtype, nullptr, 0, 0, nullptr, 0, n_tok, p, d, EPI_STORE};
    b.n = 1;
    return launch("gemm_final", s, [&] { return launch_gemm(b, s); });
}

// =========================================================================================
// Windowed (neighborhood) attention.
// =========================================================================================
int dit_neighborhood_attention(int dtype, void* stream, const void* q, long ld_q, const void* k, long ld_k,
                               const void* v, long ld_v, void* o, long ld_o, const int* grid, const int* kernel,
                               int n_heads, int head_dim, float softmax_scale) {
    clear_err();
    if (!valid_dtype(dtype)) return fail(DIT_ERR_INVALID_ARG, "dtype must be DIT_F32, DIT_BF16 or DIT_F16");
    if (!grid || !kernel) return fail(DIT_ERR_INVALID_ARG, "grid / kernel is NULL");
    if (head_dim != 128) return fail(DIT_ERR_UNSUPPORTED, "head_dim = %d (only 128 is supported)", head_dim);
    if (n_heads < 1) return fail(DIT_ERR_INVALID_ARG, "n_heads = %d", n_heads);
    long n_tok = 1;
    int keff[3];
    for (int a = 0; a < 3; ++a) {
        if (grid[a] < 1) return fail(DIT_ERR_INVALID_ARG, "grid[%d] = %d must be positive", a, grid[a]);
        if (kernel[a] < 1 || kernel[a] % 2 == 0)
            return fail(DIT_ERR_INVALID_ARG, "kernel[%d] = %d must be positive and odd", a, kernel[a]);
        keff[a] = std::min(kernel[a], grid[a]);
        n_tok *= grid[a];
        if (n_tok > (1L << 24)) return fail(DIT_ERR_UNSUPPORTED, "more than 2^24 tokens");
    }
    if (n_tok * n_heads > (1L << 30)) return fail(DIT_ERR_UNSUPPORTED, "n_tok * n_heads too large");
    if (!std::isfinite(softmax_scale)) return fail(DIT_ERR_INVALID_ARG, "softmax_scale must be finite");
    if (dtype != DIT_F32) {
        if (!(softmax_scale > 0.0f)) return fail(DIT_ERR_UNSUPPORTED, "the 16-bit kernel needs softmax_scale > 0");
        if (keff[2] > kWinMaxKW)
            return fail(DIT_ERR_UNSUPPORTED, "window of %d along W (at most %d on the 16-bit kernel)", keff[2], kWinMaxKW);
    } else if ((long)keff[0] * keff[1] * keff[2] > kWinMaxKeysF32) {
        return fail(DIT_ERR_UNSUPPORTED, "window of %ld keys (at most %d on the fp32 kernel)",
                    (long)keff[0] * keff[1] * keff[2], kWinMaxKeysF32);
    }
    const long width = (long)n_heads * head_dim;
    DIT_TRY(check_ptr(q, "q"));
    DIT_TRY(check_ptr(k, "k"));
    DIT_TRY(check_ptr(v, "v"));
    DIT_TRY(check_ptr(o, "o"));
    DIT_TRY(check_ld(ld_q, width, dtype, "ld_q"));
    DIT_TRY(check_ld(ld_k, width, dtype, "ld_k"));
    DIT_TRY(check_ld(ld_v, width, dtype, "ld_v"));
    DIT_TRY(check_ld(ld_o, width, dtype, "ld_o"));
    const Range ro = range_of(o, n_tok, ld_o, width, dtype);
    if (overlap(ro, range_of(q, n_tok, ld_q, width, dtype)) || overlap(ro, range_of(k, n_tok, ld_k, width, dtype)) ||
        overlap(ro, range_of(v, n_tok, ld_v, width, dtype)))
        return fail(DIT_ERR_INVALID_ARG, "o overlaps q, k or v");
    WinAttnArgs a{};
    a.q = q; a.ld_q = ld_q; a.k = k; a.ld_k = ld_k; a.v = v; a.ld_v = ld_v; a.o = o; a.ld_o = ld_o;
    a.T = grid[0]; a.H = grid[1]; a.W = grid[2];
    a.kT = keff[0]; a.kH = keff[1]; a.kW = keff[2];
    a.rT = kernel[0]; a.rH = kernel[1]; a.rW = kernel[2];
    a.n_heads = n_heads; a.scale = softmax_scale; a.dtype = dtype;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch("window_attention", s, [&] { return launch_window_attention(a, s); });
}

// =========================================================================================
// fp8 (OCP e4m3) quantisation and linear layer.
// =========================================================================================
int dit_convert_bf16_to_f16(void* stream, const void* src, void* dst, size_t n) {
    clear_err();
    if (n == 0) return DIT_OK;
    DIT_TRY(check_ptr(src, "src"));
    DIT_TRY(check_ptr(dst, "dst"));
    if (overlap(range_of(src, 1, (long)n, (long)n, DIT_BF16), range_of(dst, 1, (long)n, (long)n, DIT_F16)))
        return fail(DIT_ERR_INVALID_ARG, "src and dst overlap");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch("convert_bf16_to_f16", s, [&] { return launch_bf16_to_f16(src, dst, n, s); });
}

int dit_quantize_fp8(int x_dtype, void* stream, const void* x, long ld_x, int rows, int cols, void* q, long ld_q,
                     float* scales) {
    clear_err();
    if (!valid_dtype(x_dtype)) return fail(DIT_ERR_INVALID_ARG, "x_dtype must be DIT_F32, DIT_BF16 or DIT_F16");
    if (rows < 0 || cols < 8 || cols % 8) return fail(DIT_ERR_INVALID_ARG, "rows = %d, cols = %d: cols a multiple of 8", rows, cols);
    if (rows == 0) return DIT_OK;
    DIT_TRY(check_ptr(x, "x"));
    DIT_TRY(check_ptr(q, "q"));
    DIT_TRY(check_ptr(scales, "scales"));
    DIT_TRY(check_ld(ld_x, cols, x_dtype, "ld_x"));
    if (ld_q < cols || ld_q % 16) return fail(DIT_ERR_INVALID_ARG, "ld_q = %ld must be >= cols and a multiple of 16", ld_q);
    const Range rq{reinterpret_cast<uintptr_t>(q), reinterpret_cast<uintptr_t>(q) + (uintptr_t)((rows - 1) * ld_q + cols)};
    const Range rs = range_of(scales, 1, rows, rows, DIT_F32);
    if (overlap(rq, range_of(x, rows, ld_x, cols, x_dtype)) || overlap(rs, range_of(x, rows, ld_x, cols, x_dtype)) ||
        overlap(rq, rs))
        return fail(DIT_ERR_INVALID_ARG, "q, scales and x overlap");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch("quantize_fp8", s, [&] {
        return launch_quantize_fp8(x, x_dtype, ld_x, rows, cols, reinterpret_cast<uint8_t*>(q), ld_q, scales, s);
    });
}

int dit_linear_fp8(void* stream, const void* xq, long ld_x, const float* sx, const void* wq, long ld_w,
                   const float* sw, int m, int n, int k, void* y, int y_dtype, long ld_y) {
    clear_err();
    if (!valid_dtype(y_dtype)) return fail(DIT_ERR_INVALID_ARG, "y_dtype must be DIT_F32, DIT_BF16 or DIT_F16");
    if (m < 0 || n < 8 || n % 8) return fail(DIT_ERR_INVALID_ARG, "m = %d, n = %d: need m >= 0, n a multiple of 8", m, n);
    if (k < 128 || k % 128) return fail(DIT_ERR_UNSUPPORTED, "k = %d must be a positive multiple of 128", k);
    if ((long)m * n > (1L << 31) || (long)n * k > (1L << 31)) return fail(DIT_ERR_UNSUPPORTED, "matrix too large");
    DIT_TRY(check_ptr(wq, "wq"));
    DIT_TRY(check_ptr(sw, "sw"));
    if (ld_w < k || ld_w % 16) return fail(DIT_ERR_INVALID_ARG, "ld_w = %ld must be >= k and a multiple of 16", ld_w);
    if (m == 0) return DIT_OK;
    DIT_TRY(check_ptr(xq, "xq"));
    DIT_TRY(check_ptr(sx, "sx"));
    DIT_TRY(check_ptr(y, "y"));
    if (ld_x < k || ld_x % 16) return fail(DIT_ERR_INVALID_ARG, "ld_x = %ld must be >= k and a multiple of 16", ld_x);
    DIT_TRY(check_ld(ld_y, n, y_dtype, "ld_y"));
    const Range ry = range_of(y, m, ld_y, n, y_dtype);
    const Range rx{reinterpret_cast<uintptr_t>(xq), reinterpret_cast<uintptr_t>(xq) + (uintptr_t)((m - 1) * ld_x + k)};
    const Range rw{reinterpret_cast<uintptr_t>(wq), reinterpret_cast<uintptr_t>(wq) + (uintptr_t)((n - 1) * ld_w + k)};
    if (overlap(ry, rx) || overlap(ry, rw) || overlap(ry, range_of(sx, 1, m, m, DIT_F32)) ||
        overlap(ry, range_of(sw, 1, n, n, DIT_F32)))
        return fail(DIT_ERR_INVALID_ARG, "y overlaps an input");
    Fp8GemmBatch g{};
    Fp8GemmProblem& P = g.p[0];
    P.a = reinterpret_cast<const uint8_t*>(xq); P.lda = ld_x; P.sa = sx;
    P.b = reinterpret_cast<const uint8_t*>(wq); P.ldb = ld_w; P.sb = sw;
    P.c = y; P.ldc = ld_y; P.c_dtype = y_dtype;
    P.M = m; P.N = n; P.K = k; P.epi = EPI_STORE;
    g.n = 1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch("gemm_fp8", s, [&] { return launch_gemm_fp8(g, s); });
}

int dit_joint_attention_fp8(void* stream, const void* q8, long ld_q, const float* q_scale, const void* k8, long ld_k,
                            const float* k_scale, const void* v8, long ld_v, const float* v_scale, void* o,
                            int o_dtype, long ld_o, int n_tok, int n_heads, int head_dim, float softmax_scale) {
    clear_err();
    if (!valid_dtype(o_dtype)) return fail(DIT_ERR_INVALID_ARG, "o_dtype must be DIT_F32, DIT_BF16 or DIT_F16");
    if (head_dim != 128) return fail(DIT_ERR_UNSUPPORTED, "head_dim = %d (only 128 is supported)", head_dim);
    if (n_heads < 1) return fail(DIT_ERR_INVALID_ARG, "n_heads = %d", n_heads);
    if (n_tok < 0) return fail(DIT_ERR_INVALID_ARG, "n_tok = %d", n_tok);
    if (!std::isfinite(softmax_scale)) return fail(DIT_ERR_INVALID_ARG, "softmax_scale is not finite");
    if (n_tok == 0) return DIT_OK;          // nothing is read or written
    DIT_TRY(check_ptr(q8, "q"));
    DIT_TRY(check_ptr(k8, "k"));
    DIT_TRY(check_ptr(v8, "v"));
    DIT_TRY(check_ptr(q_scale, "q_scale"));
    DIT_TRY(check_ptr(k_scale, "k_scale"));
    DIT_TRY(check_ptr(v_scale, "v_scale"));
    DIT_TRY(check_ptr(o, "o"));
    const long width = (long)n_heads * head_dim;
    const long* lds[3] = {&ld_q, &ld_k, &ld_v};
    const char* names[3] = {"ld_q", "ld_k", "ld_v"};
    for (int i = 0; i < 3; ++i)
        if (*lds[i] < width || *lds[i] % 16 || *lds[i] >= (1L << 25))
            return fail(DIT_ERR_INVALID_ARG, "%s = %ld must be >= n_heads * 128, a multiple of 16 and below 2^25",
                        names[i], *lds[i]);
    if (reinterpret_cast<uintptr_t>(q8) % 16 || reinterpret_cast<uintptr_t>(k8) % 16 ||
        reinterpret_cast<uintptr_t>(v8) % 16)
        return fail(DIT_ERR_INVALID_ARG, "q, k and v must be 16-byte aligned");
    DIT_TRY(check_ld(ld_o, width, o_dtype, "ld_o"));
    if ((long)n_tok * n_heads > (1L << 30)) return fail(DIT_ERR_UNSUPPORTED, "n_tok * n_heads too large");
    const Range ro = range_of(o, n_tok, ld_o, width, o_dtype);
    auto codes = [&](const void* p, long ld) {
        return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + (uintptr_t)((n_tok - 1) * ld + width)};
    };
    if (overlap(ro, codes(q8, ld_q)) || overlap(ro, codes(k8, ld_k)) || overlap(ro, codes(v8, ld_v)) ||
        overlap(ro, range_of(q_scale, n_tok, n_heads, n_heads, DIT_F32)) ||
        overlap(ro, range_of(k_scale, 1, n_heads, n_heads, DIT_F32)) ||
        overlap(ro, range_of(v_scale, 1, n_heads, n_heads, DIT_F32)))
        return fail(DIT_ERR_INVALID_ARG, "o overlaps an input");
    AttnFp8Args a{q8, ld_q, q_scale, k8, ld_k, k_scale, v8, ld_v, v_scale, o, ld_o, o_dtype, n_tok, n_heads,
                  softmax_scale};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch("joint_attention_fp8", s, [&] { return launch_attention_fp8(a, s); });
}

int dit_mfma_loop(void* stream, int workgroups, int iters, float* out) {
    clear_err();
    if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24))
        return fail(DIT_ERR_INVALID_ARG, "workgroups = %d, iters = %d", workgroups, iters);
    DIT_TRY(check_ptr(out, "out"));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch("mfma_loop", s, [&] { return launch_mfma_loop(workgroups, iters, out, s); });
}

int dit_gemm_kloop_probe(void* stream, int mode, int workgroups, int ksteps, const void* window, size_t window_bytes,
                         float* out) {
    clear_err();
    if (mode < 0 || mode > 15 || ((mode & 8) && (mode & 2)))
        return fail(DIT_ERR_INVALID_ARG, "mode = %d (bit 3, registers only, excludes bit 1, global loads)", mode);
    if (workgroups < 1 || workgroups > (1 << 20) || ksteps < 1 || ksteps > (1 << 20))
        return fail(DIT_ERR_INVALID_ARG, "workgroups = %d, ksteps = %d", workgroups, ksteps);
    DIT_TRY(check_ptr(out, "out"));
    if (mode & 2) {
        DIT_TRY(check_ptr(window, "window"));
        if (window_bytes < ((size_t)4 << 20)) return fail(DIT_ERR_INVALID_ARG, "window_bytes = %zu < 4 MiB", window_bytes);
        if (reinterpret_cast<uintptr_t>(window) % 16) return fail(DIT_ERR_INVALID_ARG, "window must be 16-byte aligned");
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch("gemm_kloop_probe", s, [&] { return launch_gemm_kloop_probe(mode, workgroups, ksteps, window, out, s); });
}

int dit_attention_step_probe(void* stream, int mode, int workgroups, int tiles, float c2, float* out) {
    clear_err();
    if (mode < 0 || mode > 3) return fail(DIT_ERR_INVALID_ARG, "mode = %d", mode);
    if (workgroups < 1 || workgroups > (1 << 20) || tiles < 1 || tiles > (1 << 20))
        return fail(DIT_ERR_INVALID_ARG, "workgroups = %d, tiles = %d", workgroups, tiles);
    DIT_TRY(check_ptr(out, "out"));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch("attention_step_probe", s, [&] { return launch_attention_step_probe(mode, workgroups, tiles, c2, out, s); });
}

int dit_stream_probe(void* stream, int mode, const void* src, void* dst, size_t bytes, int workgroups, float* sink) {
    clear_err();
    if (mode != 0 && mode != 1) return fail(DIT_ERR_INVALID_ARG, "mode = %d", mode);
    if (bytes == 0 || bytes % 16384) return fail(DIT_ERR_INVALID_ARG, "bytes = %zu must be a positive multiple of 16384", bytes);
    if (workgroups < 1 || workgroups > (1 << 20)) return fail(DIT_ERR_INVALID_ARG, "workgroups = %d", workgroups);
    DIT_TRY(check_ptr(src, "src"));
    if (reinterpret_cast<uintptr_t>(src) % 16) return fail(DIT_ERR_INVALID_ARG, "src must be 16-byte aligned");
    if (mode == 1) {
        DIT_TRY(check_ptr(dst, "dst"));
        if (reinterpret_cast<uintptr_t>(dst) % 16) return fail(DIT_ERR_INVALID_ARG, "dst must be 16-byte aligned");
        const Range a{reinterpret_cast<uintptr_t>(src), reinterpret_cast<uintptr_t>(src) + bytes};
        const Range b{reinterpret_cast<uintptr_t>(dst), reinterpret_cast<uintptr_t>(dst) + bytes};
        if (overlap(a, b)) return fail(DIT_ERR_INVALID_ARG, "dst overlaps src");
    } else {
        DIT_TRY(check_ptr(sink, "sink"));
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch("stream_probe", s, [&] { return launch_stream_probe(src, dst, bytes, mode, workgroups, sink, s); });
}

// =========================================================================================
// 2-D convolution (NHWC), implicit GEMM.
// =========================================================================================
static int conv_impl(const char* name, int dtype, void* stream, const void* x, int batch, int frames, int height,
                     int width, int c_in, const void* weight, int c_out, int kt, int kh, int kw, const float* bias,
                     void* y, int y_dtype) {
    clear_err();
    if (dtype != DIT_BF16) return fail(DIT_ERR_UNSUPPORTED, "dtype must be DIT_BF16 (x and weight)");
    if (y_dtype != DIT_BF16 && y_dtype != DIT_F32) return fail(DIT_ERR_INVALID_ARG, "y_dtype must be DIT_BF16 or DIT_F32");
    if (batch < 0 || frames < 1 || height < 1 || width < 1)
        return fail(DIT_ERR_INVALID_ARG, "batch = %d, %d frames of %d x %d", batch, frames, height, width);
    if (c_in < 8 || c_in % 8) return fail(DIT_ERR_UNSUPPORTED, "c_in = %d must be a positive multiple of 8", c_in);
    if (c_out < 1) return fail(DIT_ERR_INVALID_ARG, "c_out = %d must be positive", c_out);
    if (kh < 1 || kw < 1 || kh % 2 == 0 || kw % 2 == 0 || kh > 7 || kw > 7)
        return fail(DIT_ERR_UNSUPPORTED, "kernel %d x %d: odd sizes up to 7", kh, kw);
    if (kt < 1 || kt > 7) return fail(DIT_ERR_UNSUPPORTED, "temporal kernel %d: 1 to 7 frames", kt);
    const long M = (long)batch * frames * height * width;
    const long K = (long)kt * kh * kw * c_in;
    if (M * c_in > (1L << 31) || M * c_out > (1L << 31) || (long)c_out * K > (1L << 31))
        return fail(DIT_ERR_UNSUPPORTED, "tensor too large");
    DIT_TRY(check_ptr(weight, "weight"));
    if (bias) DIT_TRY(check_ptr(bias, "bias"));
    if (M == 0) return DIT_OK;
    DIT_TRY(check_ptr(x, "x"));
    DIT_TRY(check_ptr(y, "y"));
    const Range ry = range_of(y, M, c_out, c_out, y_dtype);
    if (overlap(ry, range_of(x, M, c_in, c_in, dtype)) || overlap(ry, range_of(weight, c_out, K, K, dtype)) ||
        (bias && overlap(ry, range_of(bias, 1, c_out, c_out, DIT_F32))))
        return fail(DIT_ERR_INVALID_ARG, "y overlaps an input");
    ConvArgs a{};
    a.x = x; a.w = weight; a.bias = bias; a.y = y; a.y_dtype = y_dtype;
    a.B = batch; a.H = height; a.W = width; a.Cin = c_in; a.Cout = c_out; a.KH = kh; a.KW = kw;
    a.T = frames; a.KT = kt;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch(name, s, [&] { return launch_conv2d(a, s); });
}

int dit_conv2d(int dtype, void* stream, const void* x, int batch, int height, int width, int c_in, const void* weight,
               int c_out, int kh, int kw, const float* bias, void* y, int y_dtype) {
    return conv_impl("conv2d", dtype, stream, x, batch, 1, height, width, c_in, weight, c_out, 1, kh, kw, bias, y,
                     y_dtype);
}

int dit_conv3d_causal(int dtype, void* stream, const void* x, int batch, int frames, int height, int width, int c_in,
                      const void* weight, int c_out, int kt, int kh, int kw, const float* bias, void* y, int y_dtype) {
    return conv_impl("conv3d_causal", dtype, stream, x, batch, frames, height, width, c_in, weight, c_out, kt, kh, kw,
                     bias, y, y_dtype);
}
