"""MI355X (gfx950) forward pass of a FLUX-style joint text+image DiT block.

Thin ctypes binding over the C-ABI library ``libdit.so`` (``include/dit.h``):
argument marshalling only -- every step of the computation runs in the HIP
kernels of the library.  torch tensors provide device memory and the stream.
There is no CPU fallback: importing this package fails if the library is not
built (``python attention_dit_block_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence


__all__ = [
    "DIT_F32", "DIT_BF16", "DIT_F16", "DIT_OK", "DitError", "lib", "library_path",
    "BlockConfig", "StreamWeights", "SingleWeights",
    "adaln_modulate", "qk_rmsnorm_rope", "joint_attention",
    "block_workspace_size", "block_forward", "single_block_forward",
    "step_workspace_size", "step_forward", "step_shared_mod_workspace_size", "step_forward_shared_mod",
    "timestep_embedding_workspace_size", "timestep_embedding", "timestep_embedding_noalloc", "linear",
    "final_layer_workspace_size", "final_layer", "neighborhood_attention", "quantize_fp8", "linear_fp8",
    "StreamWeightsFp8", "block_fp8_workspace_size", "block_forward_fp8", "SingleWeightsFp8",
    "single_block_fp8_workspace_size", "single_block_forward_fp8", "conv2d", "conv3d_causal",
    "convert_bf16_to_f16",
    "last_error", "launch_count", "abi_version", "workspace_flags", "set_split_wait_limit", "DIT_RANGE_F16",
    "timing_begin", "timing_end", "timing_read",
    "joint_attention_fp8", "mfma_loop", "stream_probe", "gemm_kloop_probe", "attention_step_probe",
]

DIT_F32, DIT_BF16, DIT_F16 = 0, 1, 2
DIT_RANGE_F16 = 1
DIT_OK, DIT_ERR_INVALID_ARG, DIT_ERR_UNSUPPORTED, DIT_ERR_WORKSPACE, DIT_ERR_HIP = 0, 1, 2, 3, 4
STATUS_NAMES = {0: "DIT_OK", 1: "DIT_ERR_INVALID_ARG", 2: "DIT_ERR_UNSUPPORTED",
                3: "DIT_ERR_WORKSPACE", 4: "DIT_ERR_HIP"}

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdit.so")
if not os.path.exists(library_path):
    raise ImportError(f"{library_path} is not built: run `python attention_dit_block_amd/build.py`")
lib = ctypes.CDLL(library_path)

_vp, _i, _l, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_float, ctypes.c_size_t


class BlockConfig(ctypes.Structure):
    _fields_ = [("dtype", _i), ("act_dtype", _i), ("x_dtype", _i), ("y_dtype", _i), ("d", _i), ("n_heads", _i),
                ("head_dim", _i), ("ffn_inner", _i), ("d_cond", _i), ("n_txt", _i), ("n_img", _i),
                ("eps", _f), ("eps_qk", _f), ("theta", _f), ("n_axes", _i), ("axes_dim", _i * 4),
                ("gemm_w_dtype", _i)]


class StreamWeights(ctypes.Structure):
    _fields_ = [("w_mod", _vp), ("w_qkv", _vp), ("qk_norm_w", _vp), ("w_o", _vp),
                ("w_ffn_in", _vp), ("w_ffn_out", _vp)]


class SingleWeights(ctypes.Structure):
    _fields_ = [("w_mod", _vp), ("w_1", _vp), ("qk_norm_w", _vp), ("w_2", _vp)]


class SingleWeightsFp8(ctypes.Structure):
    _fields_ = [("w_mod", _vp), ("qk_norm_w", _vp), ("w_1", _vp), ("s_1", _vp), ("w_2", _vp), ("s_2", _vp)]


class StreamWeightsFp8(ctypes.Structure):
    _fields_ = [("w_mod", _vp), ("qk_norm_w", _vp), ("w_qkv", _vp), ("s_qkv", _vp), ("w_o", _vp), ("s_o", _vp),
                ("w_ffn_in", _vp), ("s_ffn_in", _vp), ("w_ffn_out", _vp), ("s_ffn_out", _vp)]


def _sig(name, res, args):
    f = getattr(lib, name)
    f.restype = res
    f.argtypes = args
    return f


_adaln = _sig("dit_adaln_modulate", _i, [_i, _vp, _vp, _i, _vp, _i, _i, _vp, _vp, _i, _i, _l, _i, _i, _f, _vp, _i,
                                         _l])
_qkrope = _sig("dit_qk_rmsnorm_rope", _i, [_i, _vp, _vp, _l, _vp, _l, _i, _i, _i, _vp, _i, _i, _f, _vp, _i,
                                           ctypes.POINTER(_i), _f])
_attn = _sig("dit_joint_attention", _i, [_i, _vp, _vp, _l, _vp, _l, _vp, _l, _vp, _l, _i, _i, _i, _f])
_wsize = _sig("dit_block_workspace_size", _sz, [ctypes.POINTER(BlockConfig), _i])
_block = _sig("dit_block_forward", _i, [ctypes.POINTER(BlockConfig), ctypes.POINTER(StreamWeights),
                                        ctypes.POINTER(StreamWeights), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_single = _sig("dit_single_block_forward", _i, [ctypes.POINTER(BlockConfig), ctypes.POINTER(SingleWeights),
                                                _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_step_wsize = _sig("dit_step_workspace_size", _sz, [ctypes.POINTER(BlockConfig), _i, _i])
_step = _sig("dit_step_forward", _i, [ctypes.POINTER(BlockConfig), _i, ctypes.POINTER(StreamWeights),
                                      ctypes.POINTER(StreamWeights), _i, ctypes.POINTER(SingleWeights), _vp, _vp,
                                      _vp, _vp, _vp, _vp, _sz, _vp])
_step_sm_wsize = _sig("dit_step_shared_mod_workspace_size", _sz, [ctypes.POINTER(BlockConfig), _i, _i])
_step_sm = _sig("dit_step_forward_shared_mod", _i, [ctypes.POINTER(BlockConfig), _i, ctypes.POINTER(StreamWeights),
                                                    ctypes.POINTER(StreamWeights), _i, ctypes.POINTER(SingleWeights),
                                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_temb_wsize = _sig("dit_timestep_embedding_workspace_size", _sz, [_i, _i])
_temb = _sig("dit_timestep_embedding", _i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _f, _vp, _vp, _sz])
_temb_na = _sig("dit_timestep_embedding_noalloc", _i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _f, _vp])
_linear = _sig("dit_linear", _i, [_i, _vp, _vp, _i, _l, _vp, _i, _i, _i, _vp, _i, _l])
_final_wsize = _sig("dit_final_layer_workspace_size", _sz, [_i, _i, _i])
_final = _sig("dit_final_layer", _i, [_i, _i, _vp, _vp, _i, _i, _i, _vp, _i, _vp, _vp, _i, _f, _vp, _i, _vp, _sz])
_natten = _sig("dit_neighborhood_attention", _i, [_i, _vp, _vp, _l, _vp, _l, _vp, _l, _vp, _l, ctypes.POINTER(_i),
                                                 ctypes.POINTER(_i), _i, _i, _f])
_quant8 = _sig("dit_quantize_fp8", _i, [_i, _vp, _vp, _l, _i, _i, _vp, _l, _vp])
_linear8 = _sig("dit_linear_fp8", _i, [_vp, _vp, _l, _vp, _vp, _l, _vp, _i, _i, _i, _vp, _i, _l])
_mfma_loop = _sig("dit_mfma_loop", _i, [_vp, _i, _i, _vp])
_stream_probe = _sig("dit_stream_probe", _i, [_vp, _i, _vp, _vp, _sz, _i, _vp])
_kloop_probe = _sig("dit_gemm_kloop_probe", _i, [_vp, _i, _i, _i, _vp, _sz, _vp])
_attn_step_probe = _sig("dit_attention_step_probe", _i, [_vp, _i, _i, _i, ctypes.c_float, _vp])
_attn8 = _sig("dit_joint_attention_fp8", _i, [_vp, _vp, _l, _vp, _vp, _l, _vp, _vp, _l, _vp, _vp, _i, _l, _i, _i, _i,
                                               _f])
_wsize8 = _sig("dit_block_fp8_workspace_size", _sz, [ctypes.POINTER(BlockConfig)])
_block8 = _sig("dit_block_forward_fp8", _i, [ctypes.POINTER(BlockConfig), ctypes.POINTER(StreamWeightsFp8),
                                             ctypes.POINTER(StreamWeightsFp8), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                             _vp])
_cvt16 = _sig("dit_convert_bf16_to_f16", _i, [_vp, _vp, _vp, _sz])
_conv3 = _sig("dit_conv3d_causal", _i, [_i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _vp, _vp, _i])
_swsize8 = _sig("dit_single_block_fp8_workspace_size", _sz, [ctypes.POINTER(BlockConfig)])
_single8 = _sig("dit_single_block_forward_fp8", _i, [ctypes.POINTER(BlockConfig), ctypes.POINTER(SingleWeightsFp8),
                                                     _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_conv = _sig("dit_conv2d", _i, [_i, _vp, _vp, _i, _i, _i, _i, _vp, _i, _i, _i, _vp, _vp, _i])
_last_error = _sig("dit_last_error", ctypes.c_char_p, [])
_launch_count = _sig("dit_launch_count", ctypes.c_uint64, [])
_abi = _sig("dit_abi_version", _i, [])
_wsflags = _sig("dit_workspace_flags", _i, [_vp, _vp, ctypes.POINTER(ctypes.c_uint32)])
_split_wait = _sig("dit_set_split_wait_limit", None, [_i])
_tbegin = _sig("dit_timing_begin", _i, [_i])
_tend = _sig("dit_timing_end", _i, [])
_tread = _sig("dit_timing_read", _i, [_i, ctypes.c_char_p, _i, ctypes.POINTER(_i), ctypes.POINTER(ctypes.c_double)])

EXPORTED = ["dit_adaln_modulate", "dit_qk_rmsnorm_rope", "dit_joint_attention", "dit_block_workspace_size",
            "dit_block_forward", "dit_single_block_forward", "dit_step_workspace_size", "dit_step_forward",
            "dit_step_shared_mod_workspace_size", "dit_step_forward_shared_mod",
            "dit_timestep_embedding_workspace_size", "dit_timestep_embedding", "dit_timestep_embedding_noalloc",
            "dit_linear",
            "dit_final_layer_workspace_size", "dit_final_layer", "dit_neighborhood_attention",
            "dit_quantize_fp8", "dit_linear_fp8", "dit_joint_attention_fp8", "dit_mfma_loop", "dit_stream_probe", "dit_gemm_kloop_probe", "dit_attention_step_probe", "dit_block_fp8_workspace_size", "dit_block_forward_fp8",
            "dit_single_block_fp8_workspace_size", "dit_single_block_forward_fp8",
            "dit_conv2d", "dit_conv3d_causal", "dit_convert_bf16_to_f16",
            "dit_last_error", "dit_launch_count", "dit_workspace_flags", "dit_set_split_wait_limit",
            "dit_abi_version", "dit_timing_begin", "dit_timing_end", "dit_timing_read"]


class DitError(RuntimeError):
    def __init__(self, code: int, fn: str):
        self.code = code
        self.status = STATUS_NAMES.get(code, str(code))
        super().__init__(f"{fn}: {self.status}: {last_error()}")


def last_error() -> str:
    return _last_error().decode()


def launch_count() -> int:
    return int(_launch_count())


def abi_version() -> int:
    return int(_abi())


def workspace_flags(workspace) -> int:
    """Range flags of the last block / step call that used ``workspace`` (waits for the current
    stream's work): DIT_RANGE_F16 set when an fp16 activation left fp16's finite range."""
    import torch
    out = ctypes.c_uint32(0)
    _check(_wsflags(_ptr(workspace, "workspace"), torch.cuda.current_stream().cuda_stream, ctypes.byref(out)),
           "dit_workspace_flags")
    return int(out.value)


def set_split_wait_limit(polls: int) -> None:
    """Test hook: bound on a split unit's owner waiting for a piece before it computes the piece
    itself (this thread's later calls; < 0 restores the default)."""
    _split_wait(int(polls))


def _check(rc: int, fn: str) -> None:
    if rc != DIT_OK:
        raise DitError(rc, fn)


# --- marshalling helpers -------------------------------------------------------------------

def _ptr(t, what: str, dtype=None) -> Optional[int]:
    """Device pointer of a torch tensor (None -> NULL).  Host tensors are refused, so a host
    address can never reach a kernel."""
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{what} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _need(t, n: int, what: str, contiguous: bool = True) -> None:
    """Refuse a tensor smaller than the call reads or writes (the C ABI sees only pointers)."""
    if t is None:
        return
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{what} has {t.numel()} elements, the call needs {n}")


def _rows(t, rows: int, width: int, what: str) -> None:
    """A strided 2-D view must cover rows x width with its own row stride."""
    if rows == 0:
        return
    if t.dim() != 2 or t.shape[0] < rows or t.shape[1] < width or t.stride(1) != 1:
        raise ValueError(f"{what} must be a [>= {rows}, >= {width}] view with unit column stride")


def _ld(t, what: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{what} must be a 2-D view with unit column stride")
    return t.stride(0)


def _dt(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DIT_BF16
    if t.dtype == torch.float32:
        return DIT_F32
    if t.dtype == torch.float16:
        return DIT_F16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# --- entry points ------------------------------------------------------------------------------

def adaln_modulate(cond, w_mod, n_chunks: int, d: int, mod_out, x=None, x_out=None, shift_chunk: int = 0,
                   scale_chunk: int = 1, eps: float = 1e-6, stream=None) -> None:
    """mod_out = W_mod SiLU(cond) (fp32); optionally x_out = (1+scale) RMSNorm(x) + shift."""
    import torch
    dtype = _dt(w_mod)
    n_tok, ld_x, ld_o, xdt, odt = 0, 0, 0, dtype, dtype
    _need(w_mod, n_chunks * d * cond.numel(), "w_mod")
    _need(cond, cond.numel(), "cond")
    _need(mod_out, n_chunks * d, "mod_out")
    if x is not None:
        if x_out is None:
            raise ValueError("x_out is required with x")
        n_tok, ld_x, ld_o, xdt, odt = x.shape[0], _ld(x, "x"), _ld(x_out, "x_out"), _dt(x), _dt(x_out)
        _rows(x, n_tok, d, "x")
        _rows(x_out, n_tok, d, "x_out")
    rc = _adaln(dtype, _stream(stream), _ptr(cond, "cond"), cond.numel(), _ptr(w_mod, "w_mod"), n_chunks, d,
                _ptr(mod_out, "mod_out", torch.float32), _ptr(x, "x"), xdt, n_tok, ld_x, shift_chunk, scale_chunk,
                eps, _ptr(x_out, "x_out"), odt, ld_o)
    _check(rc, "dit_adaln_modulate")


def qk_rmsnorm_rope(q, k, n_heads: int, qk_w, n_first: int, pos, eps: float = 1e-6,
                    axes_dim: Sequence[int] = (32, 32, 32, 32), theta: float = 1e4, head_dim: int = 128,
                    stream=None) -> None:
    """In place on the q and k views: per-head RMSNorm * weight, then 4-axis RoPE."""
    import torch
    axes = (_i * len(axes_dim))(*axes_dim)
    n = q.shape[0]
    _rows(q, n, n_heads * head_dim, "q")
    _rows(k, n, n_heads * head_dim, "k")
    _need(qk_w, (2 if n_first < n else 1) * 2 * head_dim, "qk_w")
    _need(pos, n * len(axes_dim), "pos")
    rc = _qkrope(_dt(q), _stream(stream), _ptr(q, "q"), _ld(q, "q"), _ptr(k, "k"), _ld(k, "k"), q.shape[0],
                 n_heads, head_dim, _ptr(qk_w, "qk_w"), _dt(qk_w), n_first, eps, _ptr(pos, "pos", torch.int32),
                 len(axes_dim), axes, theta)
    _check(rc, "dit_qk_rmsnorm_rope")


def joint_attention(q, k, v, o, n_heads: int, softmax_scale: Optional[float] = None, head_dim: int = 128,
                    stream=None) -> None:
    """o = softmax(q k^T * scale) v per head, over all rows (joint text+image attention)."""
    if softmax_scale is None:
        softmax_scale = head_dim ** -0.5
    n = q.shape[0]
    for t, what in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _rows(t, n, n_heads * head_dim, what)
    rc = _attn(_dt(q), _stream(stream), _ptr(q, "q"), _ld(q, "q"), _ptr(k, "k"), _ld(k, "k"), _ptr(v, "v"),
               _ld(v, "v"), _ptr(o, "o"), _ld(o, "o"), q.shape[0], n_heads, head_dim, softmax_scale)
    _check(rc, "dit_joint_attention")


@dataclass
class Shape:
    """Python-side block shape (mirrors dit_block_config).  act_dtype None: fp16
    activations for bf16 weights, fp32 for fp32 weights."""
    dtype: int
    d: int
    n_heads: int
    ffn_inner: int
    n_txt: int
    n_img: int
    d_cond: int = 0
    x_dtype: Optional[int] = None
    y_dtype: int = DIT_F32
    act_dtype: Optional[int] = None
    head_dim: int = 128
    eps: float = 1e-6
    eps_qk: float = 1e-6
    theta: float = 1e4
    axes_dim: Sequence[int] = (32, 32, 32, 32)
    gemm_w_dtype: int = 0       # 0: weights of dtype; DIT_F16: fp16 copies of the product weights

    def c_config(self) -> BlockConfig:
        c = BlockConfig()
        c.dtype = self.dtype
        if self.act_dtype is not None:
            c.act_dtype = self.act_dtype
        else:
            c.act_dtype = DIT_F16 if self.dtype == DIT_BF16 else DIT_F32
        c.x_dtype = self.dtype if self.x_dtype is None else self.x_dtype
        c.y_dtype = self.y_dtype
        c.d, c.n_heads, c.head_dim, c.ffn_inner = self.d, self.n_heads, self.head_dim, self.ffn_inner
        c.d_cond = self.d_cond or self.d
        c.n_txt, c.n_img = self.n_txt, self.n_img
        c.eps, c.eps_qk, c.theta = self.eps, self.eps_qk, self.theta
        c.n_axes = len(self.axes_dim)
        for i, a in enumerate(self.axes_dim):
            c.axes_dim[i] = a
        c.gemm_w_dtype = self.gemm_w_dtype
        return c


def block_workspace_size(shape: Shape, single_stream: bool = False) -> int:
    c = shape.c_config()
    n = _wsize(ctypes.byref(c), 1 if single_stream else 0)
    if n == 0:
        raise DitError(DIT_ERR_INVALID_ARG, "dit_block_workspace_size")
    return int(n)


def _stream_weights(shape: "Shape", w: dict, what: str, need_mod: bool = True) -> StreamWeights:
    d, F, dc, hd = shape.d, shape.ffn_inner, shape.d_cond or shape.d, shape.head_dim
    sizes = {"w_mod": 6 * d * dc, "w_qkv": 3 * d * d, "qk_norm_w": 2 * hd, "w_o": d * d,
             "w_ffn_in": 2 * F * d, "w_ffn_out": d * F}
    s = StreamWeights()
    for name, n in sizes.items():
        if name == "w_mod" and not need_mod and w.get(name) is None:
            continue
        _need(w.get(name), n, f"{what}.{name}")
        setattr(s, name, _ptr(w.get(name), f"{what}.{name}"))
    return s


def _check_block_io(shape: "Shape", cond, pos, pairs) -> None:
    _need(cond, shape.d_cond or shape.d, "cond")
    _need(pos, (shape.n_txt + shape.n_img) * len(shape.axes_dim), "pos")
    for t, n, what in pairs:
        if n:
            _need(t, n * shape.d, what)


def block_forward(shape: Shape, txt: dict, img: dict, cond, pos, x_txt, x_img, y_txt, y_img, workspace,
                  stream=None) -> None:
    """Double-stream block: y_txt, y_img from x_txt, x_img (see include/dit.h)."""
    import torch
    c = shape.c_config()
    wt, wi = _stream_weights(shape, txt, "txt"), _stream_weights(shape, img, "img")
    _check_block_io(shape, cond, pos, ((x_txt, shape.n_txt, "x_txt"), (x_img, shape.n_img, "x_img"),
                                       (y_txt, shape.n_txt, "y_txt"), (y_img, shape.n_img, "y_img")))
    rc = _block(ctypes.byref(c), ctypes.byref(wt), ctypes.byref(wi), _ptr(cond, "cond"),
                _ptr(pos, "pos", torch.int32), _ptr(x_txt, "x_txt"), _ptr(x_img, "x_img"), _ptr(y_txt, "y_txt"),
                _ptr(y_img, "y_img"), _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                _stream(stream))
    _check(rc, "dit_block_forward")


def single_block_forward(shape: Shape, w: dict, cond, pos, x, y, workspace, stream=None) -> None:
    """Single-stream block over x = [text; image] (see include/dit.h)."""
    import torch
    c = shape.c_config()
    d, F, dc, hd = shape.d, shape.ffn_inner, shape.d_cond or shape.d, shape.head_dim
    n = shape.n_txt + shape.n_img
    sw = SingleWeights()
    for name, size in (("w_mod", 3 * d * dc), ("w_1", (3 * d + 2 * F) * d), ("qk_norm_w", 2 * hd),
                       ("w_2", d * (d + F))):
        _need(w[name], size, name)
        setattr(sw, name, _ptr(w[name], name))
    _check_block_io(shape, cond, pos, ((x, n, "x"), (y, n, "y")))
    rc = _single(ctypes.byref(c), ctypes.byref(sw), _ptr(cond, "cond"), _ptr(pos, "pos", torch.int32),
                 _ptr(x, "x"), _ptr(y, "y"), _ptr(workspace, "workspace"),
                 workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "dit_single_block_forward")


def _single_weights(shape: "Shape", w: dict, what: str, need_mod: bool = True) -> SingleWeights:
    d, F, dc, hd = shape.d, shape.ffn_inner, shape.d_cond or shape.d, shape.head_dim
    sw = SingleWeights()
    for name, size in (("w_mod", 3 * d * dc), ("w_1", (3 * d + 2 * F) * d), ("qk_norm_w", 2 * hd),
                       ("w_2", d * (d + F))):
        if name == "w_mod" and not need_mod and w.get(name) is None:
            continue
        _need(w.get(name), size, f"{what}.{name}")
        setattr(sw, name, _ptr(w.get(name), f"{what}.{name}"))
    return sw


def step_workspace_size(shape: Shape, n_double: int, n_single: int) -> int:
    c = shape.c_config()
    n = int(_step_wsize(ctypes.byref(c), n_double, n_single))
    if n == 0:
        raise DitError(DIT_ERR_INVALID_ARG, "dit_step_workspace_size")
    return n


def step_forward(shape: Shape, txt: list, img: list, single: list, cond, pos, x_txt, x_img, y, workspace,
                 stream=None) -> None:
    """The block stack of a denoising step: len(txt) double-stream blocks, then len(single)
    single-stream blocks; y (fp32 [n_txt + n_img, d]) ends as the stack's output (see include/dit.h)."""
    import torch
    if len(txt) != len(img):
        raise ValueError("txt and img need one weight dict per double-stream block each")
    c = shape.c_config()
    nd, ns = len(txt), len(single)
    wt = (StreamWeights * max(nd, 1))(*[_stream_weights(shape, w, f"txt[{i}]") for i, w in enumerate(txt)])
    wi = (StreamWeights * max(nd, 1))(*[_stream_weights(shape, w, f"img[{i}]") for i, w in enumerate(img)])
    sw = (SingleWeights * max(ns, 1))(*[_single_weights(shape, w, f"single[{i}]") for i, w in enumerate(single)])
    n = shape.n_txt + shape.n_img
    _check_block_io(shape, cond, pos, ((x_txt, shape.n_txt, "x_txt"), (x_img, shape.n_img, "x_img"), (y, n, "y")))
    rc = _step(ctypes.byref(c), nd, wt, wi, ns, sw, _ptr(cond, "cond"), _ptr(pos, "pos", torch.int32),
               _ptr(x_txt, "x_txt"), _ptr(x_img, "x_img"), _ptr(y, "y", torch.float32), _ptr(workspace, "workspace"),
               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "dit_step_forward")


def step_shared_mod_workspace_size(shape: Shape, n_double: int, n_single: int) -> int:
    c = shape.c_config()
    n = int(_step_sm_wsize(ctypes.byref(c), n_double, n_single))
    if n == 0:
        raise DitError(DIT_ERR_INVALID_ARG, "dit_step_shared_mod_workspace_size")
    return n


def step_forward_shared_mod(shape: Shape, txt: list, img: list, single: list, w_mod_txt, w_mod_img, w_mod_single,
                            cond, pos, x_txt, x_img, y, workspace, stream=None) -> None:
    """step_forward with one AdaLN weight set per block kind shared by all blocks (the blocks'
    own w_mod entries are not read and may be missing); see include/dit.h."""
    import torch
    if len(txt) != len(img):
        raise ValueError("txt and img need one weight dict per double-stream block each")
    c = shape.c_config()
    nd, ns = len(txt), len(single)
    d, dc = shape.d, shape.d_cond or shape.d
    wt = (StreamWeights * max(nd, 1))(*[_stream_weights(shape, w, f"txt[{i}]", False) for i, w in enumerate(txt)])
    wi = (StreamWeights * max(nd, 1))(*[_stream_weights(shape, w, f"img[{i}]", False) for i, w in enumerate(img)])
    sw = (SingleWeights * max(ns, 1))(*[_single_weights(shape, w, f"single[{i}]", False)
                                        for i, w in enumerate(single)])
    if nd:
        _need(w_mod_txt, 6 * d * dc, "w_mod_txt")
        _need(w_mod_img, 6 * d * dc, "w_mod_img")
    if ns:
        _need(w_mod_single, 3 * d * dc, "w_mod_single")
    n = shape.n_txt + shape.n_img
    _check_block_io(shape, cond, pos, ((x_txt, shape.n_txt, "x_txt"), (x_img, shape.n_img, "x_img"), (y, n, "y")))
    rc = _step_sm(ctypes.byref(c), nd, wt, wi, ns, sw, _ptr(w_mod_txt, "w_mod_txt"), _ptr(w_mod_img, "w_mod_img"),
                  _ptr(w_mod_single, "w_mod_single"), _ptr(cond, "cond"), _ptr(pos, "pos", torch.int32),
                  _ptr(x_txt, "x_txt"), _ptr(x_img, "x_img"), _ptr(y, "y", torch.float32),
                  _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "dit_step_forward_shared_mod")


# --- the layers either side of the block stack ----------------------------------------------------

def timestep_embedding_workspace_size(freq_dim: int, d: int) -> int:
    n = int(_temb_wsize(freq_dim, d))
    if n == 0:
        raise DitError(DIT_ERR_INVALID_ARG, "dit_timestep_embedding_workspace_size")
    return n


def timestep_embedding(t, w_t_in, w_t_out, cond_out, workspace, g=None, w_g_in=None, w_g_out=None,
                       max_period: float = 1e4, time_factor: float = 1000.0, stream=None) -> None:
    """cond_out = MLP_t(emb(t)) [+ MLP_g(emb(g))]; t and g are fp32 [1] GPU tensors (see include/dit.h)."""
    import torch
    d, fd = w_t_in.shape[0], w_t_in.shape[1]
    _need(w_t_in, d * fd, "w_t_in")
    _need(w_t_out, d * d, "w_t_out")
    _need(cond_out, d, "cond_out")
    _need(t, 1, "t")
    if g is not None:
        _need(g, 1, "g")
        _need(w_g_in, d * fd, "w_g_in")
        _need(w_g_out, d * d, "w_g_out")
    rc = _temb(_dt(w_t_in), _stream(stream), _ptr(t, "t", torch.float32), _ptr(g, "g", torch.float32),
               _ptr(w_t_in, "w_t_in"), _ptr(w_t_out, "w_t_out"), _ptr(w_g_in, "w_g_in"), _ptr(w_g_out, "w_g_out"),
               fd, d, max_period, time_factor, _ptr(cond_out, "cond_out"), _ptr(workspace, "workspace"),
               workspace.numel() * workspace.element_size())
    _check(rc, "dit_timestep_embedding")


def timestep_embedding_noalloc(t, w_t_in, w_t_out, cond_out, g=None, w_g_in=None, w_g_out=None,
                               max_period: float = 1e4, time_factor: float = 1000.0, stream=None) -> None:
    """timestep_embedding with the library's static per-GPU scratch instead of a workspace (no
    allocation; calls that overlap on one GPU race -- see include/dit.h)."""
    import torch
    d, fd = w_t_in.shape[0], w_t_in.shape[1]
    _need(w_t_in, d * fd, "w_t_in")
    _need(w_t_out, d * d, "w_t_out")
    _need(cond_out, d, "cond_out")
    _need(t, 1, "t")
    if g is not None:
        _need(g, 1, "g")
        _need(w_g_in, d * fd, "w_g_in")
        _need(w_g_out, d * d, "w_g_out")
    rc = _temb_na(_dt(w_t_in), _stream(stream), _ptr(t, "t", torch.float32), _ptr(g, "g", torch.float32),
                  _ptr(w_t_in, "w_t_in"), _ptr(w_t_out, "w_t_out"), _ptr(w_g_in, "w_g_in"), _ptr(w_g_out, "w_g_out"),
                  fd, d, max_period, time_factor, _ptr(cond_out, "cond_out"))
    _check(rc, "dit_timestep_embedding_noalloc")


def linear(x, w, y, stream=None) -> None:
    """y = x w^T (x [m, k], w [n, k], y [m, n]; 2-D views with unit column stride)."""
    m, k = x.shape
    n = w.shape[0]
    _rows(x, m, k, "x")
    _rows(y, m, n, "y")
    _need(w, n * k, "w")
    rc = _linear(_dt(w), _stream(stream), _ptr(x, "x"), _dt(x), _ld(x, "x"), _ptr(w, "w"), m, n, k, _ptr(y, "y"),
                 _dt(y), _ld(y, "y"))
    _check(rc, "dit_linear")


def final_layer_workspace_size(n_tok: int, d: int, act_dtype: int) -> int:
    n = int(_final_wsize(n_tok, d, act_dtype))
    if n == 0:
        raise DitError(DIT_ERR_INVALID_ARG, "dit_final_layer_workspace_size")
    return n


def final_layer(x, cond, w_mod, w_out, y, workspace, act_dtype: Optional[int] = None, eps: float = 1e-6,
                stream=None) -> None:
    """y = ((1 + scale) LayerNorm(x) + shift) w_out^T, [shift, scale] = w_mod SiLU(cond)."""
    n_tok, d = x.shape
    p = w_out.shape[0]
    dtype = _dt(w_out)
    if act_dtype is None:
        act_dtype = DIT_F16 if dtype == DIT_BF16 else DIT_F32
    _need(x, n_tok * d, "x")
    _need(y, n_tok * p, "y")
    _need(cond, cond.numel(), "cond")
    _need(w_mod, 2 * d * cond.numel(), "w_mod")
    _need(w_out, p * d, "w_out")
    rc = _final(dtype, act_dtype, _stream(stream), _ptr(x, "x"), _dt(x), n_tok, d, _ptr(cond, "cond"), cond.numel(),
                _ptr(w_mod, "w_mod"), _ptr(w_out, "w_out"), p, eps, _ptr(y, "y"), _dt(y),
                _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size())
    _check(rc, "dit_final_layer")


def neighborhood_attention(q, k, v, o, grid: Sequence[int], kernel: Sequence[int], n_heads: int,
                           softmax_scale: Optional[float] = None, head_dim: int = 128, stream=None) -> None:
    """Windowed attention over a [T, H, W] token grid (see include/dit.h)."""
    if softmax_scale is None:
        softmax_scale = head_dim ** -0.5
    n = int(grid[0]) * int(grid[1]) * int(grid[2])
    for t, what in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _rows(t, n, n_heads * head_dim, what)
    g = (_i * 3)(*grid)
    kk = (_i * 3)(*kernel)
    rc = _natten(_dt(q), _stream(stream), _ptr(q, "q"), _ld(q, "q"), _ptr(k, "k"), _ld(k, "k"), _ptr(v, "v"),
                 _ld(v, "v"), _ptr(o, "o"), _ld(o, "o"), g, kk, n_heads, head_dim, softmax_scale)
    _check(rc, "dit_neighborhood_attention")


def quantize_fp8(x, q, scales, stream=None) -> None:
    """Per-row e4m3 quantisation of x [rows, cols] into q (uint8 [rows, cols]) and scales (fp32
    [rows]); see include/dit.h."""
    import torch
    rows, cols = x.shape
    _rows(x, rows, cols, "x")
    _rows(q, rows, cols, "q")
    _need(scales, rows, "scales")
    rc = _quant8(_dt(x), _stream(stream), _ptr(x, "x"), _ld(x, "x"), rows, cols, _ptr(q, "q", torch.uint8), _ld(q, "q"),
                 _ptr(scales, "scales", torch.float32))
    _check(rc, "dit_quantize_fp8")


def linear_fp8(xq, sx, wq, sw, y, stream=None) -> None:
    """y = diag(sx) (xq wq^T) diag(sw) on e4m3 codes (uint8 tensors); see include/dit.h."""
    import torch
    m, k = xq.shape
    n = wq.shape[0]
    _rows(xq, m, k, "xq")
    _rows(wq, n, k, "wq")
    _rows(y, m, n, "y")
    _need(sx, m, "sx")
    _need(sw, n, "sw")
    rc = _linear8(_stream(stream), _ptr(xq, "xq", torch.uint8), _ld(xq, "xq"), _ptr(sx, "sx", torch.float32),
                  _ptr(wq, "wq", torch.uint8), _ld(wq, "wq"), _ptr(sw, "sw", torch.float32), m, n, k, _ptr(y, "y"),
                  _dt(y), _ld(y, "y"))
    _check(rc, "dit_linear_fp8")


def joint_attention_fp8(q8, sq, k8, sk, v8, sv, o, n_heads: int, softmax_scale: Optional[float] = None,
                        head_dim: int = 128, stream=None) -> None:
    """Joint attention on e4m3 codes (uint8 tensors [n, n_heads*head_dim]) with per token-and-head
    q scales sq [n, n_heads] and per-head k / v scales sk, sv [n_heads]; see include/dit.h."""
    import torch
    if softmax_scale is None:
        softmax_scale = head_dim ** -0.5
    n = q8.shape[0]
    for t, what in ((q8, "q8"), (k8, "k8"), (v8, "v8"), (o, "o")):
        _rows(t, n, n_heads * head_dim, what)
    _need(sq, n * n_heads, "sq")
    _need(sk, n_heads, "sk")
    _need(sv, n_heads, "sv")
    rc = _attn8(_stream(stream), _ptr(q8, "q8", torch.uint8), _ld(q8, "q8"), _ptr(sq, "sq", torch.float32),
                _ptr(k8, "k8", torch.uint8), _ld(k8, "k8"), _ptr(sk, "sk", torch.float32),
                _ptr(v8, "v8", torch.uint8), _ld(v8, "v8"), _ptr(sv, "sv", torch.float32),
                _ptr(o, "o"), _dt(o), _ld(o, "o"), n, n_heads, head_dim, softmax_scale)
    _check(rc, "dit_joint_attention_fp8")


def mfma_loop(workgroups: int, iters: int, out, stream=None) -> None:
    """Calibration: workgroups x 4 waves x 4 chains x iters fp16 32x32x16 MFMAs (32768 flop each)."""
    import torch
    _need(out, workgroups * 256, "out")
    _check(_mfma_loop(_stream(stream), workgroups, iters, _ptr(out, "out", torch.float32)), "dit_mfma_loop")


def stream_probe(mode: int, src, dst=None, sink=None, workgroups: int = 2048, stream=None) -> None:
    """Calibration: stream src (mode 0: read into sink [workgroups*256] fp32; mode 1: copy to dst)."""
    import torch
    nbytes = src.numel() * src.element_size()
    _need(src, src.numel(), "src")
    if mode == 1:
        _need(dst, src.numel(), "dst")
        if dst.element_size() != src.element_size():
            raise ValueError("dst must have src's element size")
    else:
        _need(sink, workgroups * 256, "sink")
    rc = _stream_probe(_stream(stream), mode, _ptr(src, "src"), _ptr(dst, "dst") if mode == 1 else None, nbytes,
                       workgroups, _ptr(sink, "sink", torch.float32) if mode == 0 else None)
    _check(rc, "dit_stream_probe")


def gemm_kloop_probe(mode: int, workgroups: int, ksteps: int, out, window=None, stream=None) -> None:
    """Calibration: the GEMM k-loop on LDS-resident operands (mode bit 0 ping-pong, bit 1 global loads
    from window, >= 4 MiB of fp16; bit 2 random operands); out [workgroups * 512] fp32 gets 2 * ksteps
    per thread with the constant operands (window of fp16 2^-6)."""
    import torch
    _need(out, workgroups * 512, "out")
    wbytes = 0
    if mode & 2:
        if window is None:
            raise ValueError("mode bit 1 needs a window")
        wbytes = window.numel() * window.element_size()
    rc = _kloop_probe(_stream(stream), mode, workgroups, ksteps, _ptr(window, "window") if mode & 2 else None, wbytes,
                      _ptr(out, "out", torch.float32))
    _check(rc, "dit_gemm_kloop_probe")


def attention_step_probe(mode: int, workgroups: int, tiles: int, out, c2: float = 0.0, stream=None) -> None:
    """Calibration: the attention step on LDS-resident K / V (mode bit 0 ping-pong, bit 1 random
    operands); out [workgroups * 512] fp32 gets 48 * tiles (+ 16 with bit 0) per thread when c2 = 0
    and the operands are constant."""
    import torch
    _need(out, workgroups * 512, "out")
    _check(_attn_step_probe(_stream(stream), mode, workgroups, tiles, c2, _ptr(out, "out", torch.float32)),
           "dit_attention_step_probe")


def block_fp8_workspace_size(shape: Shape) -> int:
    c = shape.c_config()
    n = _wsize8(ctypes.byref(c))
    if n == 0:
        raise DitError(DIT_ERR_INVALID_ARG, "dit_block_fp8_workspace_size")
    return int(n)


def _stream_weights_fp8(shape: "Shape", w: dict, what: str) -> StreamWeightsFp8:
    """w: w_mod, qk_norm_w (16-bit) and, per product, codes (uint8) and scales (fp32): w_qkv / s_qkv,
    w_o / s_o, w_ffn_in / s_ffn_in, w_ffn_out / s_ffn_out."""
    import torch
    d, F, dc, hd = shape.d, shape.ffn_inner, shape.d_cond or shape.d, shape.head_dim
    s = StreamWeightsFp8()
    _need(w.get("w_mod"), 6 * d * dc, f"{what}.w_mod")
    _need(w.get("qk_norm_w"), 2 * hd, f"{what}.qk_norm_w")
    s.w_mod = _ptr(w.get("w_mod"), f"{what}.w_mod")
    s.qk_norm_w = _ptr(w.get("qk_norm_w"), f"{what}.qk_norm_w")
    for name, rows, k in (("qkv", 3 * d, d), ("o", d, d), ("ffn_in", 2 * F, d), ("ffn_out", d, F)):
        codes, scales = w.get("w_" + name), w.get("s_" + name)
        _need(codes, rows * k, f"{what}.w_{name}")
        _need(scales, rows, f"{what}.s_{name}")
        setattr(s, "w_" + name, _ptr(codes, f"{what}.w_{name}", torch.uint8))
        setattr(s, "s_" + name, _ptr(scales, f"{what}.s_{name}", torch.float32))
    return s


def block_forward_fp8(shape: Shape, txt: dict, img: dict, cond, pos, x_txt, x_img, y_txt, y_img, workspace,
                      stream=None) -> None:
    """Double-stream block with its four weight products on e4m3 codes (see include/dit.h)."""
    import torch
    c = shape.c_config()
    wt, wi = _stream_weights_fp8(shape, txt, "txt"), _stream_weights_fp8(shape, img, "img")
    _check_block_io(shape, cond, pos, ((x_txt, shape.n_txt, "x_txt"), (x_img, shape.n_img, "x_img"),
                                       (y_txt, shape.n_txt, "y_txt"), (y_img, shape.n_img, "y_img")))
    rc = _block8(ctypes.byref(c), ctypes.byref(wt), ctypes.byref(wi), _ptr(cond, "cond"),
                 _ptr(pos, "pos", torch.int32), _ptr(x_txt, "x_txt"), _ptr(x_img, "x_img"), _ptr(y_txt, "y_txt"),
                 _ptr(y_img, "y_img"), _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                 _stream(stream))
    _check(rc, "dit_block_forward_fp8")


def convert_bf16_to_f16(src, dst, stream=None) -> None:
    """dst (fp16) = src (bf16), elementwise: the weight format of Shape.gemm_w_dtype = DIT_F16."""
    import torch
    if not src.is_contiguous() or not dst.is_contiguous() or dst.numel() != src.numel():
        raise ValueError("src and dst must be contiguous tensors of the same size")
    rc = _cvt16(_stream(stream), _ptr(src, "src", torch.bfloat16), _ptr(dst, "dst", torch.float16), src.numel())
    _check(rc, "dit_convert_bf16_to_f16")


def single_block_fp8_workspace_size(shape: Shape) -> int:
    c = shape.c_config()
    n = _swsize8(ctypes.byref(c))
    if n == 0:
        raise DitError(DIT_ERR_INVALID_ARG, "dit_single_block_fp8_workspace_size")
    return int(n)


def single_block_forward_fp8(shape: Shape, w: dict, cond, pos, x, y, workspace, stream=None) -> None:
    """Single-stream block with its two weight products on e4m3 codes (see include/dit.h).  w: w_mod,
    qk_norm_w (16-bit), w_1 / s_1 and w_2 / s_2 (uint8 codes, fp32 row scales)."""
    import torch
    c = shape.c_config()
    d, F, dc, hd = shape.d, shape.ffn_inner, shape.d_cond or shape.d, shape.head_dim
    n = shape.n_txt + shape.n_img
    _need(w.get("w_mod"), 3 * d * dc, "w_mod")
    _need(w.get("qk_norm_w"), 2 * hd, "qk_norm_w")
    _need(w.get("w_1"), (3 * d + 2 * F) * d, "w_1")
    _need(w.get("s_1"), 3 * d + 2 * F, "s_1")
    _need(w.get("w_2"), d * (d + F), "w_2")
    _need(w.get("s_2"), d, "s_2")
    sw = SingleWeightsFp8()
    sw.w_mod, sw.qk_norm_w = _ptr(w.get("w_mod"), "w_mod"), _ptr(w.get("qk_norm_w"), "qk_norm_w")
    sw.w_1, sw.s_1 = _ptr(w.get("w_1"), "w_1", torch.uint8), _ptr(w.get("s_1"), "s_1", torch.float32)
    sw.w_2, sw.s_2 = _ptr(w.get("w_2"), "w_2", torch.uint8), _ptr(w.get("s_2"), "s_2", torch.float32)
    _need(cond, dc, "cond")
    _need(pos, n * len(shape.axes_dim), "pos")
    _need(x, n * d, "x")
    _need(y, n * d, "y")
    rc = _single8(ctypes.byref(c), ctypes.byref(sw), _ptr(cond, "cond"), _ptr(pos, "pos", torch.int32), _ptr(x, "x"),
                  _ptr(y, "y"), _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                  _stream(stream))
    _check(rc, "dit_single_block_forward_fp8")


def conv2d(x, weight, y, bias=None, stream=None) -> None:
    """NHWC 2-D convolution, stride 1, zero border: x [B, H, W, Cin], weight [Cout, KH, KW, Cin],
    y [B, H, W, Cout] (see include/dit.h)."""
    import torch
    B, H, W, cin = x.shape
    cout, kh, kw, cin2 = weight.shape
    if cin2 != cin or tuple(y.shape) != (B, H, W, cout):
        raise ValueError("shape mismatch between x, weight and y")
    for t, what in ((x, "x"), (weight, "weight"), (y, "y")):
        if not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous")
    if bias is not None:
        _need(bias, cout, "bias")
    rc = _conv(_dt(x), _stream(stream), _ptr(x, "x"), B, H, W, cin, _ptr(weight, "weight"), cout, kh, kw,
               _ptr(bias, "bias", torch.float32), _ptr(y, "y"), _dt(y))
    _check(rc, "dit_conv2d")


# --- kernel timing -----------------------------------------------------------------------------

def timing_begin(capacity: int) -> None:
    _check(_tbegin(capacity), "dit_timing_begin")


def timing_end() -> None:
    _tend()


def timing_read() -> dict:
    """{kernel launch-site name: (launches, total_ms)} for the launches recorded on this thread."""
    out = {}
    n = _tread(-1, None, 0, None, None)
    if n < 0:
        raise DitError(DIT_ERR_HIP, "dit_timing_read")
    for i in range(n):
        buf = ctypes.create_string_buffer(128)
        cnt = _i()
        ms = ctypes.c_double()
        _tread(i, buf, 128, ctypes.byref(cnt), ctypes.byref(ms))
        out[buf.value.decode()] = (cnt.value, ms.value)
    return out


def conv3d_causal(x, weight, y, bias=None, stream=None) -> None:
    """Causal 3-D convolution over frames: x [B, T, H, W, Cin], weight [Cout, KT, KH, KW, Cin],
    y [B, T, H, W, Cout] (see include/dit.h)."""
    import torch
    B, T, H, W, cin = x.shape
    cout, kt, kh, kw, cin2 = weight.shape
    if cin2 != cin or tuple(y.shape) != (B, T, H, W, cout):
        raise ValueError("shape mismatch between x, weight and y")
    for t, what in ((x, "x"), (weight, "weight"), (y, "y")):
        if not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous")
    if bias is not None:
        _need(bias, cout, "bias")
    rc = _conv3(_dt(x), _stream(stream), _ptr(x, "x"), B, T, H, W, cin, _ptr(weight, "weight"), cout, kt, kh, kw,
                _ptr(bias, "bias", torch.float32), _ptr(y, "y"), _dt(y))
    _check(rc, "dit_conv3d_causal")
