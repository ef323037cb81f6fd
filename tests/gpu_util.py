"""Helpers for the GPU parity tests: move the generator's storage bits to the GPU,
bring results back as float64, and the parity metric max|gpu - oracle| / RMS(oracle)."""
import sys

import numpy as np
import torch

import dit_inputs as di


def dev(a, dtype: str):
    """numpy storage (bf16 bits as uint16, float32, int32) -> cuda tensor with the same bits."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32, copy=False)).cuda()
    if dtype == "f16":
        return torch.from_numpy(a.astype(np.float16, copy=False)).cuda()
    if dtype == "i32":
        return torch.from_numpy(a.astype(np.int32, copy=False)).cuda()
    raise ValueError(dtype)


def host(t) -> np.ndarray:
    """cuda tensor -> float64 numpy (exact widening)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def tdtype(dtype: str):
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]


def metric(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - oracle| / RMS(oracle)."""
    rms = float(np.sqrt(np.mean(np.asarray(ref, np.float64) ** 2)))
    return float(np.max(np.abs(np.asarray(gpu, np.float64) - ref))) / rms


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the storage type's values at |x| (bf16: 8 significant bits; fp16: 11, with
    the subnormal spacing 2^-24 below 2^-14; fp32: 24)."""
    ax = np.abs(np.asarray(x, np.float64))
    if dtype == "bf16":
        return bf16_ulp(ax)
    if dtype == "f16":
        return 2.0 ** (np.floor(np.log2(np.maximum(ax, 2.0 ** -14))) - 10)
    return 2.0 ** (np.floor(np.log2(np.maximum(ax, 2.0 ** -126))) - 23)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


PRODUCT_WEIGHTS = ("w_qkv", "w_o", "w_ffn_in", "w_ffn_out", "w_1", "w_2")


def upload_stream_weights(w: dict, dtype: str, f16_products: bool = False) -> dict:
    """Weights to the GPU; f16_products: the matrix-product weights as fp16 copies of the bf16
    weights made by dit_convert_bf16_to_f16 (the block's gemm_w_dtype = DIT_F16 format)."""
    out = {k: dev(v, dtype) for k, v in w.items()}
    if f16_products:
        import attention_dit_block_amd as dit
        for k in PRODUCT_WEIGHTS:
            if k in out:
                f = torch.empty(out[k].shape, dtype=torch.float16, device="cuda")
                dit.convert_bf16_to_f16(out[k], f)
                out[k] = f
    return out


def shape_of(cfg: di.BlockConfig, mod, x_dtype=None, y_dtype=None, n_txt=None, n_img=None, act_dtype=None):
    """attention_dit_block_amd.Shape for a generator config."""
    dt = mod.DIT_BF16 if cfg.dtype == "bf16" else mod.DIT_F32
    return mod.Shape(dtype=dt, act_dtype=act_dtype, d=cfg.d, n_heads=cfg.n_heads, ffn_inner=cfg.ffn_inner,
                     n_txt=cfg.n_txt if n_txt is None else n_txt, n_img=cfg.n_img if n_img is None else n_img,
                     d_cond=cfg.dc, x_dtype=dt if x_dtype is None else x_dtype,
                     y_dtype=mod.DIT_F32 if y_dtype is None else y_dtype, eps=cfg.eps, eps_qk=cfg.eps_qk,
                     theta=cfg.theta, axes_dim=cfg.axes_dim)
