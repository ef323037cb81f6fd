"""Seeded synthetic inputs for the FLUX-style joint text+image DiT block.

This module is the only code shared by the fp64 oracle (``oracle/``) and the
HIP path (``attention_dit_block_amd``).  It draws numbers and lays them out;
it holds none of the block's arithmetic.

Workload shapes follow the DiT block the "CUDA codepath !" thread (antirez/
iris.c issue #15) describes: a FLUX Klein transformer whose block is AdaLN +
custom 4-axis RoPE + joint text/image attention (GGML update, "bottom line"),
with RoPE axes [32, 32, 32, 32] and separate text / image positions (GGML
update, item 3).  A 1024x1024 image (the thread's opening benchmark) at a
16x pixel-to-token stride is a 64x64 token grid.

Recipe (every tensor):
  * ``np.random.default_rng([seed, block, stream, tensor_id])`` draws float32
    standard normals;
  * activations and the conditioning vector are N(0, 1); Linear weights are
    N(0, 0.02^2); QK-norm weights are ones (or 1 + 0.1 N(0,1) on request);
  * bf16 workloads round the float32 draw to bf16 with round-to-nearest-even
    and keep the raw 16-bit patterns (``uint16``); the oracle and the GPU both
    receive exactly these bits.

Positions (int32, 4 axes): text token n -> (0, 0, 0, n); image token at grid
row r, column c (row-major raster, token index n_txt + r*W + c) -> (0, r, c, 0).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os as _os
from dataclasses import dataclass, replace
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "BlockConfig", "CONFIGS", "config_by_name", "positions",
    "bf16_bits_from_f32", "f32_from_bf16_bits",
    "draw", "double_block_inputs", "single_block_inputs",
    "activation_inputs", "TENSOR_IDS", "fp8_attention_inputs",
]


@dataclass(frozen=True)
class BlockConfig:
    """Shape of one workload.  ``dtype`` is 'f32' or 'bf16' (storage type)."""
    name: str
    dtype: str
    d: int                      # hidden size
    n_heads: int
    ffn_inner: int              # F, SwiGLU inner width (3d)
    n_txt: int
    grid_h: int
    grid_w: int
    head_dim: int = 128
    d_cond: int = 0             # 0 -> d
    n_double: int = 1
    n_single: int = 0
    eps: float = 1e-6
    eps_qk: float = 1e-6
    theta: float = 1e4
    axes_dim: Tuple[int, int, int, int] = (32, 32, 32, 32)

    @property
    def n_img(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def n_tok(self) -> int:
        return self.n_txt + self.n_img

    @property
    def dc(self) -> int:
        return self.d_cond if self.d_cond else self.d

    def with_(self, **kw) -> "BlockConfig":
        return replace(self, **kw)

    def flops_double(self) -> float:
        """Algorithmic flops of one double block: GEMMs 26 N d^2 (with F=3d)
        plus attention QK^T and PV, 4 N^2 d (2 flop per multiply-add)."""
        n, d, f = self.n_tok, self.d, self.ffn_inner
        gemm = 2.0 * n * d * (3 * d) + 2.0 * n * d * d + 2.0 * n * d * (2 * f) + 2.0 * n * f * d
        return gemm + 4.0 * n * n * d

    def flops_single(self) -> float:
        n, d, f = self.n_tok, self.d, self.ffn_inner
        gemm = 2.0 * n * d * (3 * d + 2 * f) + 2.0 * n * (d + f) * d
        return gemm + 4.0 * n * n * d

    def flops_step(self) -> float:
        return self.n_double * self.flops_double() + self.n_single * self.flops_single()


CONFIGS = (
    BlockConfig("c0_f32_d256_t16_i64", "f32", d=256, n_heads=2, ffn_inner=768,
                n_txt=16, grid_h=8, grid_w=8),
    BlockConfig("c1_bf16_d3072_t512_i1024", "bf16", d=3072, n_heads=24, ffn_inner=9216,
                n_txt=512, grid_h=32, grid_w=32),
    BlockConfig("c2_bf16_d3072_t512_i4096", "bf16", d=3072, n_heads=24, ffn_inner=9216,
                n_txt=512, grid_h=64, grid_w=64),
    BlockConfig("c3_bf16_step_5x2_20x1_t512_i4096", "bf16", d=3072, n_heads=24, ffn_inner=9216,
                n_txt=512, grid_h=64, grid_w=64, n_double=5, n_single=20),
    BlockConfig("c4_bf16_d3072_t512_i16384", "bf16", d=3072, n_heads=24, ffn_inner=9216,
                n_txt=512, grid_h=128, grid_w=128),
)


def config_by_name(prefix: str) -> BlockConfig:
    for c in CONFIGS:
        if c.name.startswith(prefix):
            return c
    raise KeyError(prefix)


def positions(n_txt: int, grid_h: int, grid_w: int) -> np.ndarray:
    """int32 [n_txt + grid_h*grid_w, 4]: text (0,0,0,n), image (0,r,c,0)."""
    n = n_txt + grid_h * grid_w
    pos = np.zeros((n, 4), dtype=np.int32)
    pos[:n_txt, 3] = np.arange(n_txt, dtype=np.int32)
    r, c = np.meshgrid(np.arange(grid_h, dtype=np.int32), np.arange(grid_w, dtype=np.int32),
                       indexing="ij")
    pos[n_txt:, 1] = r.reshape(-1)
    pos[n_txt:, 2] = c.reshape(-1)
    return pos


# --- bf16 bit patterns (storage format only) --------------------------------

def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even) and return uint16 bits.
    NaN inputs are not produced by the generator and are not handled."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32 (a format change)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --- tensors -----------------------------------------------------------------

# Fixed ids so that every tensor has its own stream of draws.
TENSOR_IDS: Dict[str, int] = {
    "cond": 1, "x_txt": 2, "x_img": 3, "x": 4,
    "w_mod": 10, "w_qkv": 11, "qk_norm_w": 12, "w_o": 13, "w_ffn_in": 14, "w_ffn_out": 15,
    "w_1": 16, "w_2": 17,
    "q": 20, "k": 21, "v": 22, "q_scale": 23, "k_scale": 24, "v_scale": 25,
    "w_t_in": 30, "w_t_out": 31, "w_g_in": 32, "w_g_out": 33, "w_patch": 34, "latent": 35,
    "w_final_mod": 36, "w_final_out": 37, "w_mod_shared": 38,
}
STREAM_IDS = {"txt": 0, "img": 1, "single": 2, "none": 3}


def draw(shape, std: float, dtype: str, seed: int, name: str, block: int = 0,
         stream: str = "none") -> np.ndarray:
    """N(0, std^2) draw.  Returns float32 ('f32'), bf16 bits as uint16 ('bf16') or float16
    ('f16', rounded to nearest even)."""
    rng = np.random.default_rng([int(seed), int(block), STREAM_IDS[stream], TENSOR_IDS[name]])
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype == "f32":
        return a
    if dtype == "bf16":
        return bf16_bits_from_f32(a)
    if dtype == "f16":
        return a.astype(np.float16)      # round to nearest even
    raise ValueError(dtype)


def _qk_norm_weights(cfg: BlockConfig, seed: int, block: int, stream: str, mode: str) -> np.ndarray:
    """[2 (q, k)][head_dim]."""
    if mode == "ones":
        a = np.ones((2, cfg.head_dim), dtype=np.float32)
    elif mode == "random":
        rng = np.random.default_rng([int(seed), int(block), STREAM_IDS[stream], TENSOR_IDS["qk_norm_w"]])
        a = (1.0 + 0.1 * rng.standard_normal(size=(2, cfg.head_dim), dtype=np.float32)).astype(np.float32)
    else:
        raise ValueError(mode)
    return a if cfg.dtype == "f32" else bf16_bits_from_f32(a)


_POOL = None


def _pool():
    """Thread pool for independent draws (numpy's generators release the GIL)."""
    global _POOL
    if _POOL is None:
        n = min(16, max(1, len(_os.sched_getaffinity(0))))
        _POOL = _cf.ThreadPoolExecutor(max_workers=n)
    return _POOL


def _draw_many(specs) -> Dict[str, np.ndarray]:
    """specs: {key: (shape, std, dtype, seed, name, block, stream)} drawn concurrently."""
    futs = {k: _pool().submit(draw, *v) for k, v in specs.items()}
    return {k: f.result() for k, f in futs.items()}


def stream_weights(cfg: BlockConfig, seed: int, block: int, stream: str,
                   qk_norm: str = "ones", std: float = 0.02) -> Dict[str, np.ndarray]:
    """Weights of one stream of a double block; Linear weights are [out, in]."""
    d, f, dc, t = cfg.d, cfg.ffn_inner, cfg.dc, cfg.dtype
    out = _draw_many({
        "w_mod": ((6 * d, dc), std, t, seed, "w_mod", block, stream),
        "w_qkv": ((3 * d, d), std, t, seed, "w_qkv", block, stream),
        "w_o": ((d, d), std, t, seed, "w_o", block, stream),
        "w_ffn_in": ((2 * f, d), std, t, seed, "w_ffn_in", block, stream),
        "w_ffn_out": ((d, f), std, t, seed, "w_ffn_out", block, stream),
    })
    out["qk_norm_w"] = _qk_norm_weights(cfg, seed, block, stream, qk_norm)
    return out


def single_weights(cfg: BlockConfig, seed: int, block: int, qk_norm: str = "ones",
                   std: float = 0.02) -> Dict[str, np.ndarray]:
    """Weights of a single-stream block: W1 rows [q|k|v|gate|up], W2 input [O|f]."""
    d, f, dc, t = cfg.d, cfg.ffn_inner, cfg.dc, cfg.dtype
    out = _draw_many({
        "w_mod": ((3 * d, dc), std, t, seed, "w_mod", block, "single"),
        "w_1": ((3 * d + 2 * f, d), std, t, seed, "w_1", block, "single"),
        "w_2": ((d, d + f), std, t, seed, "w_2", block, "single"),
    })
    out["qk_norm_w"] = _qk_norm_weights(cfg, seed, block, "single", qk_norm)
    return out


def activation_inputs(cfg: BlockConfig, seed: int) -> Dict[str, np.ndarray]:
    """cond [d_c], x_txt [n_txt, d], x_img [n_img, d], pos [n_tok, 4]."""
    t = cfg.dtype
    return {
        "cond": draw((cfg.dc,), 1.0, t, seed, "cond"),
        "x_txt": draw((cfg.n_txt, cfg.d), 1.0, t, seed, "x_txt"),
        "x_img": draw((cfg.n_img, cfg.d), 1.0, t, seed, "x_img"),
        "pos": positions(cfg.n_txt, cfg.grid_h, cfg.grid_w),
    }


def double_block_inputs(cfg: BlockConfig, seed: int = 0, block: int = 0,
                        qk_norm: str = "ones") -> Dict[str, object]:
    out: Dict[str, object] = dict(activation_inputs(cfg, seed))
    out["txt"] = stream_weights(cfg, seed, block, "txt", qk_norm)
    out["img"] = stream_weights(cfg, seed, block, "img", qk_norm)
    return out


def single_block_inputs(cfg: BlockConfig, seed: int = 0, block: int = 0,
                        qk_norm: str = "ones") -> Dict[str, object]:
    act = activation_inputs(cfg, seed)
    t = cfg.dtype
    x = draw((cfg.n_tok, cfg.d), 1.0, t, seed, "x", block, "single")
    return {"cond": act["cond"], "x": x, "pos": act["pos"],
            "w": single_weights(cfg, seed, block, qk_norm)}


def qkv_inputs(cfg: BlockConfig, seed: int = 0, std: float = 1.0) -> Dict[str, np.ndarray]:
    """Standalone q, k, v [n_tok, d] for the attention and QK-norm/RoPE calls."""
    t = cfg.dtype
    shape = (cfg.n_tok, cfg.d)
    return {"q": draw(shape, std, t, seed, "q"), "k": draw(shape, std, t, seed, "k"),
            "v": draw(shape, std, t, seed, "v")}


def fp8_attention_inputs(n_tok: int, n_heads: int, head_dim: int = 128, seed: int = 0) -> Dict[str, np.ndarray]:
    """Operands of the fp8 attention call, drawn directly as e4m3 codes (no rounding involved).
    q8, k8, v8 [n_tok, n_heads*head_dim] uint8: magnitude codes uniform over 0x30 .. 0x77 (values
    0.5 .. 240, log-uniformly spread, rms about 68) with a random sign bit, 1% of them zeros.
    Scales float32: sq [n_tok, n_heads] = f_h * U(0.5, 1.5) / 68 with a per-head sharpness
    f_h ~ U(0.5, 2.5); sk [n_heads] and sv [n_heads] = U(0.8, 1.2) / 68.  The scaled scores
    q.k / sqrt(head_dim) then have a standard deviation of about f_h (diffuse to peaked rows)."""
    shape = (n_tok, n_heads * head_dim)
    out = {}
    for name in ("q", "k", "v"):
        rng = np.random.default_rng([int(seed), 0, STREAM_IDS["none"], TENSOR_IDS[name], 8])
        mag = rng.integers(0x30, 0x78, size=shape, dtype=np.uint8)
        sign = (rng.integers(0, 2, size=shape, dtype=np.uint8) << 7).astype(np.uint8)
        codes = (mag | sign).astype(np.uint8)
        codes[rng.random(shape) < 0.01] = 0
        out[name + "8"] = codes
    rng = np.random.default_rng([int(seed), 0, STREAM_IDS["none"], TENSOR_IDS["q_scale"], 8])
    sharp = rng.uniform(0.5, 2.5, n_heads)
    out["sq"] = (sharp[None, :] * rng.uniform(0.5, 1.5, (n_tok, n_heads)) / 68.0).astype(np.float32)
    rng = np.random.default_rng([int(seed), 0, STREAM_IDS["none"], TENSOR_IDS["k_scale"], 8])
    out["sk"] = (rng.uniform(0.8, 1.2, n_heads) / 68.0).astype(np.float32)
    rng = np.random.default_rng([int(seed), 0, STREAM_IDS["none"], TENSOR_IDS["v_scale"], 8])
    out["sv"] = (rng.uniform(0.8, 1.2, n_heads) / 68.0).astype(np.float32)
    return out


def edge_inputs(cfg: BlockConfig, seed: int = 0, freq_dim: int = 256, patch: int = 64) -> Dict[str, np.ndarray]:
    """Inputs of the layers either side of the block stack: image latents in 2x2 patches of 16
    channels [n_img, patch] ~ N(0, 1), and weights ~ N(0, 0.02^2) in the workload's type:
    patch embedding [d, patch], timestep and guidance MLPs [d, freq_dim] + [d, d], final
    layer modulation [2d, d_cond] and projection [patch, d]."""
    t, d = cfg.dtype, cfg.d
    return {
        "latent": draw((cfg.n_img, patch), 1.0, t, seed, "latent"),
        "w_patch": draw((d, patch), 0.02, t, seed, "w_patch"),
        "w_t_in": draw((d, freq_dim), 0.02, t, seed, "w_t_in"),
        "w_t_out": draw((d, d), 0.02, t, seed, "w_t_out"),
        "w_g_in": draw((d, freq_dim), 0.02, t, seed, "w_g_in"),
        "w_g_out": draw((d, d), 0.02, t, seed, "w_g_out"),
        "w_final_mod": draw((2 * d, cfg.dc), 0.02, t, seed, "w_final_mod"),
        "w_final_out": draw((patch, d), 0.02, t, seed, "w_final_out"),
        "cond": draw((cfg.dc,), 1.0, t, seed, "cond"),
    }


def shared_mod_weights(cfg: BlockConfig, seed: int = 0) -> Dict[str, np.ndarray]:
    """One AdaLN weight set per block kind, shared by all blocks of a step: text [6d, d_cond],
    image [6d, d_cond], single [3d, d_cond], ~ N(0, 0.02^2)."""
    t, d = cfg.dtype, cfg.d
    return {"txt": draw((6 * d, cfg.dc), 0.02, t, seed, "w_mod_shared", stream="txt"),
            "img": draw((6 * d, cfg.dc), 0.02, t, seed, "w_mod_shared", stream="img"),
            "single": draw((3 * d, cfg.dc), 0.02, t, seed, "w_mod_shared", stream="single")}
