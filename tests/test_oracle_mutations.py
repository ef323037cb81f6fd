"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins in ``test_oracle_pins.py`` and ``test_oracle_fp8.py`` catch every one of them.

Each mutant is a textual edit of ``oracle/dit_oracle.py``, executed as a
separate module; the pin tests are then run against that module.  A mutant
that no pin fails would mean the oracle could carry that mistake unnoticed.
"""
import inspect
import os
import types

import pytest

from oracle import dit_oracle
import test_oracle_fp8 as fp8_pins
import test_oracle_pins as pins

PIN_MODULES = (pins, fp8_pins)

SRC_PATH = dit_oracle.__file__

MUTANTS = {
    "silu_sign": ("z / (1.0 + np.exp(-z))", "z / (1.0 + np.exp(z))"),
    "rms_eps_outside_sqrt": ("return x / np.sqrt(ms + eps)", "return x / (np.sqrt(ms) + eps)"),
    "rms_sum_not_mean": ("ms = np.mean(x * x, axis=-1, keepdims=True)",
                         "ms = np.sum(x * x, axis=-1, keepdims=True)"),
    "modulate_scale_without_one": ("(1.0 + np.asarray(scale, F64))", "np.asarray(scale, F64)"),
    "rope_sign_first": ("out[..., 0::2] = u * c - v * s", "out[..., 0::2] = u * c + v * s"),
    "rope_sign_second": ("out[..., 1::2] = u * s + v * c", "out[..., 1::2] = -u * s + v * c"),
    "rope_half_split_pairs": (
        "    u = x[..., 0::2]\n    v = x[..., 1::2]\n    out = np.empty_like(x)\n"
        "    out[..., 0::2] = u * c - v * s\n    out[..., 1::2] = u * s + v * c\n",
        "    hd = x.shape[-1] // 2\n    u = x[..., :hd]\n    v = x[..., hd:]\n    out = np.empty_like(x)\n"
        "    out[..., :hd] = u * c - v * s\n    out[..., hd:] = u * s + v * c\n"),
    "rope_freq_exponent": ("-2.0 * j / axis_dim", "-1.0 * j / axis_dim"),
    "rope_axis_order": ("pos[:, a:a + 1]", "pos[:, 3 - a:4 - a]"),
    "attn_scale": ("scale = 1.0 / np.sqrt(F64(head_dim))", "scale = 1.0 / F64(head_dim)"),
    "softmax_axis": ("return e / np.sum(e, axis=-1, keepdims=True)",
                     "return e / np.sum(e, axis=0, keepdims=True)"),
    "swiglu_halves": ("return silu(g) * u", "return silu(u) * g"),
    "gate1_chunk": ("h = x_r + m[s][2] *", "h = x_r + m[s][5] *"),
    "shift2_scale2_swapped": ("b = modulate(h, m[s][3], m[s][4]", "b = modulate(h, m[s][4], m[s][3]"),
    "ffn_residual_from_x": ("y = h + m[s][5]", "y = x_r + m[s][5]"),
    "qk_sets_swapped": ("np.where(np.arange(n) < n_first, 0, min(1, w.shape[0] - 1))",
                        "np.where(np.arange(n) < n_first, min(1, w.shape[0] - 1), 0)"),
    "qk_weights_swapped": ("for which, t in ((0, q), (1, k)):", "for which, t in ((1, q), (0, k)):"),
    "single_ffn_rows": ("gu = _product(a[r], w1[3 * d:], fp8)", "gu = _product(a[r], w1[2 * d:2 * d + 2 * F], fp8)"),
    "fp8_product_drops_weight_scales": ("return linear_fp8(xq, sx, wq, sw)", "return linear_fp8(xq, sx, wq, np.ones_like(sw))"),
    "fp8_attn_k_scale_for_v": ("out[:, c] = (wq @ (sv[h] * v[:, c]))", "out[:, c] = (wq @ (sk[h] * v[:, c]))"),
    "fp8_attn_q_scale_per_head": ("s = (sq[:, h:h + 1] * q[:, c])", "s = (sq[0, h] * q[:, c])"),
    "fp8_attn_no_softmax_scale": ("@ (sk[h] * k[:, c]).T * scale", "@ (sk[h] * k[:, c]).T"),
    "fp8_attn_normalise_rounded": ("/ np.sum(w, axis=1, keepdims=True)", "/ np.sum(wq, axis=1, keepdims=True)"),
    "fp8_attn_k_bound_head_dim_64": ("K_BOUND_PER_WEIGHT = np.float32(math.sqrt(128.0) / E4M3_MAX)",
                                     "K_BOUND_PER_WEIGHT = np.float32(math.sqrt(64.0) / E4M3_MAX)"),
    "fp8_attn_v_scale_per_token": ("vmax = np.max(np.abs(v32).reshape(n, H, D), axis=(0, 2))",
                                   "vmax = np.max(np.abs(v32).reshape(n, H, D), axis=(1, 2))[:H]"),
    "single_o_f_order": ("np.concatenate([o, f], axis=1)", "np.concatenate([f, o], axis=1)"),
    "v_from_k_block": ('v = np.concatenate([qkv["txt"][:, 2 * d:], qkv["img"][:, 2 * d:]], axis=0)',
                       'v = np.concatenate([qkv["txt"][:, d:2 * d], qkv["img"][:, d:2 * d]], axis=0)'),
    "attention_not_joint": (
        "o = joint_attention(q, k, v, H, D, q_rows=q_rows)",
        "o = np.concatenate([joint_attention(q[:nt], k[:nt], v[:nt], H, D, q_rows=rows['txt']),"
        " joint_attention(q[nt:], k[nt:], v[nt:], H, D, q_rows=rows['img'])])"),
}


def _pin_tests():
    out = []
    for mod in PIN_MODULES:
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if name.startswith("test_") and fn.__module__ == mod.__name__:
                out.append((f"{mod.__name__}.{name}", fn))
    return out


def _run_pins(module):
    """Run every pin against ``module``; return the names of the failing pins."""
    failed = []
    saved = [m.o for m in PIN_MODULES]
    for m in PIN_MODULES:
        m.o = module
    try:
        cfg = pins.tiny_cfg()
        fixture_val = (cfg, pins.di.double_block_inputs(cfg, seed=3, qk_norm="random"))
        for name, fn in _pin_tests():
            params = inspect.signature(fn).parameters
            args = [fixture_val] if "tiny_inputs" in params else []
            try:
                fn(*args)
            except AssertionError:
                failed.append(name)
            except Exception:       # a mutant may also break shapes: that counts as caught
                failed.append(name)
    finally:
        for m, o in zip(PIN_MODULES, saved):
            m.o = o
    return failed


def _load_mutant(old, new):
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique / missing: {old!r}"
    mod = types.ModuleType("dit_oracle_mutant")
    mod.__file__ = SRC_PATH
    exec(compile(src.replace(old, new), SRC_PATH + ".mutant", "exec"), mod.__dict__)
    return mod


def test_unmutated_oracle_passes_all_pins():
    assert _run_pins(dit_oracle) == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant):
    old, new = MUTANTS[mutant]
    failed = _run_pins(_load_mutant(old, new))
    assert failed, f"mutant {mutant} passed every pin"
