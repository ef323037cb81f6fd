"""The C-ABI library loads, exports every symbol include/dit.h declares, and rejects
invalid arguments on the host with the documented status, an error text and no
launch (CPU only: every call here fails validation before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    import importlib.util
    path = os.path.join(ROOT, "attention_dit_block_amd", "build.py")
    spec = importlib.util.spec_from_file_location("dit_build", path)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.fixture(scope="module")
def dit():
    b = _build_module()
    if not os.path.exists(b.LIB):
        b.build()
    import attention_dit_block_amd as m
    return m


def declared_functions():
    with open(os.path.join(ROOT, "include", "dit.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("dit_adaln_modulate", "dit_qk_rmsnorm_rope", "dit_joint_attention", "dit_block_forward",
                     "dit_single_block_forward", "dit_block_workspace_size", "dit_last_error",
                     "dit_launch_count", "dit_abi_version"):
        assert required in names


def test_library_exports_every_declared_symbol(dit):
    lib = ctypes.CDLL(dit.library_path)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(dit.EXPORTED) == declared_functions()


def test_abi_version(dit):
    assert dit.abi_version() == 1


def _cfg(dit, **kw):
    s = dit.Shape(dtype=dit.DIT_BF16, d=3072, n_heads=24, ffn_inner=9216, n_txt=512, n_img=4096)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def test_workspace_size_matches_plan(dit):
    s = _cfg(dit)
    n, d, F = 4608, 3072, 9216

    def up(x):
        return (x + 255) // 256 * 256
    # the 4-byte range-flag word (first, 256-byte slot), then the buffers of the block
    # ... and the (cos, sin) table of the 64 rotation angles per token for the fused QK RMSNorm + RoPE
    want = (up(4) + up(2 * 6 * d * 4) + up(n * d * 2) + up(n * 3 * d * 2) + up(n * d * 2) + up(n * d * 4) +
            up(n * F * 2) + up(n * 64 * 2 * 4))
    assert dit.block_workspace_size(s) == want
    want1 = up(4) + up(3 * d * 4) + up(n * d * 2) + up(n * 3 * d * 2) + up(n * (d + F) * 2)
    assert dit.block_workspace_size(s, single_stream=True) == want1


@pytest.mark.parametrize("kw, status, text", [
    (dict(head_dim=64, d=64 * 24), "DIT_ERR_UNSUPPORTED", "head_dim"),
    (dict(d=3000), "DIT_ERR_INVALID_ARG", "n_heads"),
    (dict(ffn_inner=9200), "DIT_ERR_INVALID_ARG", "ffn_inner"),
    (dict(ffn_inner=(1 << 20) + 128), "DIT_ERR_UNSUPPORTED", "ffn_inner"),
    (dict(n_txt=0, n_img=0), "DIT_ERR_INVALID_ARG", "token"),
    (dict(n_txt=-1), "DIT_ERR_INVALID_ARG", "n_txt"),
    (dict(axes_dim=(32, 32, 32, 30)), "DIT_ERR_INVALID_ARG", "sum"),
    (dict(axes_dim=(32, 32, 31, 33)), "DIT_ERR_INVALID_ARG", "even"),
    (dict(theta=0.0), "DIT_ERR_INVALID_ARG", "theta"),
    (dict(d_cond=3071), "DIT_ERR_INVALID_ARG", "d_cond"),
    (dict(dtype=0, y_dtype=1), "DIT_ERR_UNSUPPORTED", "fp32"),
    (dict(eps=-1.0), "DIT_ERR_INVALID_ARG", "eps"),
])
def test_invalid_config_rejected(dit, kw, status, text):
    s = _cfg(dit, **kw)
    with pytest.raises(dit.DitError) as e:
        dit.block_workspace_size(s)
    assert text in str(e.value)


class FakeDev:
    """Stands in for a device tensor: the calls below fail validation before any use."""
    is_cuda = True

    def __init__(self, addr, shape=(16, 3072), stride=None, dtype=None, esize=2):
        import torch
        self.addr, self.shape = addr, shape
        self._stride = stride or (shape[-1], 1)
        self.dtype = dtype or torch.bfloat16
        self._es = esize

    def data_ptr(self):
        return self.addr

    def dim(self):
        return len(self.shape)

    def stride(self, i):
        return self._stride[i]

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def element_size(self):
        return self._es

    def is_contiguous(self):
        return True


def _no_launch(dit, fn):
    before = dit.launch_count()
    with pytest.raises(dit.DitError) as e:
        fn()
    assert dit.launch_count() == before
    assert dit.last_error()
    return e.value


def test_attention_validation(dit):
    import torch
    q = FakeDev(0x100000)
    o = FakeDev(0x900000)
    # misaligned pointer
    e = _no_launch(dit, lambda: dit.joint_attention(FakeDev(0x100008), q, q, o, n_heads=24, stream=FakeStream()))
    assert e.status == "DIT_ERR_INVALID_ARG" and "aligned" in str(e)
    # head_dim other than 128
    e = _no_launch(dit, lambda: dit.joint_attention(q, q, q, o, n_heads=48, head_dim=64, stream=FakeStream()))
    assert e.status == "DIT_ERR_UNSUPPORTED"
    # row stride smaller than the width
    e = _no_launch(dit, lambda: dit.joint_attention(FakeDev(0x100000, stride=(1024, 1)), q, q, o, n_heads=24,
                                                    stream=FakeStream()))
    assert "smaller than the row width" in str(e)
    # output overlapping the input
    e = _no_launch(dit, lambda: dit.joint_attention(q, q, q, FakeDev(0x100000 + 4096), n_heads=24,
                                                    stream=FakeStream()))
    assert "overlaps" in str(e)
    # stride not a multiple of 16 bytes
    e = _no_launch(dit, lambda: dit.joint_attention(FakeDev(0x100000, stride=(3073, 1)), q, q, o, n_heads=24,
                                                    stream=FakeStream()))
    assert "16 bytes" in str(e)


class FakeStream:
    cuda_stream = 0


def test_rope_validation(dit):
    import torch
    q = FakeDev(0x100000, stride=(9216, 1))
    k = FakeDev(0x100000 + 3072 * 2, stride=(9216, 1))
    pos = FakeDev(0x800000, shape=(16, 8), dtype=torch.int32, esize=4)
    w = FakeDev(0x700000, shape=(2, 2, 128))
    e = _no_launch(dit, lambda: dit.qk_rmsnorm_rope(q, k, 24, w, 16, pos, axes_dim=(32, 32, 32, 34),
                                                    stream=FakeStream()))
    assert "sum" in str(e)
    e = _no_launch(dit, lambda: dit.qk_rmsnorm_rope(q, k, 24, w, 16, pos, axes_dim=(32, 32, 32, 32, 0),
                                                    stream=FakeStream()))
    assert e.status == "DIT_ERR_UNSUPPORTED"
    # q and k overlapping columns of one buffer
    k2 = FakeDev(0x100000 + 3000 * 2, stride=(9216, 1))
    e = _no_launch(dit, lambda: dit.qk_rmsnorm_rope(q, k2, 24, w, 16, pos, stream=FakeStream()))
    assert "overlap" in str(e)


def test_adaln_validation(dit):
    import torch
    cond = FakeDev(0x100000, shape=(3072,))
    w = FakeDev(0x200000, shape=(1 << 27,))
    mod = FakeDev(0x300000, shape=(1 << 16,), dtype=torch.float32, esize=4)
    x = FakeDev(0x400000, shape=(16, 3072))
    e = _no_launch(dit, lambda: dit.adaln_modulate(cond, w, 6, 3072, mod, x=x, x_out=FakeDev(0x400000 + 64),
                                                   stream=FakeStream()))
    assert "overlaps" in str(e)
    e = _no_launch(dit, lambda: dit.adaln_modulate(cond, w, 6, 3072, mod, x=x, x_out=FakeDev(0x900000),
                                                   shift_chunk=6, stream=FakeStream()))
    assert "chunk" in str(e)
    e = _no_launch(dit, lambda: dit.adaln_modulate(cond, w, 6, 3076, mod, stream=FakeStream()))
    assert "multiple of 8" in str(e)


def test_block_validation_workspace_and_alias(dit):
    import torch
    s = _cfg(dit, n_txt=16, n_img=64, d=256, n_heads=2, ffn_inner=768)
    need = dit.block_workspace_size(s)
    wts = {n: FakeDev(0x1000000 * (i + 1), shape=(1 << 20,)) for i, n in enumerate(
        ("w_mod", "w_qkv", "qk_norm_w", "w_o", "w_ffn_in", "w_ffn_out"))}
    cond = FakeDev(0x10000000, shape=(256,))
    pos = FakeDev(0x11000000, shape=(80, 4), dtype=torch.int32, esize=4)
    xt, xi = FakeDev(0x12000000, shape=(16, 256)), FakeDev(0x13000000, shape=(64, 256))
    yt, yi = FakeDev(0x14000000, shape=(16, 256)), FakeDev(0x15000000, shape=(64, 256))
    small = FakeDev(0x20000000, shape=(need - 256,), dtype=torch.uint8, esize=1)
    e = _no_launch(dit, lambda: dit.block_forward(s, wts, wts, cond, pos, xt, xi, yt, yi, small,
                                                  stream=FakeStream()))
    assert e.status == "DIT_ERR_WORKSPACE"
    ws = FakeDev(0x20000000, shape=(need,), dtype=torch.uint8, esize=1)
    # y (fp32) partly overlapping x (bf16): not an exact alias of the same dtype
    e = _no_launch(dit, lambda: dit.block_forward(s, wts, wts, cond, pos, xt, xi, FakeDev(0x12000000 + 256), yi,
                                                  ws, stream=FakeStream()))
    assert "alias" in str(e)
    bad = dict(wts)
    bad["w_o"] = FakeDev(0x1000004, shape=(1 << 20,))
    e = _no_launch(dit, lambda: dit.block_forward(s, wts, bad, cond, pos, xt, xi, yt, yi, ws, stream=FakeStream()))
    assert "img.w_o" in str(e)


def test_host_tensor_refused_by_binding(dit):
    import torch
    q = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dit.joint_attention(q, q, q, q, n_heads=1, stream=FakeStream())


def test_undersized_tensor_refused_by_binding(dit):
    # the binding refuses buffers smaller than the call would touch
    q = FakeDev(0x100000, shape=(16, 3072))
    o = FakeDev(0x900000, shape=(15, 3072))
    with pytest.raises(ValueError):
        dit.joint_attention(q, q, q, o, n_heads=24, stream=FakeStream())
    s = _cfg(dit, n_txt=16, n_img=64, d=256, n_heads=2, ffn_inner=768)
    wts = {n: FakeDev(0x1000000 * (i + 1), shape=(1 << 20,)) for i, n in enumerate(
        ("w_mod", "w_qkv", "qk_norm_w", "w_o", "w_ffn_in", "w_ffn_out"))}
    wts["w_ffn_in"] = FakeDev(0x7000000, shape=(2 * 768 * 256 - 1,))
    x = FakeDev(0x12000000, shape=(80, 256))
    with pytest.raises(ValueError):
        dit.block_forward(s, wts, wts, x, x, x, x, x, x, x, stream=FakeStream())


def test_step_validation_checks_every_block_first(dit):
    """dit_step_forward validates all blocks' arguments before its first launch."""
    import torch
    s = _cfg(dit, n_txt=16, n_img=64, d=256, n_heads=2, ffn_inner=768)
    need = dit.step_workspace_size(s, 2, 3)
    assert need >= dit.block_workspace_size(s) and need >= dit.block_workspace_size(s, single_stream=True)
    wts = {n: FakeDev(0x1000000 * (i + 1), shape=(1 << 20,)) for i, n in enumerate(
        ("w_mod", "w_qkv", "qk_norm_w", "w_o", "w_ffn_in", "w_ffn_out"))}
    sw = {n: FakeDev(0x8000000 * (i + 1), shape=(1 << 20,)) for i, n in enumerate(("w_mod", "w_1", "qk_norm_w", "w_2"))}
    cond = FakeDev(0x10000000, shape=(256,))
    pos = FakeDev(0x11000000, shape=(80, 4), dtype=torch.int32, esize=4)
    xt, xi = FakeDev(0x12000000, shape=(16, 256)), FakeDev(0x13000000, shape=(64, 256))
    y = FakeDev(0x14000000, shape=(80, 256), dtype=torch.float32, esize=4)
    ws = FakeDev(0x40000000, shape=(need,), dtype=torch.uint8, esize=1)
    run = lambda txt, img, single, **kw: dit.step_forward(s, txt, img, single, cond, pos, kw.get("xt", xt),
                                                          kw.get("xi", xi), y, kw.get("ws", ws), stream=FakeStream())
    # a misaligned weight in the last single-stream block: nothing of the earlier blocks launches
    bad = dict(sw)
    bad["w_1"] = FakeDev(0x8000000 * 2 + 8, shape=(1 << 20,))
    e = _no_launch(dit, lambda: run([wts, wts], [wts, wts], [sw, sw, bad]))
    assert "single[2].w_1" in str(e)
    bad_img = dict(wts)
    bad_img["w_qkv"] = FakeDev(0x1000000 * 2 + 4, shape=(1 << 20,))
    e = _no_launch(dit, lambda: run([wts, wts], [wts, bad_img], [sw]))
    assert "img[1].w_qkv" in str(e)
    e = _no_launch(dit, lambda: run([], [], []))
    assert e.status == "DIT_ERR_INVALID_ARG"
    small = FakeDev(0x40000000, shape=(need - 256,), dtype=torch.uint8, esize=1)
    e = _no_launch(dit, lambda: run([wts, wts], [wts, wts], [sw, sw, sw], ws=small))
    assert e.status == "DIT_ERR_WORKSPACE"
    # single-stream blocks only: the input must be one [n_txt + n_img, d] array
    e = _no_launch(dit, lambda: run([], [], [sw], xi=FakeDev(0x13000000, shape=(64, 256))))
    assert "directly follow" in str(e)
    # y overlapping the input
    e = _no_launch(dit, lambda: dit.step_forward(s, [wts], [wts], [sw], cond, pos, xt, xi,
                                                 FakeDev(0x12000000, shape=(80, 256), dtype=torch.float32, esize=4),
                                                 ws, stream=FakeStream()))
    assert "overlaps" in str(e)


def _up(x):
    return (x + 255) // 256 * 256


def test_edge_layer_sizes_and_validation(dit):
    import torch
    assert dit.timestep_embedding_workspace_size(256, 3072) == _up(256 * 4) + 2 * _up(3072 * 4)
    assert dit.final_layer_workspace_size(4096, 3072, dit.DIT_F16) == _up(2 * 3072 * 4) + _up(4096 * 3072 * 2)
    x = FakeDev(0x100000, shape=(64, 64))
    w = FakeDev(0x200000, shape=(3072, 64))
    y = FakeDev(0x400000, shape=(64, 3072))
    # linear: n not a multiple of 8; k not a multiple of the MFMA k-step; y overlapping x
    e = _no_launch(dit, lambda: dit.linear(x, FakeDev(0x200000, shape=(3070, 64)), FakeDev(0x400000, shape=(64, 3070)),
                                           stream=FakeStream()))
    assert "multiple of 8" in str(e)
    e = _no_launch(dit, lambda: dit.linear(FakeDev(0x100000, shape=(64, 48)), FakeDev(0x200000, shape=(3072, 48)), y,
                                           stream=FakeStream()))
    assert e.status == "DIT_ERR_UNSUPPORTED"
    e = _no_launch(dit, lambda: dit.linear(x, w, FakeDev(0x100000 + 1024, shape=(64, 3072)), stream=FakeStream()))
    assert "overlaps" in str(e)
    # final layer: d not a multiple of 64; undersized workspace
    cond = FakeDev(0x600000, shape=(3072,))
    e = _no_launch(dit, lambda: dit.final_layer(FakeDev(0x1000000, shape=(16, 3000)), cond,
                                                FakeDev(0x2000000, shape=(6000, 3072)),
                                                FakeDev(0x3000000, shape=(64, 3000)),
                                                FakeDev(0x4000000, shape=(16, 64), dtype=torch.float32, esize=4),
                                                FakeDev(0x5000000, shape=(1 << 20,), dtype=torch.uint8, esize=1),
                                                stream=FakeStream()))
    assert "multiple of 64" in str(e)
    need = dit.final_layer_workspace_size(16, 3072, dit.DIT_F16)
    e = _no_launch(dit, lambda: dit.final_layer(FakeDev(0x1000000, shape=(16, 3072)), cond,
                                                FakeDev(0x2000000, shape=(6144, 3072)),
                                                FakeDev(0x3000000, shape=(64, 3072)),
                                                FakeDev(0x4000000, shape=(16, 64), dtype=torch.float32, esize=4),
                                                FakeDev(0x5000000, shape=(need - 256,), dtype=torch.uint8, esize=1),
                                                stream=FakeStream()))
    assert e.status == "DIT_ERR_WORKSPACE"
    # timestep embedding: max_period must exceed 1; guidance needs its weights
    t = FakeDev(0x700000, shape=(1,), dtype=torch.float32, esize=4)
    wi, wo = FakeDev(0x800000, shape=(3072, 256)), FakeDev(0x1800000, shape=(3072, 3072))
    c = FakeDev(0x3800000, shape=(3072,))
    ws = FakeDev(0x4000000, shape=(1 << 20,), dtype=torch.uint8, esize=1)
    e = _no_launch(dit, lambda: dit.timestep_embedding(t, wi, wo, c, ws, max_period=1.0, stream=FakeStream()))
    assert "max_period" in str(e)
    g = FakeDev(0x700100, shape=(1,), dtype=torch.float32, esize=4)
    e = _no_launch(dit, lambda: dit.timestep_embedding(t, wi, wo, c, ws, g=g, stream=FakeStream()))
    assert "w_g_in" in str(e)


def test_shared_mod_step_validation(dit):
    import torch
    s = _cfg(dit, n_txt=16, n_img=64, d=256, n_heads=2, ffn_inner=768)
    need = dit.step_shared_mod_workspace_size(s, 1, 1)
    assert need == _up(dit.step_workspace_size(s, 1, 1)) + _up(15 * 256 * 4)
    wts = {n: FakeDev(0x1000000 * (i + 1), shape=(1 << 20,)) for i, n in enumerate(
        ("w_qkv", "qk_norm_w", "w_o", "w_ffn_in", "w_ffn_out"))}     # no per-block w_mod
    sw = {n: FakeDev(0x8000000 * (i + 1), shape=(1 << 20,)) for i, n in enumerate(("w_1", "qk_norm_w", "w_2"))}
    mt, mi, ms = (FakeDev(0x20000000 + i * 0x1000000, shape=(1 << 20,)) for i in range(3))
    cond = FakeDev(0x10000000, shape=(256,))
    pos = FakeDev(0x11000000, shape=(80, 4), dtype=torch.int32, esize=4)
    xt, xi = FakeDev(0x12000000, shape=(16, 256)), FakeDev(0x13000000, shape=(64, 256))
    y = FakeDev(0x14000000, shape=(80, 256), dtype=torch.float32, esize=4)
    ws = FakeDev(0x40000000, shape=(need,), dtype=torch.uint8, esize=1)
    # the shared single-block matrix is missing
    e = _no_launch(dit, lambda: dit.step_forward_shared_mod(s, [wts], [wts], [sw], mt, mi, None, cond, pos, xt, xi, y,
                                                            ws, stream=FakeStream()))
    assert "w_mod_single" in str(e)
    # the plain step's workspace is too small for the shared-modulation step
    small = FakeDev(0x40000000, shape=(dit.step_workspace_size(s, 1, 1),), dtype=torch.uint8, esize=1)
    e = _no_launch(dit, lambda: dit.step_forward_shared_mod(s, [wts], [wts], [sw], mt, mi, ms, cond, pos, xt, xi, y,
                                                            small, stream=FakeStream()))
    assert e.status == "DIT_ERR_WORKSPACE"
    # the plain step still needs every block's w_mod
    e = _no_launch(dit, lambda: dit.step_forward(s, [dict(wts, w_mod=None)], [dict(wts, w_mod=None)],
                                                 [dict(sw, w_mod=None)], cond, pos, xt, xi, y, ws, stream=FakeStream()))
    assert "txt[0].w_mod is NULL" in str(e)


def test_gemm_weight_format_validation(dit):
    import dit_inputs as di
    from gpu_util import shape_of
    cfg = di.CONFIGS[1]
    sh = shape_of(cfg, dit)
    base = dit.block_workspace_size(sh)
    sh.gemm_w_dtype = dit.DIT_F16
    assert dit.block_workspace_size(sh) == base
    sh.act_dtype = dit.DIT_BF16            # fp16 weights need fp16 activations
    with pytest.raises(dit.DitError) as e:
        dit.block_workspace_size(sh)
    assert "gemm_w_dtype" in dit.last_error()
    cfg0 = di.CONFIGS[0]                   # fp32 block
    sh0 = shape_of(cfg0, dit)
    sh0.gemm_w_dtype = dit.DIT_F16
    with pytest.raises(dit.DitError):
        dit.block_workspace_size(sh0)


def test_linear_row_stride_limit(dit):
    """The 16-bit GEMM addresses a tile's rows by 32-bit offsets: row strides of 2^22 elements or
    more are refused before any launch."""
    x = FakeDev(0x100000, shape=(2, 64), stride=(1 << 22, 1))
    w = FakeDev(0x200000, shape=(8, 64))
    y = FakeDev(0x300000, shape=(2, 8))
    e = _no_launch(dit, lambda: dit.linear(x, w, y, stream=FakeStream()))
    assert e.status == "DIT_ERR_UNSUPPORTED" and "2^22" in str(e)


def test_conv_channel_limits(dit):
    """Input channels must come in 8s (16-byte chunks of a pixel); any positive output count works."""
    x = FakeDev(0x100000, shape=(1, 4, 4, 60))
    w = FakeDev(0x200000, shape=(8, 3, 3, 60))
    y = FakeDev(0x300000, shape=(1, 4, 4, 8), esize=4)
    e = _no_launch(dit, lambda: dit.conv2d(x, w, y, stream=FakeStream()))
    assert e.status == "DIT_ERR_UNSUPPORTED" and "multiple of 8" in str(e)
    x = FakeDev(0x100000, shape=(1, 4, 4, 64))
    w = FakeDev(0x200000, shape=(0, 3, 3, 64))
    y = FakeDev(0x300000, shape=(1, 4, 4, 0), esize=4)
    e = _no_launch(dit, lambda: dit.conv2d(x, w, y, stream=FakeStream()))
    assert e.status == "DIT_ERR_INVALID_ARG" and "c_out" in str(e)
