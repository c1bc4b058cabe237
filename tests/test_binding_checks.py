"""Host-side argument checks of the Python binding: caller-supplied output buffers of
the wrong shape or dtype and out-of-range windows are refused with ValueError before
any device work (the kernels write the full extent of every output, so a short or
narrower buffer would be written past its end). Runs without a GPU: the checks come
before the device check, so CPU tensors reach them."""
import pytest
import torch

import mask_mods_amd as mm


def _qkv(dtype=torch.bfloat16, B=1, Hq=4, Hkv=2, Sq=16, Skv=24, D=64):
    q = torch.zeros(B, Hq, Sq, D, dtype=dtype)
    k = torch.zeros(B, Hkv, Skv, D, dtype=dtype)
    return q, k, k.clone()


@pytest.mark.parametrize("out_shape,out_dtype", [
    ((1, 4, 16, 32), torch.bfloat16),      # short head dim
    ((1, 4, 8, 64), torch.bfloat16),       # too few rows
    ((1, 4, 16, 64), torch.float16),       # wrong dtype
    ((1, 4, 16, 64), torch.float32),       # wider dtype
])
def test_fwd_out_buffer_rejected(out_shape, out_dtype):
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="out must be"):
        mm.attn_fwd(q, k, v, 0.1, out=torch.empty(out_shape, dtype=out_dtype))


def test_fwd_fp8_out_must_be_bf16():
    q, k, v = _qkv(torch.float8_e4m3fn)
    with pytest.raises(ValueError, match="out must be"):
        mm.attn_fwd(q, k, v, 0.1, out=torch.empty(1, 4, 16, 64, dtype=torch.float8_e4m3fn))


@pytest.mark.parametrize("lse", [torch.empty(1, 4, 15), torch.empty(1, 4, 16, dtype=torch.float16),
                                 torch.empty(1, 16, 4).transpose(1, 2)])
def test_fwd_lse_buffer_rejected(lse):
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="lse must be"):
        mm.attn_fwd(q, k, v, 0.1, lse=lse)


@pytest.mark.parametrize("name", ["dq", "dk", "dv"])
def test_bwd_grad_buffers_rejected(name):
    q, k, v = _qkv()
    o, do = torch.zeros_like(q), torch.zeros_like(q)
    lse = torch.zeros(1, 4, 16, dtype=torch.float32)
    bad = {"dq": torch.empty(1, 4, 16, 32, dtype=torch.bfloat16),
           "dk": torch.empty(1, 2, 24, 64, dtype=torch.float16),
           "dv": torch.empty(1, 4, 24, 64, dtype=torch.bfloat16)}[name]
    with pytest.raises(ValueError, match=f"{name} must be"):
        mm.attn_bwd(q, k, v, o, lse, do, 0.1, **{name: bad})


def test_bwd_workspace_dtype_rejected():
    q, k, v = _qkv()
    lse = torch.zeros(1, 4, 16, dtype=torch.float32)
    with pytest.raises(ValueError, match="workspace"):
        mm.attn_bwd(q, k, v, torch.zeros_like(q), lse, torch.zeros_like(q), 0.1,
                    workspace=torch.empty(4096, dtype=torch.uint8))


@pytest.mark.parametrize("kw,match", [
    (dict(out=torch.empty(2, 8, 1, 64, dtype=torch.float16)), "out must be"),
    (dict(out=torch.empty(2, 8, 1, 128, dtype=torch.bfloat16)), "out must be"),
    (dict(lse=torch.empty(2, 8, 1)), "lse must be"),
    (dict(lse=torch.empty(2, 8, dtype=torch.float16)), "lse must be"),
    (dict(workspace=torch.empty(64, dtype=torch.float16)), "workspace"),
])
def test_decode_buffers_rejected(kw, match):
    q = torch.zeros(2, 8, 1, 128, dtype=torch.float16)
    kc = torch.zeros(2, 8, 64, 128, dtype=torch.float16)
    with pytest.raises(ValueError, match=match):
        mm.attn_decode(q, kc, kc.clone(), 64, 0.0884, **kw)


@pytest.mark.parametrize("window", [-1, 2 ** 31, 2 ** 32 + 5])
def test_window_out_of_int32_range_rejected(window):
    # (a window of 2**32 + 5 would otherwise reach the C struct as 5)
    with pytest.raises(ValueError, match="window must lie"):
        mm._mods(0, 0, window, None, None, None, 4, 16, 16, 1)


def test_window_int32_max_accepted():
    m = mm._mods(0, 0, 2 ** 31 - 1, None, None, None, 4, 16, 16, 1)
    assert m.window == 2 ** 31 - 1 and m.mask_flags & mm.MASK_WINDOW
