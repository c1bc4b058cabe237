"""mm_attn_decode_noalloc (the decode entry point that allocates nothing: its split
partials live in the library's static per-GPU scratch) against mm_attn_decode with the
same arguments, through the C ABI: two calls in a row, the second smaller, so the
second reads a scratch that still holds the first call's partials."""
import ctypes

import numpy as np
import pytest

import oracle
from helpers import LSE_ATOL, LSE_RTOL, O_ATOL, O_RTOL, assert_parity, to_f64, to_torch
from mask_mods_amd import inputs

pytestmark = pytest.mark.gpu

SCALE = 0.08837890625


def _case(seed, B, Hq, Hkv, lens, D, Scap):
    import torch
    x = inputs.decode_inputs(seed, B, Hq, Hkv, lens, D, "f16", Scap=Scap)
    t = {n: to_torch(x[n], "f16") for n in ("q", "k", "v", "mask")}
    t["lens"] = torch.tensor(x["lens"], dtype=torch.int32, device="cuda")
    return x, t


def _noalloc_direct(t, kv_len, out, lse, num_splits=0):
    """One mm_attn_decode_noalloc call built by hand (no workspace pointer at all)."""
    import torch
    import mask_mods_amd as mm
    lib = mm.load_library()
    q, k, v, m = t["q"], t["k"], t["v"], t["mask"]
    a = mm.DecodeArgs()
    a.q, a.k_cache, a.v_cache, a.out, a.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr()
    a.mask, a.seq_lens = m.data_ptr(), t["lens"].data_ptr()
    a.dtype = 1
    a.B, a.Hq, a.Hkv = q.shape[0], q.shape[1], k.shape[1]
    a.kv_len, a.Scap, a.D = kv_len, k.shape[2], q.shape[3]
    a.scale = SCALE
    a.q_strides = mm._I64x2(*q.stride()[:2])
    a.kv_strides = mm._I64x3(*k.stride()[:3])
    a.o_strides = mm._I64x2(*out.stride()[:2])
    a.mask_strides = mm._I64x2(*m.stride()[:2])
    a.num_splits = num_splits
    st = lib.mm_attn_decode_noalloc(ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
    assert st == 0, st


def test_noalloc_matches_decode_on_two_calls_second_smaller():
    import torch
    import mask_mods_amd as mm
    print("[noalloc] call 1: B=2 Hq=32 Hkv=8 lens=[5000, 3001] D=128 f16; "
          "call 2: B=1 Hq=8 Hkv=8 lens=[300] D=64", flush=True)
    runs = [(41, 2, 32, 8, [5000, 3001], 128, 5000), (42, 1, 8, 8, [300], 64, 320)]
    for i, (seed, B, Hq, Hkv, lens, D, Scap) in enumerate(runs):
        x, t = _case(seed, B, Hq, Hkv, lens, D, Scap)
        kv_len = max(lens)
        out_n = torch.full((B, Hq, 1, D), float("nan"), dtype=torch.float16, device="cuda")
        lse_n = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        _noalloc_direct(t, kv_len, out_n, lse_n)
        out_r, lse_r = mm.attn_decode(t["q"], t["k"], t["v"], kv_len, SCALE, mask=t["mask"], seq_lens=t["lens"])
        torch.cuda.synchronize()
        print(f"[noalloc] call {i + 1}: bitwise O {torch.equal(out_n, out_r)} LSE {torch.equal(lse_n, lse_r)}",
              flush=True)
        # the same kernels with the same split count: the same bits
        assert torch.equal(out_n, out_r) and torch.equal(lse_n, lse_r)
        O, L = oracle.attention(*(inputs.bits_to_f64(x[n], "f16") for n in ("q", "k", "v")),
                                scale=SCALE, Skv=kv_len, add_mask=inputs.bits_to_f64(x["mask"], "f16"),
                                lens=x["lens"])
        assert_parity(to_f64(out_n), O, O_ATOL, O_RTOL, "O")
        assert_parity(to_f64(lse_n).reshape(L.shape), L, LSE_ATOL, LSE_RTOL, "LSE")


def test_noalloc_binding_and_forced_splits():
    """The binding's attn_decode_noalloc with a forced split count (and so a different
    scratch layout than the call before) equals attn_decode with the same count."""
    import torch
    import mask_mods_amd as mm
    print("[noalloc] binding: B=1 Hq=32 Hkv=32 L=4096 D=128, splits 0 / 64 / 3", flush=True)
    x, t = _case(43, 1, 32, 32, [4096], 128, 4096)
    for ns in (0, 64, 3):
        o1, l1 = mm.attn_decode_noalloc(t["q"], t["k"], t["v"], 4096, SCALE, mask=t["mask"], num_splits=ns)
        o2, l2 = mm.attn_decode(t["q"], t["k"], t["v"], 4096, SCALE, mask=t["mask"], num_splits=ns)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), ns


def test_noalloc_rejects_oversize_without_launching():
    import torch
    import mask_mods_amd as mm
    print("[noalloc] oversize: B=4 Hq=32 D=128 with 256 forced splits (17 MB of partials)", flush=True)
    assert mm.decode_workspace_size(4, 32, 8192, 128, 256) > mm.DECODE_SCRATCH_BYTES
    q = torch.zeros(4, 32, 1, 128, dtype=torch.float16, device="cuda")
    k = torch.zeros(4, 32, 8192, 128, dtype=torch.float16, device="cuda")
    out = torch.full((4, 32, 1, 128), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(mm.MaskModsError, match="WORKSPACE"):
        mm.attn_decode_noalloc(q, k, k, 8192, SCALE, num_splits=256, out=out, return_lse=False)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing was launched
