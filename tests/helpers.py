"""Shared test helpers: bit arrays -> torch tensors, and the parity comparison.

Holds no attention arithmetic: the expected values always come from ``oracle``.
"""
from __future__ import annotations

import numpy as np

# Parity bar for 16-bit outputs: |gpu - ref| <= atol + rtol * |ref| with 2e-2 / 2e-2
# on O and 1e-3 / 1e-3 on the fp32 LSE (-inf must match exactly).
O_ATOL = O_RTOL = 2e-2
LSE_ATOL = LSE_RTOL = 1e-3
# fp32 inputs: the kernel accumulates in fp32 and writes fp32, so it is held to 1e-4.
F32_ATOL = F32_RTOL = 1e-4


def to_torch(bits: np.ndarray, dtype: str, device="cuda"):
    import torch
    bits = np.ascontiguousarray(bits)
    if dtype == "f32":
        t = torch.from_numpy(bits.view(np.int32)).view(torch.float32)
    else:
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.to(device)


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def assert_parity(got, ref, atol, rtol, what=""):
    """Element-wise allclose with non-finite reference values required to match exactly."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    fin = np.isfinite(ref)
    bad_nf = ~fin & (got != ref)
    assert not bad_nf.any(), f"{what}: {int(bad_nf.sum())} non-finite mismatches, e.g. " \
                             f"got {got[bad_nf][:4]} want {ref[bad_nf][:4]}"
    assert np.isfinite(got[fin]).all(), f"{what}: non-finite output where the reference is finite"
    err = np.abs(got[fin] - ref[fin])
    # atol / rtol may be scalars or per-element arrays shaped like ref
    atol = np.broadcast_to(np.asarray(atol, dtype=np.float64), ref.shape)[fin]
    rtol = np.broadcast_to(np.asarray(rtol, dtype=np.float64), ref.shape)[fin]
    lim = atol + rtol * np.abs(ref[fin])
    ok = err <= lim
    if not ok.all():
        idx = np.argmax(err - lim)
        raise AssertionError(f"{what}: {int((~ok).sum())}/{ok.size} outside tolerance; worst "
                             f"err {err[idx]:.3e} > lim {lim[idx]:.3e} (got {got[fin][idx]}, "
                             f"ref {ref[fin][idx]})")
    return float(err.max()) if err.size else 0.0
