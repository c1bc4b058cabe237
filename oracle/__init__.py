"""The oracle: a plain fp64 CPU attention (``attn_oracle.c``) and its ctypes binding.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``; never by the product package, which
shares no code with it. The C source states the definition it implements and
where on the pages each part comes from.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point this at a deliberately broken build of the oracle (mutation check).
_LIB_OVERRIDE = os.environ.get("MASKMODS_ORACLE_LIB")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_lp = ctypes.POINTER(ctypes.c_int64)
_bp = ctypes.POINTER(ctypes.c_uint8)
BLOCK_Q, BLOCK_KV = 128, 64  # block-mask granularity (query rows x keys)


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    path = _LIB_OVERRIDE or _LIB
    if not _LIB_OVERRIDE and not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(path)
    lib.oracle_fmix32.argtypes = [ctypes.c_uint32]
    lib.oracle_fmix32.restype = ctypes.c_uint32
    lib.oracle_row_dropped.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64]
    lib.oracle_row_dropped.restype = ctypes.c_int
    lib.oracle_alibi_slope.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.oracle_alibi_slope.restype = ctypes.c_double
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    lib.oracle_attention_bwd.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _dp, _dp, _dp, _dp,
        ctypes.c_double, ctypes.c_int, _dp,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32,
        _bp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        _ip, _ip, ctypes.c_int64, ctypes.c_int64,
        _dp, _dp, _dp,
    ]
    lib.oracle_attention_bwd.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _dp, _dp, _dp, ctypes.c_int,
        ctypes.c_double, ctypes.c_int, _dp,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32,
        _dp, ctypes.c_int64, _ip,
        _bp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        _ip, _ip, ctypes.c_int64, ctypes.c_int64,
        _lp, ctypes.c_int64, _dp, _dp, _dp, _dp,
    ]
    lib.oracle_attention.restype = ctypes.c_int
    _lib = lib
    return lib


def fmix32(x: int) -> int:
    return int(load().oracle_fmix32(x & 0xFFFFFFFF))


def row_dropped(seed: int, threshold: int, row: int) -> bool:
    return bool(load().oracle_row_dropped(seed & 0xFFFFFFFF, threshold & 0xFFFFFFFF, row))


def alibi_slope(h: int, H: int) -> float:
    return float(load().oracle_alibi_slope(h, H))


def max_threads() -> int:
    return int(load().oracle_max_threads())


def set_threads(n: int) -> None:
    load().oracle_set_threads(int(n))


def _ptr(a, typ):
    return None if a is None else a.ctypes.data_as(typ)


def _docs(q_doc, kv_doc, B, Sq, Skv):
    """Document ids: None, or int [B, Sq] and int [B, Skv] (kv_doc defaults to q_doc)."""
    if q_doc is None:
        return None, None, 0, 0
    kv_doc = q_doc if kv_doc is None else kv_doc
    q_doc = np.ascontiguousarray(q_doc, dtype=np.int32).reshape(B, -1)
    kv_doc = np.ascontiguousarray(kv_doc, dtype=np.int32).reshape(B, -1)
    assert q_doc.shape[1] >= Sq and kv_doc.shape[1] >= Skv
    return q_doc, kv_doc, q_doc.shape[1], kv_doc.shape[1]


def attention(q, k, v, *, scale, Skv=None, causal=False, window=None, alibi=False,
              slopes=None, rowdrop=None, add_mask=None, lens=None, rows=None, block_mask=None,
              q_doc=None, kv_doc=None, sensitivity=False):
    """Run the oracle.

    q: float64 [B,Hq,Sq,D]; k, v: float64 [B,Hkv,kv_cap,D] (first ``Skv`` keys used,
    default kv_cap). window: None or int >= 0. rowdrop: None or (seed, threshold).
    add_mask: None or float64 [B,Hq,Sq,mask_ld]. lens: None or int [B].
    rows: None (all rows; returns O [B,Hq,Sq,D], LSE [B,Hq,Sq]) or flat row ids
    (b*Hq + h)*Sq + i (returns O [n,D], LSE [n]).
    block_mask: None or uint8 [B or 1, Hq or 1, ceil(Sq/128), ceil(Skv/64)] with
    0 = block masked, 1 = predicates decide, 2 = block kept (size-1 dims broadcast).
    q_doc, kv_doc: None, or document ids [B, Sq] and [B, Skv]: a pair is kept only where
    they are equal (kv_doc defaults to q_doc).
    sensitivity: also return wsq (per row, sum of squared weights) and wvar (per
    element, sum_j w_j^2 (V[j,d] - O[d])^2), shaped like LSE and O.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Hq, Sq, D = q.shape
    Bk, Hkv, kv_cap, Dk = k.shape
    assert v.shape == k.shape and Bk == B and Dk == D
    if Skv is None:
        Skv = kv_cap
    if slopes is not None:
        slopes = np.ascontiguousarray(slopes, dtype=np.float64)
        assert slopes.shape == (Hq,)
    mask_ld = 0
    if add_mask is not None:
        add_mask = np.ascontiguousarray(add_mask, dtype=np.float64)
        assert add_mask.shape[:3] == (B, Hq, Sq) and add_mask.shape[3] >= Skv
        mask_ld = add_mask.shape[3]
    if lens is not None:
        lens = np.ascontiguousarray(lens, dtype=np.int32).reshape(B)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        n = rows.size
    else:
        n = B * Hq * Sq
    out = np.zeros((n, D), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    wsq = np.zeros((n,), dtype=np.float64) if sensitivity else None
    wvar = np.zeros((n, D), dtype=np.float64) if sensitivity else None
    seed, thr = (0, 0) if rowdrop is None else rowdrop
    bm_s = (0, 0, 0)
    if block_mask is not None:
        block_mask = np.ascontiguousarray(block_mask, dtype=np.uint8)
        Bb, Hb, nqb, nkb = block_mask.shape
        assert Bb in (1, B) and Hb in (1, Hq)
        assert nqb >= -(-Sq // BLOCK_Q) and nkb >= -(-Skv // BLOCK_KV)
        bm_s = (0 if Bb == 1 else Hb * nqb * nkb, 0 if Hb == 1 else nqb * nkb, nkb)
    qd_, kd_, qds, kds = _docs(q_doc, kv_doc, B, Sq, Skv)
    rc = load().oracle_attention(
        B, Hq, Hkv, Sq, Skv, D, _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), kv_cap,
        float(scale), int(bool(alibi)), _ptr(slopes, _dp),
        int(bool(causal)), -1 if window is None else int(window), int(rowdrop is not None),
        seed & 0xFFFFFFFF, thr & 0xFFFFFFFF,
        _ptr(add_mask, _dp), mask_ld, _ptr(lens, _ip),
        _ptr(block_mask, _bp), bm_s[0], bm_s[1], bm_s[2],
        _ptr(qd_, _ip), _ptr(kd_, _ip), qds, kds,
        _ptr(rows, _lp), n if rows is not None else 0, _ptr(out, _dp), _ptr(lse, _dp),
        _ptr(wsq, _dp), _ptr(wvar, _dp))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    if rows is None:
        res = (out.reshape(B, Hq, Sq, D), lse.reshape(B, Hq, Sq))
        if sensitivity:
            res += (wsq.reshape(B, Hq, Sq), wvar.reshape(B, Hq, Sq, D))
        return res
    return (out, lse, wsq, wvar) if sensitivity else (out, lse)


def block_classes(Sq: int, Skv: int, *, causal: bool = False, window=None) -> np.ndarray:
    """Block-mask classes of the causal / sliding-window predicates, by brute force.

    Evaluates the predicates (causal: kv_idx <= q_idx; window: |q_idx - kv_idx| <= w)
    on every pair (q_idx < Sq, kv_idx < Skv) and classifies each block of BLOCK_Q x
    BLOCK_KV pairs: 0 if no pair is kept, 2 if every pair is kept, else 1 (the classes
    the oracle's ``block_mask`` argument reads). Returns uint8 [ceil(Sq/128), ceil(Skv/64)].
    """
    nqb, nkb = -(-Sq // BLOCK_Q), -(-Skv // BLOCK_KV)
    out = np.zeros((nqb, nkb), dtype=np.uint8)
    i = np.arange(Sq)[:, None]
    j = np.arange(Skv)[None, :]
    for qb in range(nqb):
        ii = i[qb * BLOCK_Q:(qb + 1) * BLOCK_Q]
        for kb in range(nkb):
            jj = j[:, kb * BLOCK_KV:(kb + 1) * BLOCK_KV]
            keep = np.ones((ii.shape[0], jj.shape[1]), dtype=bool)
            if causal:
                keep &= jj <= ii
            if window is not None:
                keep &= np.abs(ii - jj) <= window
            out[qb, kb] = 2 if keep.all() else (1 if keep.any() else 0)
    return out


def attention_bwd(q, k, v, dout, *, scale, causal=False, window=None, alibi=False, slopes=None,
                  rowdrop=None, block_mask=None, q_doc=None, kv_doc=None):
    """Gradients (dq, dk, dv) of sum(dout * O) for the forward of ``attention`` (no
    additive mask or lengths), in float64. Shapes as ``attention`` with kv_cap = Skv."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    dout = np.ascontiguousarray(dout, dtype=np.float64)
    B, Hq, Sq, D = q.shape
    _, Hkv, Skv, _ = k.shape
    assert v.shape == k.shape and dout.shape == q.shape
    if slopes is not None:
        slopes = np.ascontiguousarray(slopes, dtype=np.float64)
    seed, thr = (0, 0) if rowdrop is None else rowdrop
    bm_s = (0, 0, 0)
    if block_mask is not None:
        block_mask = np.ascontiguousarray(block_mask, dtype=np.uint8)
        Bb, Hb, nqb, nkb = block_mask.shape
        assert Bb in (1, B) and Hb in (1, Hq)
        assert nqb >= -(-Sq // BLOCK_Q) and nkb >= -(-Skv // BLOCK_KV)
        bm_s = (0 if Bb == 1 else Hb * nqb * nkb, 0 if Hb == 1 else nqb * nkb, nkb)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    qd_, kd_, qds, kds = _docs(q_doc, kv_doc, B, Sq, Skv)
    rc = load().oracle_attention_bwd(
        B, Hq, Hkv, Sq, Skv, D, _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(dout, _dp),
        float(scale), int(bool(alibi)), _ptr(slopes, _dp),
        int(bool(causal)), -1 if window is None else int(window), int(rowdrop is not None),
        seed & 0xFFFFFFFF, thr & 0xFFFFFFFF,
        _ptr(block_mask, _bp), bm_s[0], bm_s[1], bm_s[2],
        _ptr(qd_, _ip), _ptr(kd_, _ip), qds, kds,
        _ptr(dq, _dp), _ptr(dk, _dp), _ptr(dv, _dp))
    if rc != 0:
        raise ValueError("oracle_attention_bwd rejected its arguments")
    return dq, dk, dv
