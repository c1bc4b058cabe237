"""mask_mods_amd: flex-style fused attention for MI355X (gfx950).

A thin ctypes binding over ``libmaskmods.so`` (C ABI in ``include/maskmods.h``).
This layer only marshals arguments: it takes torch tensors for device memory and
the current HIP stream, fills the argument struct and calls the library. Every
step of the computation runs in the library's HIP kernels; there is no fallback.
If the library is missing, importing works but every call raises.

    from mask_mods_amd import attn_fwd, attn_decode
    out, lse = attn_fwd(q, k, v, scale, causal=True)              # [B,H,S,D]
    out, lse = attn_decode(q, k_cache, v_cache, kv_len, scale, mask=mask)
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "attn_fwd", "attn_bwd", "bwd_workspace_size", "attn_decode", "attn_decode_noalloc",
    "decode_workspace_size", "DECODE_SCRATCH_BYTES",
    "decode_auto_splits", "block_mask_create",
    "MaskModsError", "library_path", "load_library",
    "SCORE_NONE", "SCORE_ALIBI", "MASK_CAUSAL", "MASK_WINDOW", "MASK_ROWDROP",
    "ROWDROP_5PCT", "BLOCK_Q", "BLOCK_KV", "BLOCK_EMPTY", "BLOCK_PARTIAL", "BLOCK_FULL",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmaskmods.so")

MM_F32, MM_F16, MM_BF16, MM_FP8_E4M3 = 0, 1, 2, 3
SCORE_NONE, SCORE_ALIBI = 0, 1
MASK_CAUSAL, MASK_WINDOW, MASK_ROWDROP, MASK_DOCUMENT = 1, 2, 4, 8
ROWDROP_5PCT = int(0.05 * 2 ** 32)  # threshold that drops ~5% of rows
# block mask: query rows x keys per block, and the per-block classes
BLOCK_Q, BLOCK_KV = 128, 64
BLOCK_EMPTY, BLOCK_PARTIAL, BLOCK_FULL = 0, 1, 2
# bytes of the static per-GPU decode scratch of mm_attn_decode_noalloc
DECODE_SCRATCH_BYTES = 16 * 1024 * 1024

_STATUS = {
    0: "MM_OK", -1: "MM_ERR_NULL", -2: "MM_ERR_SHAPE", -3: "MM_ERR_DTYPE",
    -4: "MM_ERR_UNSUPPORTED", -5: "MM_ERR_STRIDE", -6: "MM_ERR_LAUNCH", -7: "MM_ERR_WORKSPACE",
}


class MaskModsError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {_STATUS.get(status, status)}")


class _Mods(ctypes.Structure):
    _fields_ = [
        ("score_mod", ctypes.c_int32),
        ("mask_flags", ctypes.c_uint32),
        ("window", ctypes.c_int32),
        ("rowdrop_seed", ctypes.c_uint32),
        ("rowdrop_threshold", ctypes.c_uint32),
        ("alibi_slopes", ctypes.c_void_p),
        ("block_mask", ctypes.c_void_p),
        ("block_mask_strides", ctypes.c_int64 * 3),
        ("q_doc_ids", ctypes.c_void_p),
        ("kv_doc_ids", ctypes.c_void_p),
        ("doc_strides", ctypes.c_int64 * 2),
    ]


_I64x3 = ctypes.c_int64 * 3
_I64x2 = ctypes.c_int64 * 2


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Sq", ctypes.c_int32), ("Skv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("q_strides", _I64x3), ("k_strides", _I64x3), ("v_strides", _I64x3), ("o_strides", _I64x3),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("mods", _Mods),
        ("descale_q", ctypes.c_float), ("descale_k", ctypes.c_float), ("descale_v", ctypes.c_float),
    ]


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Sq", ctypes.c_int32), ("Skv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("q_strides", ctypes.c_int64 * 3), ("k_strides", ctypes.c_int64 * 3),
        ("v_strides", ctypes.c_int64 * 3), ("o_strides", ctypes.c_int64 * 3),
        ("do_strides", ctypes.c_int64 * 3), ("dq_strides", ctypes.c_int64 * 3),
        ("dk_strides", ctypes.c_int64 * 3), ("dv_strides", ctypes.c_int64 * 3),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("mods", _Mods),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("mask", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("kv_len", ctypes.c_int32), ("Scap", ctypes.c_int32), ("D", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q_strides", _I64x2), ("kv_strides", _I64x3), ("o_strides", _I64x2), ("mask_strides", _I64x2),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("num_splits", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("block_table_stride", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmaskmods.so and check the struct layouts match this binding."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -m mask_mods_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.mm_attn_fwd.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p]
    lib.mm_attn_fwd.restype = ctypes.c_int32
    lib.mm_attn_decode.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]
    lib.mm_attn_decode.restype = ctypes.c_int32
    lib.mm_attn_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]
    lib.mm_attn_decode_noalloc.restype = ctypes.c_int32
    lib.mm_attn_decode_workspace_size.argtypes = [ctypes.c_int32] * 6
    lib.mm_attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.mm_attn_decode_auto_splits.argtypes = [ctypes.c_int32] * 4
    lib.mm_attn_decode_auto_splits_varlen.argtypes = [ctypes.c_int32] * 4
    lib.mm_attn_decode_auto_splits_varlen.restype = ctypes.c_int32
    lib.mm_attn_decode_auto_splits.restype = ctypes.c_int32
    lib.mm_block_mask_create.argtypes = [ctypes.c_uint32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.mm_block_mask_create.restype = ctypes.c_int32
    lib.mm_attn_bwd.argtypes = [ctypes.POINTER(BwdArgs), ctypes.c_void_p]
    lib.mm_attn_bwd.restype = ctypes.c_int32
    lib.mm_attn_bwd_workspace_size.argtypes = [ctypes.c_int32] * 3
    lib.mm_attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.mm_bwd_args_size.restype = ctypes.c_size_t
    lib.mm_status_str.argtypes = [ctypes.c_int32]
    lib.mm_status_str.restype = ctypes.c_char_p
    lib.mm_fwd_args_size.restype = ctypes.c_size_t
    lib.mm_decode_args_size.restype = ctypes.c_size_t
    lib.mm_version.restype = ctypes.c_int32
    lib.mm_source_hash.restype = ctypes.c_char_p
    # the library must come from the sources beside it: a stale build would run kernels
    # and a workspace contract this binding does not describe
    from .build import source_hash
    built, here = lib.mm_source_hash().decode(), source_hash()
    if built != here:
        raise RuntimeError(
            f"{_LIB_PATH} was built from other sources (library {built}, sources {here}); "
            "run `python -m mask_mods_amd.build` (or __graft_entry__.build()) again")
    if lib.mm_fwd_args_size() != ctypes.sizeof(FwdArgs):
        raise RuntimeError("mm_fwd_args layout mismatch between library and binding")
    if lib.mm_decode_args_size() != ctypes.sizeof(DecodeArgs):
        raise RuntimeError("mm_decode_args layout mismatch between library and binding")
    if lib.mm_bwd_args_size() != ctypes.sizeof(BwdArgs):
        raise RuntimeError("mm_bwd_args layout mismatch between library and binding")
    _lib = lib
    return lib


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: MM_F32, torch.float16: MM_F16, torch.bfloat16: MM_BF16,
         torch.float8_e4m3fn: MM_FP8_E4M3}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _stream_ptr(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _check_buf(t, shape, dtype, name, contiguous=False):
    """A caller-supplied output buffer must have exactly the shape and dtype the kernel
    writes (it writes the full extent without bounds of its own)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {list(shape)}, got {t.dtype} {list(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("mask_mods_amd operates on device tensors only")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if t.dim() >= 1 and t.stride(-1) != 1 and t.size(-1) > 1 and t.numel() > 0:
            raise ValueError("the last (head) dimension must be contiguous")
    return dev


def attn_fwd(q, k, v, scale=None, *, causal=False, score_mod=SCORE_NONE, alibi_slopes=None,
             mask_flags=0, window=None, rowdrop=None, block_mask=None, q_doc=None, kv_doc=None,
             descale=None, return_lse=True, out=None, lse=None):
    """Fused attention forward.

    q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D] (bf16, f16, f32 or float8_e4m3fn; D in {64,128}).
    fp8 inputs: ``descale=(dq, dk, dv)`` gives the per-tensor factors of the real
    tensors (dq * q etc., default 1); the output is bf16.
    score_mod: SCORE_NONE or SCORE_ALIBI (or the string "alibi").
    mask_flags: OR of MASK_CAUSAL / MASK_WINDOW / MASK_ROWDROP; ``window`` sets
    MASK_WINDOW, ``rowdrop=(seed, threshold)`` sets MASK_ROWDROP.
    block_mask: optional uint8 device tensor [B|1, Hq|1, >=ceil(Sq/128), >=ceil(Skv/64)],
    one class per (query block of BLOCK_Q rows, key block of BLOCK_KV keys):
    BLOCK_EMPTY (skipped), BLOCK_PARTIAL (the mask predicates decide) or BLOCK_FULL
    (all kept); size-1 leading dims broadcast.
    q_doc, kv_doc: document mask, int32 device tensors [B|1, >=Sq] and [B|1, >=Skv] of
    ids that do not decrease along the sequence (kv_doc defaults to q_doc): a pair is
    kept only where the two ids are equal (AND-composed with the other mods).
    Returns (out, lse) with lse fp32 [B,Hq,Sq] (None if return_lse is False).
    """
    torch = _torch()
    lib = load_library()
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q/k/v shapes or dtypes disagree")
    fp8 = q.dtype == torch.float8_e4m3fn
    _check_buf(out, (B, Hq, Sq, D), torch.bfloat16 if fp8 else q.dtype, "out")
    _check_buf(lse, (B, Hq, Sq), torch.float32, "lse", contiguous=True)
    dev = _check_dev(q, k, v, out, lse, alibi_slopes, block_mask, q_doc, kv_doc)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16 if fp8 else q.dtype, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    a = FwdArgs()
    a.q, a.k, a.v, a.out = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    a.dtype = _dtype_code(q)
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = B, Hq, Hkv, Sq, Skv, D
    a.q_strides = _I64x3(*q.stride()[:3])
    a.k_strides = _I64x3(*k.stride()[:3])
    a.v_strides = _I64x3(*v.stride()[:3])
    a.o_strides = _I64x3(*out.stride()[:3])
    a.scale = float(scale)
    a.causal = 1 if causal else 0
    a.mods = _mods(score_mod, mask_flags, window, rowdrop, alibi_slopes, block_mask, Hq, Sq, Skv, B,
                   q_doc, kv_doc)
    a.descale_q, a.descale_k, a.descale_v = (1.0, 1.0, 1.0) if descale is None else map(float, descale)
    st = lib.mm_attn_fwd(ctypes.byref(a), _stream_ptr(dev))
    if st != 0:
        raise MaskModsError(st, "mm_attn_fwd")
    return out, (lse if return_lse else None)


def block_mask_create(Sq, Skv, *, causal=False, window=None, device=None, out=None):
    """Block-mask classes of the built-in predicates, uint8 [1, 1, ceil(Sq/128), ceil(Skv/64)].

    Pass the result to attn_fwd(block_mask=...) together with the same causal / window
    arguments: empty blocks are then never read and full blocks skip the predicates.
    """
    torch = _torch()
    lib = load_library()
    nqb, nkb = -(-Sq // BLOCK_Q), -(-Skv // BLOCK_KV)
    if out is None:
        out = torch.empty((1, 1, nqb, nkb), dtype=torch.uint8,
                          device=device if device is not None else "cuda")
    dev = _check_dev(out)
    if out.dtype != torch.uint8 or out.dim() != 4 or out.shape[2] < nqb or out.shape[3] < nkb \
            or (out.shape[3] > 1 and out.stride(3) != 1):
        raise ValueError("out must be uint8 [.., .., >=ceil(Sq/128), >=ceil(Skv/64)], last dim contiguous")
    flags = (MASK_CAUSAL if causal else 0) | (MASK_WINDOW if window is not None else 0)
    st = lib.mm_block_mask_create(flags, int(window) if window is not None else 0, Sq, Skv,
                                  out.data_ptr() if out.numel() else None, out.stride(2), _stream_ptr(dev))
    if st != 0:
        raise MaskModsError(st, "mm_block_mask_create")
    return out


def _mods(score_mod, mask_flags, window, rowdrop, alibi_slopes, block_mask, Hq, Sq, Skv, B,
          q_doc=None, kv_doc=None):
    """Fill an mm_mods struct (shared by the forward and backward calls)."""
    torch = _torch()
    m = _Mods()
    if isinstance(score_mod, str):
        score_mod = {"none": SCORE_NONE, "alibi": SCORE_ALIBI}[score_mod]
    flags = int(mask_flags)
    if window is not None:
        if not 0 <= int(window) <= 2 ** 31 - 1:
            raise ValueError(f"window must lie in [0, 2**31 - 1], got {window}")
        flags |= MASK_WINDOW
    seed, thr = 0, 0
    if rowdrop is not None:
        flags |= MASK_ROWDROP
        seed, thr = rowdrop
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or tuple(alibi_slopes.shape) != (Hq,) \
                or not alibi_slopes.is_contiguous():
            raise ValueError("alibi_slopes must be contiguous fp32 [Hq]")
    bm_strides = (0, 0, 0)
    if block_mask is not None:
        nqb, nkb = -(-Sq // BLOCK_Q), -(-Skv // BLOCK_KV)
        if block_mask.dtype != torch.uint8 or block_mask.dim() != 4:
            raise ValueError("block_mask must be a 4-D uint8 tensor")
        bb, bh, bq, bk = block_mask.shape
        if bb not in (1, B) or bh not in (1, Hq) or bq < nqb or bk < nkb:
            raise ValueError(f"block_mask shape {tuple(block_mask.shape)} does not cover "
                             f"[{B}|1, {Hq}|1, {nqb}, {nkb}]")
        if bk > 1 and block_mask.stride(3) != 1:
            raise ValueError("block_mask's last dimension must be contiguous")
        bm_strides = tuple(0 if n == 1 else st for n, st in zip(block_mask.shape[:3], block_mask.stride()[:3]))
    m.score_mod = int(score_mod)
    m.mask_flags = flags
    m.window = int(window) if window is not None else 0
    m.rowdrop_seed = seed & 0xFFFFFFFF
    m.rowdrop_threshold = thr & 0xFFFFFFFF
    m.alibi_slopes = alibi_slopes.data_ptr() if alibi_slopes is not None else None
    m.block_mask = block_mask.data_ptr() if block_mask is not None and block_mask.numel() else None
    m.block_mask_strides = _I64x3(*bm_strides)
    if kv_doc is not None and q_doc is None:
        raise ValueError("kv_doc needs q_doc")
    if q_doc is not None:
        kv_doc = q_doc if kv_doc is None else kv_doc
        for name, t, n in (("q_doc", q_doc, Sq), ("kv_doc", kv_doc, Skv)):
            if t.dtype != torch.int32 or t.dim() != 2 or t.shape[0] not in (1, B) or t.shape[1] < n:
                raise ValueError(f"{name} must be int32 [{B}|1, >={n}], got {t.dtype} {tuple(t.shape)}")
        m.mask_flags = flags | MASK_DOCUMENT
        m.q_doc_ids = q_doc.data_ptr() if q_doc.numel() else None
        m.kv_doc_ids = kv_doc.data_ptr() if kv_doc.numel() else None
        m.doc_strides = _I64x2(0 if q_doc.shape[0] == 1 else q_doc.stride(0),
                               0 if kv_doc.shape[0] == 1 else kv_doc.stride(0))
    return m


def bwd_workspace_size(B, Hq, Sq) -> int:
    return int(load_library().mm_attn_bwd_workspace_size(B, Hq, Sq))


def attn_bwd(q, k, v, out, lse, dout, scale=None, *, causal=False, score_mod=SCORE_NONE,
             alibi_slopes=None, mask_flags=0, window=None, rowdrop=None, block_mask=None,
             q_doc=None, kv_doc=None, workspace=None, dq=None, dk=None, dv=None):
    """Backward of attn_fwd: gradients (dq, dk, dv) of sum(dout * out).

    q, k, v, out, lse: the forward's inputs and outputs (lse is required); dout like out.
    The mods must be the forward's. bf16 or f16, D in {64, 128}.
    """
    torch = _torch()
    lib = load_library()
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shapes disagree")
    if any(t.dtype != q.dtype for t in (k, v, out, dout)):
        raise ValueError("q/k/v/out/dout dtypes disagree")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("lse must be contiguous fp32 [B,Hq,Sq]")
    _check_buf(dq, q.shape, q.dtype, "dq")
    _check_buf(dk, k.shape, k.dtype, "dk")
    _check_buf(dv, v.shape, v.dtype, "dv")
    if workspace is not None and workspace.dtype != torch.float32:
        raise ValueError("workspace must be a float32 tensor")
    dev = _check_dev(q, k, v, out, lse, dout, alibi_slopes, block_mask, q_doc, kv_doc, workspace, dq, dk, dv)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = bwd_workspace_size(B, Hq, Sq)
    if workspace is None:
        workspace = torch.empty(need // 4 + 4, dtype=torch.float32, device=dev)
    a = BwdArgs()
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.out, a.dout, a.lse = out.data_ptr(), dout.data_ptr(), lse.data_ptr()
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    a.dtype = _dtype_code(q)
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = B, Hq, Hkv, Sq, Skv, D
    for name, t in (("q", q), ("k", k), ("v", v), ("o", out), ("do", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        setattr(a, name + "_strides", _I64x3(*t.stride()[:3]))
    a.scale = float(scale)
    a.causal = 1 if causal else 0
    a.mods = _mods(score_mod, mask_flags, window, rowdrop, alibi_slopes, block_mask, Hq, Sq, Skv, B,
                   q_doc, kv_doc)
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib.mm_attn_bwd(ctypes.byref(a), _stream_ptr(dev))
    if st != 0:
        raise MaskModsError(st, "mm_attn_bwd")
    return dq, dk, dv


def decode_workspace_size(B, Hq, kv_len, D, num_splits=0, Hkv=None) -> int:
    Hkv = Hq if Hkv is None else Hkv
    return int(load_library().mm_attn_decode_workspace_size(B, Hq, Hkv, kv_len, D, num_splits))


def decode_auto_splits(B, Hq, kv_len, Hkv=None, varlen=False) -> int:
    """Automatic split count of attn_decode; varlen: for a call with seq_lens."""
    Hkv = Hq if Hkv is None else Hkv
    lib = load_library()
    fn = lib.mm_attn_decode_auto_splits_varlen if varlen else lib.mm_attn_decode_auto_splits
    return int(fn(B, Hq, Hkv, kv_len))


def attn_decode_noalloc(q, k_cache, v_cache, kv_len, scale, *, mask=None, seq_lens=None,
                        return_lse=True, num_splits=0, out=None, lse=None, block_table=None):
    """attn_decode through mm_attn_decode_noalloc: the split partials go to the library's
    static per-GPU scratch (DECODE_SCRATCH_BYTES) instead of a workspace, so the call
    allocates no device memory when ``out`` (and ``lse``, or return_lse=False) are
    given. Calls that overlap in time on one GPU share the scratch and race."""
    return attn_decode(q, k_cache, v_cache, kv_len, scale, mask=mask, seq_lens=seq_lens,
                       return_lse=return_lse, num_splits=num_splits, out=out, lse=lse,
                       block_table=block_table, _noalloc=True)


def attn_decode(q, k_cache, v_cache, kv_len, scale, *, mask=None, seq_lens=None,
                return_lse=True, num_splits=0, workspace=None, out=None, lse=None,
                block_table=None, _noalloc=False):
    """Decode attention: q [B,Hq,1,D] against caches [B,Hkv,Scap,D] (f16/bf16).

    kv_len: number of cache positions in use (<= Scap). mask: optional f16
    additive mask [B,Hq,1,Scap] (last dim contiguous). seq_lens: optional int32
    device tensor [B] of per-sequence lengths (<= kv_len).
    block_table: optional int32 device tensor [B, max_pages]; the caches are then page
    pools [pages, Hkv, page_size, D] (page_size a power of two) and Scap is
    max_pages * page_size.
    Returns (out [B,Hq,1,D], lse fp32 [B,Hq] or None).
    """
    torch = _torch()
    lib = load_library()
    B, Hq, one, D = q.shape
    _check_buf(out, (B, Hq, 1, D), q.dtype, "out")
    _check_buf(lse, (B, Hq), torch.float32, "lse", contiguous=True)
    if workspace is not None and workspace.dtype != torch.float32:
        raise ValueError("workspace must be a float32 tensor")
    dev = _check_dev(q, k_cache, v_cache, mask, seq_lens, out, lse, workspace, block_table)
    if block_table is not None:
        _, Hkv, page_size, Dk = k_cache.shape
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B \
                or (block_table.shape[1] > 1 and block_table.stride(1) != 1):
            raise ValueError("block_table must be int32 [B, max_pages] with unit column stride")
        Scap = block_table.shape[1] * page_size
        Bk = B
    else:
        Bk, Hkv, Scap, Dk = k_cache.shape
        page_size = 0
    if one != 1 or Bk != B or Dk != D or v_cache.shape != k_cache.shape:
        raise ValueError("decode shapes disagree")
    if k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must share strides")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q/k/v dtypes disagree")
    if mask is not None and (mask.dtype != torch.float16 or mask.shape[0] != B or mask.shape[1] != Hq
                             or mask.shape[-1] < kv_len):
        raise ValueError("mask must be f16 [B,Hq,1,>=kv_len]")
    if seq_lens is not None and (seq_lens.dtype != torch.int32 or seq_lens.numel() != B):
        raise ValueError("seq_lens must be int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, 1, D), dtype=q.dtype, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if not _noalloc and workspace is None:
        need = lib.mm_attn_decode_workspace_size(B, Hq, Hkv, int(kv_len), D, int(num_splits))
        workspace = torch.empty((max(need, 16) + 3) // 4, dtype=torch.float32, device=dev)
    a = DecodeArgs()
    a.q, a.k_cache, a.v_cache, a.out = q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    a.mask = mask.data_ptr() if mask is not None else None
    a.seq_lens = seq_lens.data_ptr() if seq_lens is not None else None
    a.dtype = _dtype_code(q)
    a.B, a.Hq, a.Hkv, a.kv_len, a.Scap, a.D = B, Hq, Hkv, int(kv_len), Scap, D
    a.scale = float(scale)
    a.q_strides = _I64x2(*q.stride()[:2])
    a.kv_strides = _I64x3(*k_cache.stride()[:3])
    a.o_strides = _I64x2(*out.stride()[:2])
    a.mask_strides = _I64x2(*(mask.stride()[:2] if mask is not None else (0, 0)))
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    a.num_splits = int(num_splits)
    if block_table is not None:
        a.block_table = block_table.data_ptr()
        a.block_table_stride = block_table.stride(0)
        a.page_size = int(page_size)
    fn, name = (lib.mm_attn_decode_noalloc, "mm_attn_decode_noalloc") if _noalloc else (lib.mm_attn_decode, "mm_attn_decode")
    st = fn(ctypes.byref(a), _stream_ptr(dev))
    if st != 0:
        raise MaskModsError(st, name)
    return out, (lse if return_lse else None)
