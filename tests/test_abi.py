"""Host-side checks of the C ABI: the library loads, exports what the header
declares, mirrors the struct layouts, and rejects bad arguments before any
launch (no compute calls: these run without a GPU)."""
import ctypes
import os
import re

import pytest

import mask_mods_amd as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "maskmods.h")

OK, NULL, SHAPE, DTYPE, UNSUP, STRIDE, LAUNCH, WORKSPACE = 0, -1, -2, -3, -4, -5, -6, -7
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below is rejected on the host


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = mm.load_library()
    names = _declared_functions()
    assert "mm_attn_fwd" in names and "mm_attn_decode" in names
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layouts_match():
    lib = mm.load_library()
    assert lib.mm_fwd_args_size() == ctypes.sizeof(mm.FwdArgs)
    assert lib.mm_decode_args_size() == ctypes.sizeof(mm.DecodeArgs)
    assert lib.mm_bwd_args_size() == ctypes.sizeof(mm.BwdArgs)
    assert lib.mm_version() >= 400


def test_library_built_from_these_sources():
    """The in-tree library carries the hash of the sources beside it (the binding refuses
    a mismatch at load, so a stale build cannot run)."""
    from mask_mods_amd.build import source_hash
    lib = mm.load_library()
    assert lib.mm_source_hash().decode() == source_hash()
    assert len(source_hash()) == 16


def test_status_strings():
    lib = mm.load_library()
    for st in (OK, NULL, SHAPE, DTYPE, UNSUP, STRIDE, LAUNCH, WORKSPACE):
        assert lib.mm_status_str(st)
    assert lib.mm_status_str(12345) == b"unknown status"


def _fwd(**kw):
    a = mm.FwdArgs()
    a.q = a.k = a.v = a.out = FAKE
    a.dtype = 2
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = 1, 4, 2, 16, 16, 128
    a.q_strides = mm._I64x3(4 * 16 * 128, 16 * 128, 128)
    a.k_strides = mm._I64x3(2 * 16 * 128, 16 * 128, 128)
    a.v_strides = mm._I64x3(2 * 16 * 128, 16 * 128, 128)
    a.o_strides = mm._I64x3(4 * 16 * 128, 16 * 128, 128)
    a.scale = 0.1
    for key, val in kw.items():
        if key.startswith("mods_"):
            setattr(a.mods, key[5:], val)
        else:
            setattr(a, key, val)
    return mm.load_library().mm_attn_fwd(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NULL),
    (dict(out=None), NULL),
    (dict(k=None), NULL),
    (dict(q=None, Sq=0), OK),
    (dict(k=None, v=None, Skv=0, B=0), OK),
    (dict(dtype=7), DTYPE),
    (dict(Hq=3), SHAPE),
    (dict(Hkv=0), SHAPE),
    (dict(Sq=-1), SHAPE),
    (dict(Skv=-5), SHAPE),
    (dict(Sq=1 << 30), SHAPE),                   # lengths stay below 2^30
    (dict(Skv=1 << 30), SHAPE),
    (dict(D=96), UNSUP),
    (dict(D=256), UNSUP),
    (dict(mods_score_mod=9), UNSUP),
    (dict(mods_mask_flags=16), UNSUP),
    (dict(mods_mask_flags=2, mods_window=-1), SHAPE),
    (dict(q_strides=mm._I64x3(-1, 0, 0)), STRIDE),
    (dict(k_strides=mm._I64x3(100, 12, 128)), STRIDE),
    (dict(q=FAKE + 2), STRIDE),
    (dict(scale=float("nan")), SHAPE),
    (dict(mods_block_mask=FAKE, mods_block_mask_strides=mm._I64x3(0, -4, 1)), STRIDE),
    (dict(B=0), OK),
    (dict(Sq=0), OK),
])
def test_fwd_rejects_before_launch(kw, status):
    assert _fwd(**kw) == status


def test_fwd_null_args():
    assert mm.load_library().mm_attn_fwd(None, None) == NULL


def _dec(**kw):
    a = mm.DecodeArgs()
    a.q = a.k_cache = a.v_cache = a.out = FAKE
    a.dtype = 1
    a.B, a.Hq, a.Hkv, a.kv_len, a.Scap, a.D = 1, 32, 32, 100, 128, 128
    a.scale = 0.08837890625
    a.q_strides = mm._I64x2(32 * 128, 128)
    a.kv_strides = mm._I64x3(32 * 128 * 128, 128 * 128, 128)
    a.o_strides = mm._I64x2(32 * 128, 128)
    a.workspace = FAKE
    a.workspace_bytes = 1 << 30
    for key, val in kw.items():
        setattr(a, key, val)
    return mm.load_library().mm_attn_decode(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NULL),
    (dict(v_cache=None), NULL),
    (dict(dtype=0), DTYPE),
    (dict(Hq=30, Hkv=8), SHAPE),
    (dict(kv_len=200), SHAPE),
    (dict(kv_len=-1), SHAPE),
    (dict(D=80), UNSUP),
    (dict(num_splits=-2), UNSUP),
    (dict(num_splits=100000), UNSUP),
    (dict(kv_strides=mm._I64x3(0, -128, 128)), STRIDE),
    (dict(kv_strides=mm._I64x3(0, 128, 130)), STRIDE),
    (dict(k_cache=FAKE + 8), STRIDE),
    (dict(workspace=None), WORKSPACE),
    (dict(workspace_bytes=16), WORKSPACE),
    (dict(B=0), OK),
])
def test_decode_rejects_before_launch(kw, status):
    assert _dec(**kw) == status


def test_decode_workspace_and_splits():
    # 1 x 32 heads x 32 splits x (128 + 2) floats
    assert mm.decode_auto_splits(1, 32, 32768) == 32
    assert mm.decode_workspace_size(1, 32, 32768, 128) == 32 * 32 * 130 * 4
    assert mm.decode_workspace_size(1, 32, 32768, 128, num_splits=3) == 32 * 3 * 130 * 4
    assert mm.decode_auto_splits(1, 32, 1) == 1
    assert mm.decode_auto_splits(1, 32, 0) == 1
    assert mm.decode_workspace_size(1, 32, 100, 96) == 0
    # no more splits than 256-key chunks, at most 256 splits
    for B, L in [(1, 1000), (8, 4096), (1, 10 ** 7), (64, 32768)]:
        s = mm.decode_auto_splits(B, 32, L)
        assert 1 <= s <= min(256, -(-L // 256))


@pytest.mark.parametrize("args,status", [
    ((4, 0, 128, 128, FAKE, 2), UNSUP),          # row drop is not a block predicate
    ((8, 0, 128, 128, FAKE, 2), UNSUP),
    ((2, -1, 128, 128, FAKE, 2), SHAPE),         # window < 0
    ((1, 0, -1, 128, FAKE, 2), SHAPE),
    ((1, 0, 128, 128, None, 2), NULL),
    ((1, 0, 128, 129, FAKE, 2), STRIDE),         # ld below ceil(129/64) = 3
    ((1, 0, 0, 128, None, 0), OK),               # nothing to write
    ((3, 5, 128, 0, None, 0), OK),
])
def test_block_mask_create_rejects_before_launch(args, status):
    lib = mm.load_library()
    fl, w, sq, skv, out, ld = args
    assert lib.mm_block_mask_create(fl, w, sq, skv, out, ld, None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3, descale_q=1.0, descale_k=1.0, descale_v=1.0, q_strides=mm._I64x3(4 * 16 * 128, 16 * 128, 136)), STRIDE),
    (dict(dtype=3, descale_q=0.0, descale_k=1.0, descale_v=1.0), SHAPE),
    (dict(dtype=3, descale_q=1.0, descale_k=float("nan"), descale_v=1.0), SHAPE),
    (dict(dtype=3, descale_q=1.0, descale_k=1.0, descale_v=-2.0), SHAPE),
    (dict(dtype=3, descale_q=1.0, descale_k=1.0, descale_v=1.0, Sq=0), OK),
    # 16-bit inputs ignore the descale fields: with zeros there the call still gets as
    # far as the stride check (a bad stride keeps it on the host)
    (dict(dtype=2, descale_q=0.0, q_strides=mm._I64x3(-1, 0, 0)), STRIDE),
])
def test_fp8_args_rejected_before_launch(kw, status):
    assert _fwd(**kw) == status


def test_decode_splits_count_head_groups():
    """With GQA a split workgroup serves up to 4 query heads. The automatic split count
    aims at 1024 workgroups with one head per workgroup and 512 with 2 or 4, rounding
    down; when a kv head's group spans several workgroups it is a multiple of 8."""
    assert mm.decode_auto_splits(1, 32, 32768, Hkv=8) == 64       # group 4: 8 head groups, 512 / 8
    assert mm.decode_auto_splits(1, 32, 32768, Hkv=4) == 64       # group 8: two workgroups of 4 per kv head
    assert mm.decode_auto_splits(1, 32, 32768, Hkv=16) == 32      # group 2: 16 head groups, 512 / 16
    assert mm.decode_auto_splits(1, 32, 32768, Hkv=32) == 32      # one head per workgroup, 1024 / 32
    assert mm.decode_auto_splits(2, 24, 8192, Hkv=8) == 16        # group 3: one head each, 1024 // 48 = 21 -> 16
    assert mm.decode_auto_splits(8, 32, 32768, Hkv=32) == 4
    assert mm.decode_workspace_size(1, 32, 32768, 128, Hkv=8) == 32 * 64 * 130 * 4
    assert mm.load_library().mm_attn_decode_auto_splits(1, 32, 5, 100) == 0  # Hq % Hkv != 0


def test_decode_auto_splits_properties():
    """Over many shapes: at most one round of split workgroups (1024 with one head per
    workgroup, 512 with 2 or 4), never more splits than 256-key chunks or 256, and a
    multiple of 8 whenever a kv head's group spans several workgroups."""
    for B in (1, 2, 3, 8, 64):
        for Hq, Hkv in ((32, 32), (32, 16), (32, 8), (32, 4), (24, 8), (48, 8), (64, 4), (40, 5), (7, 1)):
            for L in (1, 255, 256, 1000, 8192, 32768, 262144):
                s = mm.decode_auto_splits(B, Hq, L, Hkv=Hkv)
                group = Hq // Hkv
                G = next(g for g in (4, 2, 1) if group % g == 0)
                assert 1 <= s <= min(256, -(-L // 256)), (B, Hq, Hkv, L, s)
                if s > 1:
                    assert (B * Hq // G) * s <= (1024 if G == 1 else 512), (B, Hq, Hkv, L, s)
                if group > G and s >= 8:
                    assert s % 8 == 0, (B, Hq, Hkv, L, s)


@pytest.mark.parametrize("page_size,stride,status", [(12, 64, SHAPE), (0, 64, SHAPE), (16, -1, STRIDE),
                                                     (16, 2, STRIDE)])
def test_decode_rejects_bad_page_tables(page_size, stride, status):
    # B = 2 with Scap = 128: 8 pages of 16 per sequence
    assert _dec(B=2, Scap=128, kv_len=100, block_table=FAKE, page_size=page_size,
                block_table_stride=stride) == status


DOC = dict(mods_mask_flags=8, mods_q_doc_ids=FAKE, mods_kv_doc_ids=FAKE + 64)
BAD_Q_STRIDE = dict(q_strides=mm._I64x3(-1, 0, 0))


@pytest.mark.parametrize("kw,status", [
    (dict(mods_mask_flags=8), NULL),                               # ids missing
    (dict(DOC, mods_kv_doc_ids=None), NULL),
    (dict(DOC, mods_mask_flags=8 | 2, mods_window=4, **BAD_Q_STRIDE), STRIDE),  # with the window
    (dict(DOC, mods_doc_strides=mm._I64x2(0, -16)), STRIDE),
    (dict(DOC, mods_q_doc_ids=FAKE + 2), STRIDE),                  # int32 alignment
    (dict(DOC, **BAD_Q_STRIDE), STRIDE),                           # ids accepted: reaches the stride check
    (dict(DOC, mods_mask_flags=8 | 1 | 4, **BAD_Q_STRIDE), STRIDE),
    (dict(mods_mask_flags=8, Sq=0), OK),                           # no pair: ids not needed
])
def test_document_mask_args_rejected_before_launch(kw, status):
    assert _fwd(**kw) == status


def _bwd(**kw):
    a = mm.BwdArgs()
    a.q = a.k = a.v = a.out = a.dout = a.lse = a.dq = a.dk = a.dv = FAKE
    a.dtype = 2
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = 1, 4, 2, 16, 16, 128
    for name, h in (("q", 4), ("k", 2), ("v", 2), ("o", 4), ("do", 4), ("dq", 4), ("dk", 2), ("dv", 2)):
        setattr(a, name + "_strides", mm._I64x3(h * 16 * 128, 16 * 128, 128))
    a.scale = 0.1
    a.workspace = FAKE
    a.workspace_bytes = 1 << 20
    for key, val in kw.items():
        if key.startswith("mods_"):
            setattr(a.mods, key[5:], val)
        else:
            setattr(a, key, val)
    return mm.load_library().mm_attn_bwd(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,status", [
    (dict(dq=None), NULL),
    (dict(dk=None), NULL),
    (dict(dtype=0), DTYPE),                      # the backward is 16-bit only
    (dict(dtype=3), DTYPE),
    (dict(Hq=3), SHAPE),
    (dict(Sq=1 << 30), SHAPE),
    (dict(Skv=1 << 30), SHAPE),
    (dict(D=32), UNSUP),
    (dict(mods_mask_flags=16), UNSUP),
    (dict(do_strides=mm._I64x3(0, 0, 12)), STRIDE),
    (dict(dv=FAKE + 4), STRIDE),
    (dict(workspace=None), WORKSPACE),
    (dict(workspace_bytes=8), WORKSPACE),
    (dict(mods_mask_flags=8), NULL),
    (dict(DOC, mods_mask_flags=8 | 2, do_strides=mm._I64x3(0, 0, 12)), STRIDE),
    (dict(DOC, mods_doc_strides=mm._I64x2(-1, 0)), STRIDE),
    (dict(DOC, do_strides=mm._I64x3(0, 0, 12)), STRIDE),
    (dict(B=0), OK),
])
def test_bwd_rejects_before_launch(kw, status):
    assert _bwd(**kw) == status


def test_bwd_workspace_size():
    # lse2 and D per row, rows padded to 64 per (b, h)
    assert mm.bwd_workspace_size(2, 3, 100) == 2 * 2 * 3 * 128 * 4
    assert mm.bwd_workspace_size(1, 1, 0) == 0


def test_decode_varlen_splits():
    """With per-sequence lengths the automatic split count is raised towards what a batch
    of one sequence gets (one sequence may hold nearly all the keys), keeping the split
    workgroups within 8 resident rounds; the workspace size covers that count."""
    assert mm.decode_auto_splits(8, 32, 32768, varlen=True) == 32      # as B = 1: 1024 / 32
    assert mm.decode_auto_splits(8, 32, 32768) == 4
    assert mm.decode_workspace_size(8, 32, 32768, 128) == 8 * 32 * 32 * 130 * 4
    assert mm.decode_auto_splits(64, 32, 32768, varlen=True) == 4      # 8192 / 2048 rows
    assert mm.decode_auto_splits(8, 32, 32768, Hkv=8, varlen=True) == 64  # G 4: 512 / 8, 4096 / 64 rows
    assert mm.load_library().mm_attn_decode_auto_splits_varlen(1, 32, 5, 100) == 0
    for B in (1, 2, 3, 8, 64, 1000):
        for Hq, Hkv in ((32, 32), (32, 8), (32, 4), (24, 8), (7, 1)):
            for L in (1, 255, 1000, 32768, 262144):
                s0 = mm.decode_auto_splits(B, Hq, L, Hkv=Hkv)
                s1 = mm.decode_auto_splits(B, Hq, L, Hkv=Hkv, varlen=True)
                group = Hq // Hkv
                G = next(g for g in (4, 2, 1) if group % g == 0)
                assert s1 >= s0 and 1 <= s1 <= min(256, -(-L // 256)), (B, Hq, Hkv, L, s0, s1)
                if B == 1:
                    assert s1 == s0
                if s1 > s0:
                    assert (B * Hq // G) * s1 <= 8 * (1024 if G == 1 else 512)
                if group > G and s1 >= 8:
                    assert s1 % 8 == 0
                for D in (64, 128):
                    assert mm.decode_workspace_size(B, Hq, L, D, Hkv=Hkv) == B * Hq * s1 * (D + 2) * 4
                    # the raised count never pushes a call past the static scratch
                    if B * Hq * s0 * (D + 2) * 4 <= mm.DECODE_SCRATCH_BYTES:
                        assert B * Hq * s1 * (D + 2) * 4 <= mm.DECODE_SCRATCH_BYTES


def test_decode_noalloc_rejects_oversize_before_any_device_work():
    """mm_attn_decode_noalloc refuses, before touching a device, a call whose partials
    exceed the static scratch; calls with nothing to do return OK."""
    lib = mm.load_library()
    a = mm.DecodeArgs()
    a.q = a.k_cache = a.v_cache = a.out = FAKE
    a.dtype = 1
    a.B, a.Hq, a.Hkv, a.kv_len, a.Scap, a.D = 4, 32, 32, 8192, 8192, 128
    a.scale = 0.088
    a.q_strides = mm._I64x2(32 * 128, 128)
    a.kv_strides = mm._I64x3(32 * 8192 * 128, 8192 * 128, 128)
    a.o_strides = mm._I64x2(32 * 128, 128)
    a.num_splits = 256  # 4*32*256*130*4 bytes > 16 MiB
    assert 4 * 32 * 256 * 130 * 4 > mm.DECODE_SCRATCH_BYTES
    assert lib.mm_attn_decode_noalloc(ctypes.byref(a), None) == WORKSPACE
    a.B = 0
    assert lib.mm_attn_decode_noalloc(ctypes.byref(a), None) == OK
    a.B, a.D = 4, 96
    assert lib.mm_attn_decode_noalloc(ctypes.byref(a), None) == UNSUP
