"""GPU parity of the backward (mm_attn_bwd through the C ABI) against the oracle.

The kernel backward consumes the kernel forward's O and LSE (as training does); the
oracle computes its own forward in fp64. Every case prints its parameters first so a
failing GPU step names itself.
"""
import math

import numpy as np
import pytest

import oracle
from helpers import O_ATOL, O_RTOL, assert_parity, to_f64, to_torch
from mask_mods_amd import inputs

pytestmark = pytest.mark.gpu

RD = (20240, int(0.05 * 2 ** 32))


def _grads(B, Hq, Hkv, Sq, Skv, D, dtype, *, causal=False, window=None, alibi=False,
           rowdrop=False, block_mask=None, q_doc=None, kv_doc=None, seed=0, scale=None):
    """Run forward + backward on the GPU; return device grads and the f64 inputs."""
    import torch
    import mask_mods_amd as mm
    print(f"[bwd] B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Skv={Skv} D={D} {dtype} causal={causal} "
          f"window={window} alibi={alibi} rowdrop={rowdrop} block={block_mask is not None} "
          f"docs={None if q_doc is None else int(q_doc.max()) + 1} seed={seed}",
          flush=True)
    x = inputs.attention_inputs(seed, B, Hq, Hkv, Sq, Skv, D, dtype)
    g = inputs.rng(seed + 1000)
    do_bits = inputs.f32_to_bits(g.standard_normal((B, Hq, Sq, D), dtype=np.float32), dtype)
    q, k, v, do = (to_torch(b_, dtype) for b_ in (x["q"], x["k"], x["v"], do_bits))
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    kw = dict(causal=causal, window=window, score_mod=mm.SCORE_ALIBI if alibi else mm.SCORE_NONE,
              rowdrop=RD if rowdrop else None,
              block_mask=torch.from_numpy(block_mask).cuda() if block_mask is not None else None,
              q_doc=_ids(q_doc), kv_doc=_ids(kv_doc))
    out, lse = mm.attn_fwd(q, k, v, scale, **kw)
    dq, dk, dv = mm.attn_bwd(q, k, v, out, lse, do, scale, **kw)
    torch.cuda.synchronize()
    f64 = [inputs.bits_to_f64(b_, dtype) for b_ in (x["q"], x["k"], x["v"], do_bits)]
    return (dq, dk, dv), f64, scale


def _ids(ids):
    import torch
    return None if ids is None else torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()


def _check(B, Hq, Hkv, Sq, Skv, D, dtype, **mods):
    (dq, dk, dv), (qd, kd, vd, dod), scale = _grads(B, Hq, Hkv, Sq, Skv, D, dtype, **mods)
    ref = oracle.attention_bwd(qd, kd, vd, dod, scale=scale, causal=mods.get("causal", False),
                               window=mods.get("window"), alibi=mods.get("alibi", False),
                               rowdrop=RD if mods.get("rowdrop") else None,
                               block_mask=mods.get("block_mask"), q_doc=mods.get("q_doc"),
                               kv_doc=mods.get("kv_doc"))
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        err = assert_parity(to_f64(got), want, O_ATOL, O_RTOL, name)
        print(f"[bwd] {name} max|err| {err:.3e} max|ref| {np.abs(want).max():.3e}", flush=True)
    return dq, dk, dv


CASES = {
    "none": dict(),
    "causal": dict(causal=True),
    "alibi": dict(alibi=True),
    "alibi_causal": dict(alibi=True, causal=True),
    "sliding_window": dict(window=64, causal=True),
    "window_only": dict(window=40),
    "rowdrop": dict(rowdrop=True, causal=True),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_matrix(dtype, D, case):
    _check(1, 2, 2, 250, 250, D, dtype, seed=1, **CASES[case])


@pytest.mark.parametrize("D", [64, 128])
def test_int32_max_window_with_causal(D):
    """A window of 2**31 - 1 together with causal keeps exactly the causal pairs (its
    bound arithmetic must not wrap into an empty key range): the gradients match the
    oracle's, and the plain causal backward's."""
    import torch
    W = 2 ** 31 - 1
    g1 = _check(1, 2, 2, 300, 300, D, "bf16", seed=41, causal=True, window=W)
    (g2, _, _) = _grads(1, 2, 2, 300, 300, D, "bf16", seed=41, causal=True)
    for a, b_ in zip(g1, g2):
        assert torch.allclose(a.float(), b_.float(), atol=2e-2, rtol=2e-2)
        assert a.abs().max() > 0


def test_multi_tile_1024():
    _check(1, 2, 2, 1024, 1024, 128, "bf16", seed=2, causal=True, alibi=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_gqa(dtype):
    _check(2, 8, 2, 300, 300, 128, dtype, seed=3, causal=True, alibi=True)
    _check(1, 8, 1, 129, 257, 64, dtype, seed=4, window=33)


@pytest.mark.parametrize("shape,mods", [
    ((200, 700), dict(alibi=True)),
    ((700, 200), dict(causal=True)),
    ((129, 1000), dict(window=40)),
    ((1, 300), dict()),
    ((300, 1), dict(causal=True)),
    ((600, 130), dict(causal=True, window=100)),  # rows >= 231 see no key
])
def test_cross_attention(shape, mods):
    Sq, Skv = shape
    _check(1, 4, 2, Sq, Skv, 128, "bf16", seed=5, **mods)


@pytest.mark.parametrize("pred", ["none", "causal"])
def test_block_mask(pred):
    S = 384
    bm = inputs.random_block_mask(6, (1, 4, -(-S // 128), -(-S // 64)))
    _check(1, 4, 2, S, S, 128, "bf16", seed=6, block_mask=bm, **({"causal": True} if pred == "causal" else {}))


def test_block_mask_sparse_gqa_ragged():
    """A mostly empty table (90% of blocks empty) with GQA group 4 and ragged lengths:
    a dK/dV workgroup visits only its non-empty (query head, query tile) items, and with
    4 heads x 18 query tiles per key block it walks more than one 64-item window."""
    Sq, Skv = 1100, 1060
    bm = inputs.random_block_mask(41, (1, 8, -(-Sq // 128), -(-Skv // 64)), p_empty=0.9, p_full=0.05)
    _check(1, 8, 2, Sq, Skv, 64, "bf16", seed=41, block_mask=bm)


def test_block_mask_per_batch_broadcast_over_heads():
    """A table per batch, broadcast over heads (head stride 0), with causal."""
    S = 500
    bm = inputs.random_block_mask(42, (2, 1, -(-S // 128), -(-S // 64)), p_empty=0.5, p_full=0.25)
    _check(2, 4, 2, S, S, 128, "bf16", seed=42, causal=True, block_mask=bm)


def test_block_mask_all_empty():
    """Every block empty: no item is visited, every gradient is zero."""
    import torch
    S = 300
    bm = np.zeros((1, 1, -(-S // 128), -(-S // 64)), dtype=np.uint8)
    dq, dk, dv = _check(1, 4, 2, S, S, 64, "bf16", seed=43, block_mask=bm)
    for t in (dq, dk, dv):
        assert torch.count_nonzero(t).item() == 0


def test_created_causal_classes_match_plain_causal_bitwise():
    import torch
    import mask_mods_amd as mm
    S = 700
    bm = mm.block_mask_create(S, S, causal=True)
    ga, _, _ = _grads(1, 2, 2, S, S, 128, "bf16", seed=7, causal=True, block_mask=bm.cpu().numpy())
    gb, _, _ = _grads(1, 2, 2, S, S, 128, "bf16", seed=7, causal=True)
    for x, y in zip(ga, gb):
        assert torch.equal(x, y)


def test_fully_masked_rows_and_empty_keys():
    dq, _, _ = _check(1, 2, 2, 600, 130, 64, "bf16", seed=8, causal=True, window=100)
    assert np.all(to_f64(dq)[:, :, 231:] == 0)
    import torch
    import mask_mods_amd as mm
    q = torch.randn(1, 2, 40, 128, device="cuda", dtype=torch.bfloat16)
    k = torch.empty(1, 2, 0, 128, device="cuda", dtype=torch.bfloat16)
    out, lse = mm.attn_fwd(q, k, k.clone(), 0.1)
    dq, dk, dv = mm.attn_bwd(q, k, k.clone(), out, lse, torch.randn_like(q), 0.1)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.numel() == 0


def test_deterministic():
    import torch
    g1, _, _ = _grads(1, 4, 2, 512, 512, 128, "bf16", seed=9, causal=True)
    g2, _, _ = _grads(1, 4, 2, 512, 512, 128, "bf16", seed=9, causal=True)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_config_2048_sampled_heads(causal):
    """B2 H32 D128 S2048 on the GPU; the oracle recomputes two (b, h) heads in full."""
    B, H, S, D = 2, 32, 2048, 128
    (dq, dk, dv), (qd, kd, vd, dod), scale = _grads(B, H, H, S, S, D, "bf16", seed=10, causal=causal)
    for b, h in ((0, 0), (1, 31)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.attention_bwd(qd[sl], kd[sl], vd[sl], dod[sl], scale=scale, causal=causal)
        for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert_parity(to_f64(got[sl]), want, O_ATOL, O_RTOL, f"{name}[{b},{h}]")


# ------------------------------------------------------------ document mask
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_document_mask(dtype, D, causal):
    docs = inputs.packed_document_ids(30, 2, 300, 5)
    _check(2, 4, 2, 300, 300, D, dtype, seed=30, causal=causal, q_doc=docs)


def test_document_mask_tile_aligned_and_single_token_documents():
    docs = inputs.document_ids_from_lengths([64, 1, 63, 128, 1, 200, 55], 512)[None]
    _check(1, 4, 4, 512, 512, 128, "bf16", seed=31, causal=True, alibi=True, q_doc=docs)


def test_document_mask_cross_attention_with_a_document_without_keys():
    """Query document 2 has no keys and key document 4 no queries: zero gradients there."""
    qd = inputs.document_ids_from_lengths([90, 70, 40, 100], 300)[None]
    kd = np.concatenate([inputs.document_ids_from_lengths([200, 150], 350),
                         np.full(300, 3, np.int32), np.full(50, 4, np.int32)])[None]
    dq, dk, dv = _check(1, 4, 2, 300, 700, 128, "bf16", seed=32, q_doc=qd, kv_doc=kd)
    assert np.all(to_f64(dq)[:, :, 160:200] == 0)
    # key document 4 has no query rows
    assert np.all(to_f64(dk)[:, :, 650:] == 0) and np.all(to_f64(dv)[:, :, 650:] == 0)


def test_document_mask_with_block_mask():
    S = 384
    bm = inputs.random_block_mask(33, (1, 4, -(-S // 128), -(-S // 64)))
    docs = inputs.packed_document_ids(33, 1, S, 4)
    _check(1, 4, 2, S, S, 128, "bf16", seed=33, causal=True, block_mask=bm, q_doc=docs)


def test_document_mask_rowdrop_gqa():
    docs = inputs.packed_document_ids(34, 2, 257, 3)
    _check(2, 8, 2, 257, 257, 64, "f16", seed=34, causal=True, rowdrop=True, q_doc=docs)


def test_document_mask_2048_sampled_heads():
    """B2 H16 D128 S2048 causal with 12 packed documents; two heads recomputed in full."""
    B, H, S, D = 2, 16, 2048, 128
    docs = inputs.packed_document_ids(35, B, S, 12)
    (dq, dk, dv), (qd, kd, vd, dod), scale = _grads(B, H, H, S, S, D, "bf16", seed=35, causal=True,
                                                    q_doc=docs)
    for b, h in ((0, 3), (1, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.attention_bwd(qd[sl], kd[sl], vd[sl], dod[sl], scale=scale, causal=True,
                                   q_doc=docs[b:b + 1])
        for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert_parity(to_f64(got[sl]), want, O_ATOL, O_RTOL, f"{name}[{b},{h}]")


def test_document_mask_sparse_ids():
    base = inputs.packed_document_ids(36, 1, 300, 5)[0]
    docs = np.array([-9, 3, 4, 70000, 2 ** 31 - 1], dtype=np.int64)[base].astype(np.int32)[None]
    _check(1, 2, 2, 300, 300, 64, "bf16", seed=36, causal=True, q_doc=docs)


@pytest.mark.parametrize("causal", [False, True])
def test_config_8192_one_sampled_head(causal):
    """B2 H32 D128 S8192, the shape bench.py times, on the GPU; the oracle recomputes one
    full (b, h) head (about half a minute of CPU)."""
    B, H, S, D = 2, 32, 8192, 128
    (dq, dk, dv), (qd, kd, vd, dod), scale = _grads(B, H, H, S, S, D, "bf16", seed=37, causal=causal)
    b, h = (1, 17) if causal else (0, 6)
    sl = (slice(b, b + 1), slice(h, h + 1))
    ref = oracle.attention_bwd(qd[sl], kd[sl], vd[sl], dod[sl], scale=scale, causal=causal)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        err = assert_parity(to_f64(got[sl]), want, O_ATOL, O_RTOL, f"{name}[{b},{h}]")
        print(f"[bwd] 8192 {name} max|err| {err:.3e}", flush=True)



@pytest.mark.parametrize("causal", [False, True])
def test_document_mask_with_window(causal):
    docs = inputs.packed_document_ids(38, 1, 384, 4)
    _check(1, 4, 2, 384, 384, 128, "bf16", seed=38, window=70, causal=causal, q_doc=docs)
