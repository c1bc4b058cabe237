"""GPU parity of the document mask -- a mask_mod that captures per-position document ids
(packed sequences) -- in the forward through the C ABI against the oracle: the 16-bit
MFMA kernels, the fp32 kernel, the fp8 kernel, with the other mods and the block mask.
The backward's document cases sit with the other backward tests.

Every case prints its parameters first so a failing GPU step names itself.
"""
import math

import numpy as np
import pytest

import oracle
from helpers import (F32_ATOL, F32_RTOL, LSE_ATOL, LSE_RTOL, O_ATOL, O_RTOL, assert_parity,
                     to_f64, to_torch)
from mask_mods_amd import inputs

pytestmark = pytest.mark.gpu

RD = (20240, int(0.05 * 2 ** 32))


def _ids(ids):
    import torch
    return None if ids is None else torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()


def _run(B, Hq, Hkv, Sq, Skv, D, dtype, q_doc, kv_doc=None, *, causal=False, alibi=False,
         rowdrop=False, block_mask=None, window=None, seed=0, rows=None):
    """q_doc / kv_doc: int32 numpy [B|1, S] (kv_doc None: the query ids serve both)."""
    import torch
    import mask_mods_amd as mm
    print(f"[doc] B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Skv={Skv} D={D} {dtype} q_doc={q_doc.shape} "
          f"kv_doc={None if kv_doc is None else kv_doc.shape} causal={causal} alibi={alibi} "
          f"rowdrop={rowdrop} block={block_mask is not None} window={window} seed={seed}", flush=True)
    x = inputs.attention_inputs(seed, B, Hq, Hkv, Sq, Skv, D, dtype)
    q, k, v = (to_torch(x[n], dtype) for n in ("q", "k", "v"))
    scale = float(np.float32(1.0 / math.sqrt(D)))
    bm = torch.from_numpy(block_mask).cuda() if block_mask is not None else None
    out, lse = mm.attn_fwd(q, k, v, scale, causal=causal, window=window,
                           score_mod=mm.SCORE_ALIBI if alibi else mm.SCORE_NONE,
                           rowdrop=RD if rowdrop else None, block_mask=bm,
                           q_doc=_ids(q_doc), kv_doc=_ids(kv_doc))
    torch.cuda.synchronize()
    qd, kd, vd = (inputs.bits_to_f64(x[n], dtype) for n in ("q", "k", "v"))
    od = np.broadcast_to(q_doc, (B, q_doc.shape[1]))
    kdoc = od if kv_doc is None else np.broadcast_to(kv_doc, (B, kv_doc.shape[1]))
    O, L = oracle.attention(qd, kd, vd, scale=scale, causal=causal, alibi=alibi, window=window,
                            rowdrop=RD if rowdrop else None, rows=rows, block_mask=block_mask,
                            q_doc=od, kv_doc=kdoc)
    got_o, got_l = to_f64(out), to_f64(lse)
    if rows is not None:
        got_o, got_l = got_o.reshape(-1, D)[rows], got_l.reshape(-1)[rows]
    if dtype == "f32":
        assert_parity(got_o, O, F32_ATOL, F32_RTOL, "O")
        assert_parity(got_l, L, F32_ATOL, F32_RTOL, "LSE")
    else:
        assert_parity(got_o, O, O_ATOL, O_RTOL, "O")
        assert_parity(got_l, L, LSE_ATOL, LSE_RTOL, "LSE")
    return out, lse


CASES = {
    "none": dict(),
    "causal": dict(causal=True),
    "alibi_causal": dict(alibi=True, causal=True),
    "rowdrop_causal": dict(rowdrop=True, causal=True),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_matrix(dtype, D, case):
    """700 positions (5 query tiles of 128 + a ragged 60), 6 documents per sequence,
    different cuts in the two sequences, GQA 4:2."""
    docs = inputs.packed_document_ids(1, 2, 700, 6)
    _run(2, 4, 2, 700, 700, D, dtype, docs, seed=1, **CASES[case])


@pytest.mark.parametrize("causal", [False, True])
def test_tile_aligned_boundaries_and_single_token_documents(causal):
    docs = inputs.document_ids_from_lengths([128, 1, 63, 64, 1, 1, 254, 188], 700)[None]
    _run(1, 2, 2, 700, 700, 128, "bf16", docs, seed=2, causal=causal)


def test_many_short_documents():
    """200 documents over 1024 positions: most tiles straddle several documents."""
    docs = inputs.packed_document_ids(3, 1, 1024, 200)
    _run(1, 4, 4, 1024, 1024, 128, "bf16", docs, seed=3, causal=True)


def test_one_token_per_document():
    """Every position its own document: each row keeps exactly its own key."""
    docs = np.arange(300, dtype=np.int32)[None]
    out, lse = _run(1, 2, 2, 300, 300, 64, "bf16", docs, seed=4)


@pytest.mark.parametrize("D,causal", [(64, False), (64, True), (128, False), (128, True)])
def test_single_document_is_bitwise_the_unmasked_kernel(D, causal):
    """One document covering the sequence keeps every pair the other predicates keep; the
    kernel then takes the same tiles and code path as without the document mask, to the
    bit. Except at D 128 without causal: the unmasked forward there runs the
    software-pipelined kernel (other summation order), held to the parity bar instead."""
    import torch
    import mask_mods_amd as mm
    S = 900
    x = inputs.attention_inputs(5, 1, 4, 2, S, S, D, "bf16")
    q, k, v = (to_torch(x[n], "bf16") for n in ("q", "k", "v"))
    docs = _ids(np.full((1, S), 7, np.int32))
    o1, l1 = mm.attn_fwd(q, k, v, 0.09, causal=causal, q_doc=docs)
    o2, l2 = mm.attn_fwd(q, k, v, 0.09, causal=causal)
    torch.cuda.synchronize()
    if D == 128 and not causal:
        assert_parity(to_f64(o1), to_f64(o2), O_ATOL, O_RTOL, "O")
        assert_parity(to_f64(l1), to_f64(l2), LSE_ATOL, LSE_RTOL, "LSE")
    else:
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_cross_attention_with_unmatched_documents():
    """Query document 2 has no keys (rows fully masked: O = 0, LSE = -inf); key
    document 4 has no queries."""
    qd = inputs.document_ids_from_lengths([90, 70, 40, 100], 300)[None]
    kd = np.concatenate([inputs.document_ids_from_lengths([200, 150], 350),
                         np.full(300, 3, np.int32), np.full(50, 4, np.int32)])[None]
    out, lse = _run(1, 4, 2, 300, 700, 128, "bf16", qd, kd, seed=6)
    assert np.all(to_f64(lse)[:, :, 160:200] == -np.inf)
    assert np.all(to_f64(out)[:, :, 160:200] == 0)


def test_cross_attention_causal_gqa():
    qd = inputs.packed_document_ids(7, 2, 257, 3)
    kd = inputs.packed_document_ids(8, 2, 513, 3)
    _run(2, 8, 2, 257, 513, 64, "f16", qd, kd, seed=7, causal=True, alibi=True)


def test_broadcast_ids_over_the_batch():
    docs = inputs.packed_document_ids(9, 1, 500, 4)
    _run(3, 2, 1, 500, 500, 128, "bf16", docs, seed=9, causal=True)


@pytest.mark.parametrize("pred", ["none", "causal"])
def test_with_block_mask(pred):
    """Partial blocks apply the document mask with the other predicates; full blocks
    bypass it (the block mask's contract), empty blocks are skipped."""
    S = 700
    bm = inputs.random_block_mask(10, (1, 4, -(-S // 128), -(-S // 64)))
    docs = inputs.packed_document_ids(10, 1, S, 5)
    _run(1, 4, 4, S, S, 128, "bf16", docs, seed=10, block_mask=bm, causal=pred == "causal")


def test_all_partial_blocks_with_documents_match_plain_bitwise():
    """Every block partial: the kernel visits every key tile and lets the predicates
    (here causal and the documents) decide, so it processes the same tiles, in the same
    order and on the same code paths, as the unblocked kernel that narrows its key range
    from the document ids. (A full block would bypass the document test as well: a
    block mask built from causality alone does not describe documents.)"""
    import torch
    import mask_mods_amd as mm
    S = 1000
    x = inputs.attention_inputs(11, 1, 2, 2, S, S, 128, "bf16")
    q, k, v = (to_torch(x[n], "bf16") for n in ("q", "k", "v"))
    docs = _ids(inputs.packed_document_ids(11, 1, S, 6))
    bm = torch.ones((1, 1, -(-S // 128), -(-S // 64)), dtype=torch.uint8, device="cuda")
    o1, l1 = mm.attn_fwd(q, k, v, 0.09, causal=True, q_doc=docs, block_mask=bm)
    o2, l2 = mm.attn_fwd(q, k, v, 0.09, causal=True, q_doc=docs)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_f32_kernel(causal):
    docs = inputs.packed_document_ids(12, 2, 300, 4)
    _run(2, 2, 1, 300, 300, 64, "f32", docs, seed=12, causal=causal, alibi=True)


def test_f32_kernel_with_block_mask():
    S = 300
    bm = inputs.random_block_mask(13, (1, 2, -(-S // 128), -(-S // 64)))
    docs = inputs.packed_document_ids(13, 1, S, 3)
    _run(1, 2, 2, S, S, 128, "f32", docs, seed=13, block_mask=bm, causal=True)


@pytest.mark.parametrize("causal", [False, True])
def test_config_8192_sampled(causal):
    """B2 H32 D128 S8192 with 16 packed documents per sequence, on sampled rows."""
    B, H, S, D = 2, 32, 8192, 128
    docs = inputs.packed_document_ids(14, B, S, 16)
    rows = inputs.sample_rows(14, B, H, S, n_random=64)
    _run(B, H, H, S, S, D, "bf16", docs, seed=14, causal=causal, rows=rows)


@pytest.mark.parametrize("causal", [False, True])
def test_sparse_negative_and_large_ids(causal):
    """Ids need only be non-decreasing: gaps, negative values and values near the int32
    limit behave like 0, 1, 2, ... (the kernels visit only the ids present)."""
    base = inputs.packed_document_ids(15, 1, 600, 7)[0]
    remap = np.array([-2 ** 31, -7, 0, 1000, 10 ** 6, 2 ** 30, 2 ** 31 - 1], dtype=np.int64)
    docs = remap[base].astype(np.int32)[None]
    _run(1, 2, 2, 600, 600, 128, "bf16", docs, seed=15, causal=causal)



@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [40, 300])
def test_with_sliding_window(window, causal):
    """Documents AND a window: the key range is the intersection of both, and tiles
    straddling a document or the band test each pair against both."""
    docs = inputs.packed_document_ids(16, 2, 700, 5)
    _run(2, 4, 2, 700, 700, 128, "bf16", docs, seed=16, window=window, causal=causal)


def test_with_sliding_window_f16_d64_alibi():
    docs = inputs.packed_document_ids(17, 1, 513, 4)
    _run(1, 4, 4, 513, 513, 64, "f16", docs, seed=17, window=64, causal=True, alibi=True)


def test_with_sliding_window_and_block_mask():
    S = 700
    bm = inputs.random_block_mask(18, (1, 2, -(-S // 128), -(-S // 64)))
    docs = inputs.packed_document_ids(18, 1, S, 4)
    _run(1, 2, 2, S, S, 128, "bf16", docs, seed=18, window=100, causal=True, block_mask=bm)


def test_with_sliding_window_f32():
    docs = inputs.packed_document_ids(19, 1, 300, 3)
    _run(1, 2, 1, 300, 300, 64, "f32", docs, seed=19, window=50)
