"""GPU parity of the fp8 (e4m3) forward through the C ABI against the oracle.

The oracle computes the exact attention of the real tensors descale_x * X8 (decoded
exactly to float64). The kernel rounds the probabilities to e4m3 before the PV product,
so two kinds of cases are checked:

* integer scores: Q8 and K8 in {-1, 0, 1} with at most 4 nonzero products per score and
  scale = ln 2, so every probability 2^(score - running max) lies in [2^-8, 2^8] and is
  an exact e4m3 value. The kernel's only rounding is then fp32 accumulation and the
  bf16 output: the 16-bit bar (2e-2 on O, 1e-3 on LSE) applies unchanged.
* N(0,1) inputs quantised per tensor: each probability carries a relative rounding error
  e_j with |e_j| <= 2^-4 (round to nearest even, 3 mantissa bits), uniform for random
  inputs, so of standard deviation 2^-4/sqrt(3). The row sum is taken over the rounded
  values, so to first order O_d moves by sum_j e_j w_j (V[j,d] - O_d) and LSE by
  sum_j e_j w_j; the oracle returns sqrt(wvar) and sqrt(wsq), the scales of those sums.
  The bound is 6 standard deviations of that error, plus the bf16 output rounding
  (2^-8 relative) and 2e-3 absolute for probabilities below e4m3's normal range
  (absolute error <= 2^-10 against a row maximum >= 1).
"""
import math

import numpy as np
import pytest

import oracle
from helpers import LSE_ATOL, LSE_RTOL, O_ATOL, O_RTOL, assert_parity, to_f64
from mask_mods_amd import inputs

pytestmark = pytest.mark.gpu

SIGMA_E = 2.0 ** -4 / math.sqrt(3)  # std of a uniform relative rounding error in e4m3
RD = (20240, int(0.05 * 2 ** 32))


def _dev8(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).view(torch.float8_e4m3fn).cuda()


def _integer_inputs(seed, B, Hq, Hkv, Sq, Skv, D):
    """Q8 rows with exactly 4 entries of +-1, K8 in {-1, 0, 1}: scores are integers in
    [-4, 4]. V8 from N(0,1) quantised per tensor."""
    g = inputs.rng(seed)
    q = np.zeros((B, Hq, Sq, D))
    idx = np.argsort(g.random((B, Hq, Sq, D)), axis=-1)[..., :4]
    np.put_along_axis(q, idx, g.choice([-1.0, 1.0], size=idx.shape), axis=-1)
    k = g.choice([-1.0, 0.0, 0.0, 1.0], size=(B, Hkv, Skv, D))
    v = g.standard_normal((B, Hkv, Skv, D)).astype(np.float32)
    dv = np.float32(max(float(np.abs(v).max()), 1e-30) / inputs.E4M3_MAX) if v.size else np.float32(1)
    return {"q": inputs.f32_to_e4m3_bits(q), "k": inputs.f32_to_e4m3_bits(k),
            "v": inputs.f32_to_e4m3_bits(np.clip(v / dv, -448, 448)),
            "descale_q": 1.0, "descale_k": 1.0, "descale_v": float(dv)}


def _run(x, D, *, scale, exact, causal=False, window=None, alibi=False, rowdrop=False,
         block_mask=None, q_doc=None, rows=None, label=""):
    import torch
    import mask_mods_amd as mm
    B, Hq, Sq, _ = x["q"].shape
    Skv = x["k"].shape[2]
    print(f"[fp8] {label} shape={x['q'].shape}/{x['k'].shape} exact={exact} causal={causal} "
          f"window={window} alibi={alibi} rowdrop={rowdrop} block={block_mask is not None} "
          f"docs={q_doc is not None}", flush=True)
    dq, dk, dv = x["descale_q"], x["descale_k"], x["descale_v"]
    q, k, v = _dev8(x["q"]), _dev8(x["k"]), _dev8(x["v"])
    bm = torch.from_numpy(block_mask).cuda() if block_mask is not None else None
    out, lse = mm.attn_fwd(q, k, v, scale, causal=causal, window=window,
                           score_mod=mm.SCORE_ALIBI if alibi else mm.SCORE_NONE,
                           rowdrop=RD if rowdrop else None, block_mask=bm, descale=(dq, dk, dv),
                           q_doc=None if q_doc is None else torch.from_numpy(q_doc).cuda())
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    qd = inputs.e4m3_bits_to_f64(x["q"]) * dq
    kd = inputs.e4m3_bits_to_f64(x["k"]) * dk
    vd = inputs.e4m3_bits_to_f64(x["v"]) * dv
    O, L, wsq, wvar = oracle.attention(qd, kd, vd, scale=scale, causal=causal, window=window,
                                       alibi=alibi, rowdrop=RD if rowdrop else None,
                                       block_mask=block_mask, q_doc=q_doc, rows=rows, sensitivity=True)
    got_o, got_l = to_f64(out), to_f64(lse)
    if rows is not None:
        got_o, got_l = got_o.reshape(-1, D)[rows], got_l.reshape(-1)[rows]
    if exact:
        assert_parity(got_o, O, O_ATOL, O_RTOL, "O")
        assert_parity(got_l, L, LSE_ATOL, LSE_RTOL, "LSE")
    else:
        o_tol = 6 * SIGMA_E * np.sqrt(wvar) + 2.0 ** -8 * np.abs(O) + 2e-3
        l_tol = 6 * SIGMA_E * np.sqrt(wsq) + 1e-3
        assert_parity(got_o, O, o_tol, 0.0, "O")
        assert_parity(got_l, L, l_tol, 0.0, "LSE")
        err = np.abs(got_o - O)
        print(f"[fp8] max|dO| {err.max():.3e}  max|dO|/tol {np.max(err / o_tol):.3f}  "
              f"rms dO {np.sqrt(np.mean(err ** 2)):.3e}", flush=True)
    return out, lse


LN2 = float(np.float32(math.log(2.0)))

EXACT_CASES = {
    "none": dict(),
    "causal": dict(causal=True),
    "window_causal": dict(causal=True, window=100),
    "window": dict(window=70),
    "rowdrop_causal": dict(causal=True, rowdrop=True),
}


@pytest.mark.parametrize("case", sorted(EXACT_CASES))
@pytest.mark.parametrize("D", [64, 128])
def test_integer_scores_match_at_16bit_bar(D, case):
    x = _integer_inputs(1, 1, 4, 2, 300, 300, D)
    _run(x, D, scale=LN2, exact=True, label=case, **EXACT_CASES[case])


@pytest.mark.parametrize("Sq,Skv,case", [(200, 1000, "none"), (1000, 130, "causal"), (1, 77, "none"),
                                         (129, 513, "window")])
def test_integer_scores_cross_attention(Sq, Skv, case):
    x = _integer_inputs(2, 2, 4, 1, Sq, Skv, 128)
    _run(x, 128, scale=LN2, exact=True, label=case, **EXACT_CASES[case])


@pytest.mark.parametrize("pred", ["none", "causal"])
def test_integer_scores_block_mask(pred):
    S = 700
    x = _integer_inputs(3, 1, 4, 4, S, S, 128)
    bm = inputs.random_block_mask(3, (1, 4, -(-S // 128), -(-S // 64)))
    _run(x, 128, scale=LN2, exact=True, block_mask=bm, label=pred, **EXACT_CASES[pred])


def test_integer_scores_long_rows():
    x = _integer_inputs(4, 1, 2, 2, 256, 4096, 128)
    _run(x, 128, scale=LN2, exact=True, causal=False, label="long")


RANDOM_CASES = {
    "none": dict(),
    "causal": dict(causal=True),
    "alibi": dict(alibi=True),
    "alibi_causal": dict(alibi=True, causal=True),
    "sliding_window": dict(causal=True, window=256),
}


@pytest.mark.parametrize("case", sorted(RANDOM_CASES))
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [250, 1024])
def test_random_inputs_within_derived_bound(S, D, case):
    x = inputs.attention_inputs_fp8(5, 1, 4, 4, S, S, D)
    _run(x, D, scale=float(np.float32(1 / math.sqrt(D))), exact=False, label=case, **RANDOM_CASES[case])


def test_random_gqa_rowdrop():
    x = inputs.attention_inputs_fp8(6, 2, 8, 2, 384, 640, 128)
    _run(x, 128, scale=float(np.float32(1 / math.sqrt(128))), exact=False, causal=True, rowdrop=True,
         label="gqa")


def test_descale_plumbing():
    """The Q and K factors only multiply the score scale, the V factor only the output."""
    import torch
    import mask_mods_amd as mm
    x = inputs.attention_inputs_fp8(7, 1, 2, 2, 256, 256, 128)
    q, k, v = _dev8(x["q"]), _dev8(x["k"]), _dev8(x["v"])
    o1, l1 = mm.attn_fwd(q, k, v, 0.125, descale=(1.0, 1.0, 1.0))
    o2, l2 = mm.attn_fwd(q, k, v, 0.125, descale=(4.0, 0.25, 1.0))
    o3, l3 = mm.attn_fwd(q, k, v, 0.5, descale=(0.5, 0.5, 8.0))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(l1, l3)
    assert torch.equal(o3.float(), (o1.float() * 8).bfloat16().float())


@pytest.mark.parametrize("causal", [False, True])
def test_config_8192_sampled(causal):
    B, H, S, D = 2, 32, 8192, 128
    x = inputs.attention_inputs_fp8(8, B, H, H, S, S, D)
    rows = inputs.sample_rows(8, B, H, S, n_random=64)
    _run(x, D, scale=float(np.float32(1 / math.sqrt(D))), exact=False, causal=causal, rows=rows,
         label="8192")


@pytest.mark.parametrize("case", ["none", "causal", "rowdrop_causal"])
def test_integer_scores_document_mask(case):
    x = _integer_inputs(9, 2, 4, 2, 700, 700, 128)
    docs = inputs.packed_document_ids(9, 2, 700, 6)
    _run(x, 128, scale=LN2, exact=True, q_doc=docs, label="doc " + case, **EXACT_CASES[case])


def test_integer_scores_document_mask_with_window():
    x = _integer_inputs(12, 1, 4, 2, 700, 700, 128)
    docs = inputs.packed_document_ids(12, 1, 700, 5)
    _run(x, 128, scale=LN2, exact=True, q_doc=docs, causal=True, window=90, label="doc window")


def test_integer_scores_document_mask_with_block_mask():
    S = 700
    x = _integer_inputs(10, 1, 4, 4, S, S, 64)
    bm = inputs.random_block_mask(10, (1, 4, -(-S // 128), -(-S // 64)))
    docs = inputs.packed_document_ids(10, 1, S, 5)
    _run(x, 64, scale=LN2, exact=True, causal=True, block_mask=bm, q_doc=docs, label="doc block")


@pytest.mark.parametrize("D", [64, 128])
def test_random_document_mask_within_derived_bound(D):
    x = inputs.attention_inputs_fp8(11, 2, 4, 4, 1024, 1024, D)
    docs = inputs.packed_document_ids(11, 2, 1024, 7)
    _run(x, D, scale=float(np.float32(1 / math.sqrt(D))), exact=False, causal=True, alibi=True,
         q_doc=docs, label="doc")


@pytest.mark.parametrize("D", [64, 128])
def test_scores_far_above_the_first_tile(D):
    """Without a mod the kernel fixes each row's max at its first key tile. Here half the
    rows (alternating blocks of 8) see their lowest scores in that tile and scores up to
    8 units (23 in base 2 at this scale) higher later, so their P overflow e4m3 and the
    workgroup recomputes those waves with the lazy rescale; the other rows see their
    highest scores first and keep the first pass. Random V; the derived bound applies."""
    B, H, Sq, Skv = 1, 2, 512, 1024
    g = inputs.rng(41)
    sign = np.where((np.arange(Sq) // 8) % 2 == 0, 1.0, -1.0)
    q = np.zeros((B, H, Sq, D))
    q[..., :4] = sign[None, None, :, None]
    k = g.choice([-1.0, 0.0, 1.0], size=(B, H, Skv, D))
    k[..., :64, :4] = -1.0          # first tile: score -4 for rows of sign +1 (+4 for sign -1)
    k[..., 64:, 4:] = 0.0
    v = g.standard_normal((B, H, Skv, D)).astype(np.float32)
    dv = np.float32(float(np.abs(v).max()) / inputs.E4M3_MAX)
    x = {"q": inputs.f32_to_e4m3_bits(q), "k": inputs.f32_to_e4m3_bits(k),
         "v": inputs.f32_to_e4m3_bits(np.clip(v / dv, -448, 448)),
         "descale_q": 1.0, "descale_k": 1.0, "descale_v": float(dv)}
    _run(x, D, scale=2.0, exact=False, label="far-above")
