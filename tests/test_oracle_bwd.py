"""Pins for the oracle's backward (CPU only).

The backward is pinned to the forward, itself pinned in test_oracle.py: central finite
differences of L = sum(dO * O(q, k, v)) through ``oracle.attention`` must match every
element of dq, dk, dv; plus invariants of the softmax Jacobian and special cases.
"""
import numpy as np
import pytest

import oracle


def _inputs(B, Hq, Hkv, Sq, Skv, D, seed):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, Hq, Sq, D))
    k = g.standard_normal((B, Hkv, Skv, D))
    v = g.standard_normal((B, Hkv, Skv, D))
    do = g.standard_normal((B, Hq, Sq, D))
    return q, k, v, do


def _loss(q, k, v, do, kw):
    O, _ = oracle.attention(q, k, v, **kw)
    return float(np.sum(do * O))


def _finite_diff(x, f, eps=1e-5):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        x0 = x[idx]
        x[idx] = x0 + eps
        fp = f()
        x[idx] = x0 - eps
        fm = f()
        x[idx] = x0
        g[idx] = (fp - fm) / (2 * eps)
    return g


CASES = {
    "none": dict(),
    "causal": dict(causal=True),
    "window": dict(window=2),
    "causal_window": dict(causal=True, window=3),
    "alibi": dict(alibi=True),
    "alibi_causal": dict(alibi=True, causal=True),
    "rowdrop": dict(rowdrop=(7, int(0.4 * 2 ** 32))),
}


def test_document_mask_matches_finite_differences():
    B, Hq, Hkv, S, D = 1, 2, 1, 9, 3
    q, k, v, do = _inputs(B, Hq, Hkv, S, S, D, seed=9)
    docs = np.array([[0, 0, 0, 1, 1, 2, 2, 2, 2]], dtype=np.int32)
    kw = dict(scale=0.45, causal=True, q_doc=docs)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, **kw)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = _finite_diff(x, lambda: _loss(q, k, v, do, kw))
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("shape", [(1, 2, 2, 6, 6, 4), (1, 4, 2, 5, 7, 3), (2, 2, 1, 7, 4, 4)])
def test_matches_finite_differences(case, shape):
    B, Hq, Hkv, Sq, Skv, D = shape
    q, k, v, do = _inputs(B, Hq, Hkv, Sq, Skv, D, seed=sum(shape))
    kw = dict(scale=0.45, **CASES[case])
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, **kw)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = _finite_diff(x, lambda: _loss(q, k, v, do, kw))
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7)


def test_block_mask_matches_finite_differences():
    """200 x 130 keys: two query blocks, three key blocks, every class present."""
    B, Hq, Hkv, Sq, Skv, D = 1, 2, 1, 200, 130, 2
    q, k, v, do = _inputs(B, Hq, Hkv, Sq, Skv, D, seed=3)
    bm = np.array([[[[2, 0, 1], [1, 2, 0]], [[0, 1, 2], [2, 2, 1]]]], dtype=np.uint8)
    kw = dict(scale=0.3, causal=True, block_mask=bm)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, **kw)
    # finite differences on a sample of elements (all of them would take minutes)
    g = np.random.default_rng(0)
    for x, gr in ((q, dq), (k, dk), (v, dv)):
        for _ in range(25):
            idx = tuple(int(g.integers(0, n)) for n in x.shape)
            x0 = x[idx]
            x[idx] = x0 + 1e-5
            fp = _loss(q, k, v, do, kw)
            x[idx] = x0 - 1e-5
            fm = _loss(q, k, v, do, kw)
            x[idx] = x0
            assert abs(gr[idx] - (fp - fm) / 2e-5) <= 1e-6 * (1 + abs(gr[idx])), idx


def test_key_gradients_sum_to_zero():
    """Each softmax row's dS sums to zero, so sum_j dK_j = 0 (and with GQA too)."""
    q, k, v, do = _inputs(2, 4, 2, 9, 11, 5, seed=4)
    for kw in (dict(), dict(causal=True), dict(alibi=True, window=3)):
        _, dk, _ = oracle.attention_bwd(q, k, v, do, scale=0.7, **kw)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)


def test_zero_upstream_gradient():
    q, k, v, do = _inputs(1, 2, 2, 5, 5, 3, seed=5)
    for g in oracle.attention_bwd(q, k, v, np.zeros_like(do), scale=0.5, causal=True):
        assert np.all(g == 0)


def test_equal_value_rows():
    """All V rows equal: O does not depend on q or k, so dq = dk = 0 and dv_j = sum_i P_ij dO_i."""
    q, k, v, do = _inputs(1, 2, 2, 6, 8, 4, seed=6)
    v[:] = v[:, :, :1, :]
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale=0.5)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    # with Q = 0 every weight is 1/Skv, so dv_j = sum_i dO_i / Skv
    dq, dk, dv = oracle.attention_bwd(np.zeros_like(q), k, v, do, scale=0.5)
    np.testing.assert_allclose(dv, np.broadcast_to(do.sum(axis=2, keepdims=True) / 8, dv.shape), atol=1e-12)


def test_fully_masked_rows_have_zero_gradient():
    """Cross attention with a window: query rows past Skv + w see no key."""
    q, k, v, do = _inputs(1, 2, 2, 12, 4, 3, seed=7)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale=0.5, causal=True, window=2)
    assert np.all(dq[:, :, 6:] == 0)
    # and those rows do not feed dk / dv: changing their dO changes nothing
    do2 = do.copy()
    do2[:, :, 6:] = 123.0
    _, dk2, dv2 = oracle.attention_bwd(q, k, v, do2, scale=0.5, causal=True, window=2)
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)


def test_gqa_sums_the_group():
    """GQA gradient of a kv head = sum over its query heads of the expanded (MHA) gradients."""
    q, k, v, do = _inputs(1, 4, 2, 6, 7, 3, seed=8)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale=0.6, causal=True)
    ke, ve = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    dqe, dke, dve = oracle.attention_bwd(q, ke, ve, do, scale=0.6, causal=True)
    np.testing.assert_allclose(dq, dqe, atol=1e-12)
    np.testing.assert_allclose(dk, dke.reshape(1, 2, 2, 7, 3).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dv, dve.reshape(1, 2, 2, 7, 3).sum(axis=2), atol=1e-12)
