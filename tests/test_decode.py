"""GPU parity of the decode path (mm_attn_decode through the C ABI) against the oracle."""
import numpy as np
import pytest

import oracle
from helpers import LSE_ATOL, LSE_RTOL, O_ATOL, O_RTOL, assert_parity, to_f64, to_torch
from mask_mods_amd import inputs

pytestmark = pytest.mark.gpu

SCALE = 0.08837890625  # f16(1/sqrt(128)), the decode scale of the pages' example
LENGTHS = [1, 17, 1000, 4096, 32768]


def _run(B, Hq, Hkv, lens, D, dtype, *, Scap=None, kv_len=None, use_mask=True, use_lens=True,
         bias_seed=None, seed=0, num_splits=0, scale=SCALE, mask_override=None, nan_workspace=False):
    import torch
    import mask_mods_amd as mm
    lens = np.asarray(lens, dtype=np.int64)
    if kv_len is None:
        kv_len = int(lens.max())
    if Scap is None:
        Scap = kv_len
    print(f"[decode] B={B} Hq={Hq} Hkv={Hkv} lens={lens.tolist()[:8]} kv_len={kv_len} Scap={Scap} "
          f"D={D} {dtype} mask={use_mask} seq_lens={use_lens} bias={bias_seed} splits={num_splits}",
          flush=True)
    x = inputs.decode_inputs(seed, B, Hq, Hkv, lens, D, dtype, Scap=Scap, with_pad_mask=use_mask)
    q, k, v = (to_torch(x[n], dtype) for n in ("q", "k", "v"))
    mask_bits = None
    if use_mask:
        mask_bits = x["mask"]
        if bias_seed is not None:
            # finite N(0,1) bias on the valid positions, -inf kept on the pad
            bias = inputs.random_f16_bias(bias_seed, mask_bits.shape)
            mask_bits = np.where(mask_bits == inputs.F16_NEG_INF_BITS, mask_bits, bias)
        if mask_override is not None:
            mask_bits = mask_override(mask_bits)
    mask = to_torch(mask_bits, "f16") if mask_bits is not None else None
    seq = torch.tensor(x["lens"], dtype=torch.int32, device="cuda") if use_lens else None
    ws = None
    if nan_workspace:
        # every partial the kernels do not write stays NaN: reading one shows in O
        need = mm.decode_workspace_size(B, Hq, kv_len, D, num_splits=num_splits, Hkv=Hkv)
        ws = torch.full(((need + 3) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    out, lse = mm.attn_decode(q, k, v, kv_len, scale, mask=mask, seq_lens=seq, num_splits=num_splits,
                              workspace=ws)
    torch.cuda.synchronize()
    qd, kd, vd = (inputs.bits_to_f64(x[n], dtype) for n in ("q", "k", "v"))
    md = inputs.bits_to_f64(mask_bits, "f16") if mask_bits is not None else None
    O, L = oracle.attention(qd, kd, vd, scale=scale, Skv=kv_len, add_mask=md,
                            lens=x["lens"] if use_lens else None)
    assert_parity(to_f64(out), O, O_ATOL, O_RTOL, "O")
    assert_parity(to_f64(lse).reshape(B, Hq, 1), L, LSE_ATOL, LSE_RTOL, "LSE")
    return out, lse


@pytest.mark.parametrize("L", LENGTHS)
def test_config_decode_b1(L):
    _run(1, 32, 32, [L], 128, "f16", use_lens=False)


def test_config_decode_b1_capacity_larger_than_length():
    _run(1, 32, 32, [3000], 128, "f16", Scap=4096, use_lens=False)


def test_config_decode_b8_per_sequence_lengths():
    g = np.random.default_rng(1)
    lens = g.choice(LENGTHS, size=8)
    lens[0] = 32768
    _run(8, 32, 32, lens, 128, "f16", Scap=32768, seed=1)


@pytest.mark.parametrize("Hkv,use_mask", [(32, True), (32, False), (8, True), (4, False)])
def test_varlen_empty_splits_are_not_read(Hkv, use_mask):
    """With per-sequence lengths the split count is raised for the longest possible
    sequence, so most splits of the short ones are empty: they write only their (max,
    sum), and the merge must not read their output partials. The workspace starts as
    NaN, so any such read would show in O."""
    _run(8, 32, Hkv, [4096, 1, 0, 17, 1000, 300, 4096, 2], 128, "f16", Scap=4096, seed=21,
         use_mask=use_mask, nan_workspace=True)


@pytest.mark.parametrize("Hkv,D,dtype", [(32, 128, "f16"), (8, 128, "bf16"), (4, 64, "f16"), (16, 64, "bf16")])
def test_one_split_writes_the_output_itself(Hkv, D, dtype):
    """With one split the split pass normalises and writes O and LSE itself (no merge
    launch), for every head-group size; an empty sequence gives O = 0, LSE = -inf."""
    out, lse = _run(3, 32, Hkv, [300, 0, 1], D, dtype, Scap=300, seed=31, num_splits=1)
    assert np.all(to_f64(out)[1] == 0) and np.all(to_f64(lse)[1] == -np.inf)


def test_finite_bias_mask_added_after_scale():
    _run(2, 32, 32, [1500, 700], 128, "f16", bias_seed=5, seed=2)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64, 256])
def test_forced_splits(splits):
    _run(1, 32, 32, [5000], 128, "f16", num_splits=splits, use_lens=False, seed=3)


def test_split_count_does_not_change_result_beyond_rounding():
    import torch
    outs = []
    for s in (1, 5, 40):
        o, l = _run(2, 8, 8, [4000, 333], 128, "f16", num_splits=s, seed=4)
        outs.append((o.float(), l))
    for o, l in outs[1:]:
        assert torch.allclose(o, outs[0][0], atol=2e-3) and torch.allclose(l, outs[0][1], atol=1e-5)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_dtypes_and_head_dims(dtype, D):
    _run(2, 16, 16, [2100, 900], D, dtype, seed=5)


def test_gqa_decode():
    _run(2, 32, 8, [3000, 1234], 128, "f16", seed=6)


def test_no_mask_with_lens():
    _run(4, 32, 32, [1, 64, 4096, 0], 128, "f16", use_mask=False, seed=7)


def test_fully_masked_rows():
    def kill(m):
        m = m.copy()
        m[0, 3] = inputs.F16_NEG_INF_BITS  # every position of (b=0, h=3) masked
        return m
    out, lse = _run(2, 8, 8, [700, 0], 128, "f16", seed=8, mask_override=kill)
    o, l = to_f64(out), to_f64(lse)
    assert np.all(o[1] == 0) and np.all(l[1] == -np.inf)          # empty sequence
    assert np.all(o[0, 3] == 0) and l[0, 3] == -np.inf             # all -inf mask


def test_zero_length_cache():
    out, lse = _run(1, 4, 4, [0], 64, "f16", kv_len=0, Scap=8, use_mask=False, seed=9)
    assert np.all(to_f64(out) == 0) and np.all(to_f64(lse) == -np.inf)


def test_single_key_returns_v0():
    import torch
    import mask_mods_amd as mm
    x = inputs.decode_inputs(10, 2, 8, 8, [1, 1], 128, "f16", Scap=16, with_pad_mask=False)
    q, k, v = (to_torch(x[n], "f16") for n in ("q", "k", "v"))
    out, _ = mm.attn_decode(q, k, v, 1, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, 0], v[:, :, 0])


def test_deterministic():
    import torch
    import mask_mods_amd as mm
    x = inputs.decode_inputs(11, 1, 32, 32, [8000], 128, "f16")
    q, k, v = (to_torch(x[n], "f16") for n in ("q", "k", "v"))
    m = to_torch(x["mask"], "f16")
    o1, l1 = mm.attn_decode(q, k, v, 8000, SCALE, mask=m)
    o2, l2 = mm.attn_decode(q, k, v, 8000, SCALE, mask=m)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_workspace_reuse_across_calls_and_split_counts():
    """One workspace serves many calls with different split counts."""
    import torch
    import mask_mods_amd as mm
    x = inputs.decode_inputs(12, 2, 16, 16, [3000, 1200], 128, "f16")
    q, k, v = (to_torch(x[n], "f16") for n in ("q", "k", "v"))
    m = to_torch(x["mask"], "f16")
    seq = torch.tensor(x["lens"], dtype=torch.int32, device="cuda")
    ws = torch.empty(mm.decode_workspace_size(2, 16, 3000, 128, num_splits=64) // 4 + 4,
                     dtype=torch.float32, device="cuda")
    ref, lref = mm.attn_decode(q, k, v, 3000, SCALE, mask=m, seq_lens=seq)
    for splits in (64, 3, 17, 1, 64, 40):
        o, l = mm.attn_decode(q, k, v, 3000, SCALE, mask=m, seq_lens=seq, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert torch.allclose(o.float(), ref.float(), atol=2e-3) and torch.allclose(l, lref, atol=1e-5)


# ------------------------------------------------------------ GQA head groups
@pytest.mark.parametrize("Hq,Hkv", [(32, 16), (32, 8), (32, 4), (24, 8), (48, 8), (64, 4)])
def test_gqa_head_groups(Hq, Hkv):
    """Group sizes 2 and 4 (one workgroup per group), 8 and 16 (two and four workgroups
    of 4 heads per kv head), 3 (one head per workgroup) and 6 (three workgroups of 2)."""
    _run(2, Hq, Hkv, [2500, 777], 128, "f16", bias_seed=13, seed=13)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f16", 64), ("bf16", 128)])
def test_gqa_dtypes(dtype, D):
    _run(2, 16, 2, [1800, 4000], D, dtype, seed=14)


# ------------------------------------------------------------ paged KV
def _paged_run(B, Hq, Hkv, lens, D, dtype, page_size, *, seed=0, use_mask=True, num_splits=0):
    import torch
    import mask_mods_amd as mm
    lens = np.asarray(lens, dtype=np.int64)
    pages = -(-int(lens.max()) // page_size)
    Scap = pages * page_size
    print(f"[decode paged] B={B} Hq={Hq} Hkv={Hkv} lens={lens.tolist()} D={D} {dtype} page={page_size} "
          f"splits={num_splits}", flush=True)
    x = inputs.decode_inputs(seed, B, Hq, Hkv, lens, D, dtype, Scap=Scap, with_pad_mask=use_mask)
    # scatter each sequence's logical pages to random physical pages of one pool (with
    # a few unused pages between), and record the table
    g = np.random.default_rng(seed + 7)
    n_phys = B * pages + 5
    perm = g.permutation(n_phys)[:B * pages].reshape(B, pages).astype(np.int32)
    pool_k = np.zeros((n_phys, Hkv, page_size, D), dtype=x["k"].dtype)
    pool_v = np.zeros_like(pool_k)
    for b in range(B):
        for pg in range(pages):
            sl = slice(pg * page_size, (pg + 1) * page_size)
            pool_k[perm[b, pg]] = x["k"][b, :, sl, :]
            pool_v[perm[b, pg]] = x["v"][b, :, sl, :]
    q = to_torch(x["q"], dtype)
    kp, vp = to_torch(pool_k, dtype), to_torch(pool_v, dtype)
    bt = torch.from_numpy(perm).cuda()
    mask = to_torch(x["mask"], "f16") if use_mask else None
    seq = torch.tensor(x["lens"], dtype=torch.int32, device="cuda")
    out, lse = mm.attn_decode(q, kp, vp, int(lens.max()), SCALE, mask=mask, seq_lens=seq,
                              block_table=bt, num_splits=num_splits)
    torch.cuda.synchronize()
    qd, kd, vd = (inputs.bits_to_f64(x[n], dtype) for n in ("q", "k", "v"))
    md = inputs.bits_to_f64(x["mask"], "f16") if use_mask else None
    O, L = oracle.attention(qd, kd, vd, scale=SCALE, Skv=int(lens.max()), add_mask=md, lens=x["lens"])
    assert_parity(to_f64(out), O, O_ATOL, O_RTOL, "O")
    assert_parity(to_f64(lse).reshape(B, Hq, 1), L, LSE_ATOL, LSE_RTOL, "LSE")


# pages of 1 and 8 keys are smaller than the 16 keys a workgroup loads per step, so
# the lanes of one step read different pages (and their table entries) themselves
@pytest.mark.parametrize("page_size", [1, 8, 16, 64, 256])
def test_paged(page_size):
    _paged_run(3, 32, 32, [3000, 1, 1777], 128, "f16", page_size, seed=15)


def test_paged_gqa_no_mask_forced_splits():
    _paged_run(2, 32, 8, [4096, 333], 128, "bf16", 64, seed=16, use_mask=False, num_splits=7)


def test_paged_gqa_group_8():
    """Two workgroups of 4 query heads per kv head, each gathering the same pages."""
    _paged_run(2, 32, 4, [5000, 2049], 128, "f16", 16, seed=18)


def test_paged_long_and_empty():
    _paged_run(2, 16, 16, [32768, 0], 64, "f16", 128, seed=17)


def test_long_cache_262144_gqa():
    """A 262144-position cache (256 splits, the most the split count allows), GQA 4:1,
    with the pad mask and a capacity above the length."""
    _run(1, 8, 2, [262144 - 77], 128, "f16", Scap=262144, use_lens=False)
