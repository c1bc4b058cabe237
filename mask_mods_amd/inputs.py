"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This module holds no attention arithmetic. It only draws random numbers and
encodes them as the 16/32-bit patterns that both sides consume, so that the
HIP kernels and the oracle read exactly the same input values:

* values ~ N(0, 1) in float32 from numpy's PCG64 (``default_rng(seed)``);
* bf16 bits by round-to-nearest-even of the float32 bit pattern; f16 bits by
  numpy's float32 -> float16 cast (also round-to-nearest-even);
* exact decoding of those bits to float64 for the oracle.

The workloads follow the pages' shapes: Q/K/V laid out [B, H, S, D] with D
innermost (IREE issue #19015, example IR), and a decode mask [B, H, 1, L] that
is 0 on valid positions and -inf on a random trailing pad.
"""
from __future__ import annotations

import numpy as np

DTYPES = ("f32", "f16", "bf16")

# f16 bit patterns of the two additive-mask values used by the decode workload
F16_ZERO_BITS = np.uint16(0x0000)
F16_NEG_INF_BITS = np.uint16(0xFC00)


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def f32_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Encode float32 values in ``dtype``: uint16 bits for f16/bf16, uint32 for f32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "f32":
        return x.view(np.uint32).copy()
    raise ValueError(f"unknown dtype {dtype!r}")


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode bit patterns exactly to float64 (every f16/bf16/f32 value is a float64)."""
    bits = np.ascontiguousarray(bits)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---- OCP e4m3 ("float8_e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
# no infinities, NaN = S.1111.111, max 448, smallest subnormal 2^-9.
def _e4m3_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for c in range(128):
        e, m = c >> 3, c & 7
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        t[c], t[c | 0x80] = v, -v
    t[0x7F] = t[0xFF] = np.nan
    return t


E4M3_VALUES = _e4m3_table()
E4M3_MAX = 448.0


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round to e4m3 (nearest, ties to even); |x| must not exceed 448. Returns uint8."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(~np.isfinite(a)) or np.any(a > E4M3_MAX):
        raise ValueError("e4m3 encoding needs finite values of magnitude <= 448")
    ex = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    quantum = 2.0 ** (np.maximum(ex, -6) - 3)   # spacing of e4m3 values around a
    y = np.rint(a / quantum) * quantum           # np.rint rounds half to even
    pos = E4M3_VALUES[:0x7F]                     # codes 0..126: increasing magnitudes
    code = np.searchsorted(pos, y).astype(np.uint8)
    assert np.all(pos[code] == y)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.ascontiguousarray(bits, dtype=np.uint8)]


def attention_inputs_fp8(seed: int, B: int, Hq: int, Hkv: int, Sq: int, Skv: int, D: int) -> dict:
    """N(0,1) Q, K, V (same draws as attention_inputs) quantised per tensor to e4m3:
    X8 = e4m3(X / s) with s = max|X| / 448 in float32; the real tensor is s * X8.
    Returns the uint8 bits and the three factors (float32)."""
    g = rng(seed)
    out = {"dtype": "fp8"}
    for name, shape in (("q", (B, Hq, Sq, D)), ("k", (B, Hkv, Skv, D)), ("v", (B, Hkv, Skv, D))):
        x = g.standard_normal(size=shape, dtype=np.float32)
        amax = float(np.max(np.abs(x))) if x.size else 1.0
        s = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
        out[name] = f32_to_e4m3_bits(np.minimum(np.abs(x / s), E4M3_MAX) * np.sign(x))
        out["descale_" + name] = float(s)
    return out


def normal_bits(g: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) float32 draws encoded in ``dtype``."""
    return f32_to_bits(g.standard_normal(size=shape, dtype=np.float32), dtype)


def attention_inputs(seed: int, B: int, Hq: int, Hkv: int, Sq: int, Skv: int, D: int,
                     dtype: str) -> dict:
    """Q [B,Hq,Sq,D], K and V [B,Hkv,Skv,D] as bit arrays, drawn in that order."""
    g = rng(seed)
    return {
        "q": normal_bits(g, (B, Hq, Sq, D), dtype),
        "k": normal_bits(g, (B, Hkv, Skv, D), dtype),
        "v": normal_bits(g, (B, Hkv, Skv, D), dtype),
        "dtype": dtype,
    }


def rising_score_inputs(seed: int, B: int, H: int, S: int, D: int, dtype: str,
                        rise: float = 3.0, wobble: float = 8.0, period: float = 700.0) -> dict:
    """Q, K, V [B,H,S,D] whose scores at scale 1/sqrt(D) climb along the keys.

    Per (b, h) one random unit vector u; q_i = sqrt(D) u + 0.5 n_i and
    k_j = c_j u + m_j with c_j = rise * j / 64 + wobble * sin(2 pi j / period) and n, m,
    V standard normal. The scaled score of (i, j) is then about c_j plus unit-size noise:
    it gains `rise` per 64 keys on average, with stretches where it falls.
    """
    g = rng(seed)
    u = g.standard_normal(size=(B, H, 1, D))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    j = np.arange(S, dtype=np.float64)
    c = (rise * j / 64.0 + wobble * np.sin(2.0 * np.pi * j / period)).reshape(1, 1, S, 1)
    q = np.sqrt(D) * u + 0.5 * g.standard_normal(size=(B, H, S, D))
    k = c * u + g.standard_normal(size=(B, H, S, D))
    v = g.standard_normal(size=(B, H, S, D))
    return {n: f32_to_bits(a.astype(np.float32), dtype) for n, a in (("q", q), ("k", k), ("v", v))} | {"dtype": dtype}


def pad_lengths(g: np.random.Generator, B: int, L: int) -> np.ndarray:
    """One trailing-pad length per sequence, uniform on {0, ..., L-1}."""
    return g.integers(0, L, size=B, dtype=np.int64)


def decode_inputs(seed: int, B: int, Hq: int, Hkv: int, lens, D: int, dtype: str,
                  Scap: int | None = None, with_pad_mask: bool = True) -> dict:
    """Decode workload: one query per head against a KV cache of capacity Scap.

    ``lens`` holds each sequence's KV length (all <= Scap). q is [B,Hq,1,D], the
    caches [B,Hkv,Scap,D]. When ``with_pad_mask``, an f16 additive mask
    [B,Hq,1,Scap] is 0 on the first len_b - pad_b positions and -inf after them,
    with pad_b ~ U{0..len_b-1} per sequence (the same for every head), so at least
    one position stays valid. Positions at or beyond len_b hold random data that a
    correct kernel never reads into the result.
    """
    lens = np.asarray(lens, dtype=np.int64).reshape(B)
    if Scap is None:
        Scap = int(lens.max())
    assert (lens >= 0).all() and (lens <= Scap).all()
    g = rng(seed)
    out = {
        "q": normal_bits(g, (B, Hq, 1, D), dtype),
        "k": normal_bits(g, (B, Hkv, Scap, D), dtype),
        "v": normal_bits(g, (B, Hkv, Scap, D), dtype),
        "lens": lens.astype(np.int32),
        "dtype": dtype,
        "Scap": Scap,
    }
    if with_pad_mask:
        pads = np.array([g.integers(0, max(int(n), 1)) for n in lens], dtype=np.int64)
        mask = np.full((B, Hq, 1, Scap), F16_NEG_INF_BITS, dtype=np.uint16)
        for b in range(B):
            mask[b, :, :, : int(lens[b] - pads[b])] = F16_ZERO_BITS
        out["mask"] = mask
        out["pads"] = pads
    return out


def random_f16_bias(seed: int, shape) -> np.ndarray:
    """Finite additive-mask bits: N(0,1) rounded to f16."""
    return f32_to_bits(rng(seed).standard_normal(size=shape, dtype=np.float32), "f16")


def sample_rows(seed: int, B: int, H: int, S: int, n_random: int = 64, block: int = 128) -> np.ndarray:
    """Flat row ids r = (b*H + h)*S + i for sampled parity at full size.

    Every (b, h) contributes its first and last row and one row drawn uniformly inside
    each block of ``block`` consecutive rows (0 = none): with the smallest query tile of
    the forward launches, every workgroup of a launch has a checked row. n_random more
    rows are drawn uniformly over all rows. Sorted and unique.
    """
    g = rng(seed)
    rows = []
    for bh in range(B * H):
        rows.append(bh * S)
        rows.append(bh * S + S - 1)
    rows.extend(g.integers(0, B * H * S, size=n_random).tolist())
    if block > 0 and S > 0:
        starts = np.arange(0, S, block, dtype=np.int64)
        span = np.minimum(starts + block, S) - starts
        for bh in range(B * H):
            rows.extend((bh * S + starts + (g.random(starts.size) * span).astype(np.int64)).tolist())
    return np.unique(np.asarray(rows, dtype=np.int64))


def random_block_mask(seed: int, shape, p_empty: float = 0.4, p_full: float = 0.3) -> np.ndarray:
    """uint8 block classes drawn i.i.d.: 0 with p_empty, 2 with p_full, else 1.

    A stand-in for a BlockMask built from an arbitrary mask_mod: any mix of empty,
    full and partial blocks, in any order along a row.
    """
    u = rng(seed).random(shape)
    return np.where(u < p_empty, 0, np.where(u < p_empty + p_full, 2, 1)).astype(np.uint8)


def packed_document_ids(seed: int, B: int, S: int, n_docs: int, first_id: int = 0) -> np.ndarray:
    """int32 [B, S] document ids of sequences packed back to back: per batch row,
    n_docs documents (at most S) whose lengths come from n_docs - 1 distinct cut points
    drawn uniformly, so the lengths are mixed (single-token documents included as the
    draw falls) and the ids run first_id, first_id + 1, ... without decreasing.
    """
    g = rng(seed)
    out = np.empty((B, S), dtype=np.int32)
    n = max(1, min(n_docs, S))
    for b in range(B):
        cuts = np.sort(g.choice(np.arange(1, S), size=n - 1, replace=False)) if n > 1 else np.array([], int)
        ids = np.zeros(S, dtype=np.int32)
        ids[cuts] = 1
        out[b] = first_id + np.cumsum(ids)
    return out


def document_ids_from_lengths(lengths, S: int | None = None) -> np.ndarray:
    """int32 [S] ids 0, 0, .., 1, .. for documents of the given lengths, in order."""
    ids = np.repeat(np.arange(len(lengths), dtype=np.int32), np.asarray(lengths, dtype=np.int64))
    assert S is None or ids.size == S
    return ids
