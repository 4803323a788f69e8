"""Pins of oracle.lora."""

import numpy as np

from oracle.dtypes import bf16_bits_to_f64
from oracle.lora import f64_to_bf16_rne, gated_lora


def _nearest_bf16(v):
    """Exhaustive nearest bfloat16 (ties to the even pattern) of finite v."""
    pats = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    pats = pats[((pats >> 7) & 0xFF) != 0xFF]  # finite patterns (exponent not all ones)
    vals = bf16_bits_to_f64(pats)
    d = np.abs(vals - v)
    best = d.min()
    cands = pats[d == best]
    # ties: the even significand; +0 over -0 only matters for v == 0
    if v == 0:
        return np.uint16(0x8000 if np.signbit(v) else 0)
    even = [c for c in cands if (int(c) & 1) == 0]
    return np.uint16(even[0] if even else cands[0])


def test_rounding_matches_exhaustive_search():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.normal(0, 1, 300), rng.normal(0, 1e3, 100), rng.normal(0, 1e-3, 100),
        # exact ties: bf16 value plus half an ulp
        bf16_bits_to_f64(rng.integers(0x3F00, 0x4100, 100).astype(np.uint16)) * (1 + 2.0 ** -9),
        np.array([1.0, -2.0, 0.0, 1.00390625, 1.01171875, 3.0e38, 1.2e-38]),
    ])
    got = f64_to_bf16_rne(vals)
    for v, g in zip(vals, got):
        assert g == _nearest_bf16(v), (v, hex(int(g)), hex(int(_nearest_bf16(v))))


def _case(rng, B, N, H, O, r):
    M = B * (2 * N - 1)
    x = rng.integers(0x3E00, 0x3F80, size=(M, H)).astype(np.uint16) ^ np.uint16(0)
    a = (rng.normal(0, 0.05, size=(r, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    b = (rng.normal(0, 0.05, size=(O, r)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = rng.normal(0, 1, size=(M, O)).astype(np.float32)
    return y, x, a, b


def test_verify_rows_are_the_base_output():
    rng = np.random.default_rng(2)
    y, x, a, b = _case(rng, 3, 4, 64, 48, 16)
    out = gated_lora(y, x, a, b, 0.5, 4)
    base = f64_to_bf16_rne(y.astype(np.float64))
    verify = (np.arange(y.shape[0]) % 7) < 4
    assert np.array_equal(out[verify], base[verify])
    # the adapter changes MASK rows
    assert not np.array_equal(out[~verify], base[~verify])
    # a zero scale gives the base output everywhere
    assert np.array_equal(gated_lora(y, x, a, b, 0.0, 4), base)


def test_rank_one_closed_form():
    # A = e_0 (picks x[:, 0]), B = column vector c: delta[m][o] = x[m][0] * c[o]
    rng = np.random.default_rng(3)
    y, x, _, _ = _case(rng, 2, 2, 32, 16, 1)
    a = np.zeros((1, 32), dtype=np.uint16)
    a[0, 0] = 0x3F80  # 1.0
    c = rng.normal(0, 1, 16).astype(np.float32)
    b = (c.view(np.uint32) >> 16).astype(np.uint16)[:, None]
    out = gated_lora(y, x, a, b, 2.0, 2)
    xm = bf16_bits_to_f64(x[:, 0])
    want = y.astype(np.float64) + 2.0 * np.outer(xm, bf16_bits_to_f64(b[:, 0]))
    mask = (np.arange(y.shape[0]) % 3) >= 2
    assert np.array_equal(out[mask], f64_to_bf16_rne(want[mask]))
