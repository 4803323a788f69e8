"""Pins for the oracle's bfloat16 widening and the generator's bfloat16 rounding."""

import numpy as np
import torch

from oracle.dtypes import bf16_bits_to_f64
from speculative_verify_isd_amd.workloads import f32_to_bf16_bits


def test_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0080, 0x7F80, 0xFF80, 0x0001, 0x0000, 0x8000, 0x4049],
                    dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -126, np.inf, -np.inf, 2.0 ** -133, 0.0, -0.0, 3.140625]
    got = bf16_bits_to_f64(bits)
    assert got.dtype == np.float64
    for g, w in zip(got, want):
        assert g == w


def test_bf16_matches_torch_widening():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=100000, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    bits = bits[finite]
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_bits_to_f64(bits), ref)


def test_generator_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-8, 8, 200000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)
