"""Pins for the oracle's bf16 codec (CPU)."""

import numpy as np
import torch

from oracle import bf16


def test_roundtrip_all_bit_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16.to_f64(b)
    keep = ~np.isnan(x)
    assert np.array_equal(bf16.from_f64(x[keep]), b[keep])


def test_ties_round_to_even():
    # 1 + 2^-8 lies halfway between 1 (mantissa ...0) and 1 + 2^-7 (...1): even is 1.
    assert bf16.from_f64(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    assert bf16.from_f64(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
    # just above the tie rounds up
    assert bf16.from_f64(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 0x3F81
    # negative values mirror
    assert bf16.from_f64(np.array([-(1.0 + 2.0 ** -8)]))[0] == 0xBF80
    # overflow past the largest finite value becomes inf
    assert bf16.from_f64(np.array([3.5e38]))[0] == 0x7F80


def test_matches_torch_cast_of_float32():
    # torch's float32 -> bfloat16 cast is round-to-nearest-even; for inputs that
    # are exactly float32 the direct fp64 rounding must agree with it.
    g = torch.Generator().manual_seed(1)
    x = torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 8)
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16.from_f64(x.numpy().astype(np.float64))
    assert np.array_equal(got, ref)


def test_subnormals_and_ulp():
    tiny = np.array([2.0 ** -133, 3 * 2.0 ** -134, 2.0 ** -127])
    back = bf16.to_f64(bf16.from_f64(tiny))
    assert back[0] == 2.0 ** -133
    assert back[1] == 2.0 ** -132           # tie 1.5 quanta -> 2 quanta (even)
    assert back[2] == 2.0 ** -127
    assert bf16.ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert bf16.ulp(np.array([0.75]))[0] == 2.0 ** -8
    assert bf16.ulp(np.array([-3.0]))[0] == 2.0 ** -6
