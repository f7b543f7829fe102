"""Pins for the oracle's number formats (bfloat16 rounding written from its definition).

Pinned against: hand-derived bit patterns at ties, overflow and subnormals, and torch's float32 ->
bfloat16 conversion (an independent library implementation of round-to-nearest-even).
"""
import numpy as np
import pytest
import torch

from oracle.numerics import (BF16_MAX, bf16_bits_to_f64, f64_to_bf16_bits, round_to_bf16,
                             round_to_f32)


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (-2.0, 0xC000),
    (1.0 + 2.0 ** -8, 0x3F80),            # exact tie between 0x3F80 and 0x3F81 -> even
    (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie between 0x3F81 and 0x3F82 -> even
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),  # just above the tie
    (1.0 + 2.0 ** -8 - 2.0 ** -30, 0x3F80),  # just below the tie
    (BF16_MAX, 0x7F7F),
    (float.fromhex("0x1.ffp127"), 0x7F80),   # max + half an ulp: tie rounds to even -> inf
    (2.0 ** -133, 0x0001),                   # smallest subnormal
    (2.0 ** -134, 0x0000),                   # half of it: tie to even -> 0
    (1.5 * 2.0 ** -134, 0x0001),
    (2.0 ** -126, 0x0080),                   # smallest normal
    (0.0, 0x0000),
    (-0.0, 0x8000),
])
def test_bf16_rounding_hand_values(value, bits):
    assert int(f64_to_bf16_bits(np.array([value]))[0]) == bits


def test_bf16_widening_is_exact_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(bits)
    finite = np.isfinite(v)
    # every finite pattern survives a round trip (signed zeros included)
    assert np.array_equal(f64_to_bf16_bits(v[finite]), bits[finite])
    # and widening agrees with torch
    tv = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(v[finite], tv[finite])


def test_bf16_rounding_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
    ])
    ours = f64_to_bf16_bits(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_round_to_bf16_keeps_eight_significant_bits():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(10_000)
    r = round_to_bf16(v)
    m, _ = np.frexp(r)
    assert np.all(np.abs(m * 256 - np.rint(m * 256)) == 0)
    # the nearest bf16: error at most half a quantum
    _, e = np.frexp(np.abs(v))
    assert np.all(np.abs(r - v) <= np.ldexp(0.5, e - 8))


def test_round_to_f32_is_nearest():
    v = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 1.0 + 2.0 ** -24 + 2.0 ** -40])
    r = round_to_f32(v)
    assert r[0] == np.float32(1.0)
    assert r[1] == np.float32(1.0 + 2.0 ** -22)
    assert r[2] == np.float32(1.0 + 2.0 ** -23)
