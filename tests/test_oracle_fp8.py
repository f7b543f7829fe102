"""Pins for the oracle's fp8 block-scaled token rows (oracle/fp8.py).

Each check ties the oracle to something other than its own formulas: values the OCP E4M3 format fixes,
torch's independent float8_e4m3fn type, brute-force minimisation for the block exponent, and the
error bound of round-to-nearest.
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp8
from oracle.moe import dispatch
from oracle.numerics import bf16_bits_to_f64


def test_format_constants():
    # largest finite, smallest normal, smallest subnormal, one, minus one, NaN codes, signed zeros
    d = fp8.e4m3_decode(np.array([0x7E, 0x08, 0x01, 0x38, 0xB8, 0x00, 0x80, 0x7F, 0xFF, 0x77, 0x3F]))
    assert d[0] == 448.0 and d[1] == 2.0 ** -6 and d[2] == 2.0 ** -9
    assert d[3] == 1.0 and d[4] == -1.0
    assert d[5] == 0.0 and not math.copysign(1, d[5]) < 0
    assert d[6] == 0.0 and math.copysign(1, d[6]) < 0
    assert np.isnan(d[7]) and np.isnan(d[8])
    assert d[9] == 240.0          # 0 1110 111: 2^7 * 1.875
    assert d[10] == 1.875         # 0 0111 111


def test_decode_agrees_with_torch_on_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_encode_agrees_with_torch_in_range_including_ties():
    fin = fp8.e4m3_decode(np.arange(256))
    fin = fin[~np.isnan(fin)]
    pos = np.sort(np.unique(np.abs(fin)))
    mids = (pos[1:] + pos[:-1]) / 2          # every tie between neighbouring magnitudes
    rng = np.random.default_rng(0)
    v = np.concatenate([fin, mids, -mids, rng.uniform(-448, 448, 20000), rng.uniform(-0.05, 0.05, 20000),
                        np.ldexp(rng.uniform(-1, 1, 5000), -8), [-0.0, 0.0, -1e-6, 1e-6]])
    ref = torch.tensor(v, dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(v), ref)


def test_encode_ties_go_to_even_mantissa_and_saturate():
    # 1.0625 lies halfway between 1.0 (m=0) and 1.125 (m=1): even -> 1.0; 1.1875 between 1.125 and 1.25 -> 1.25
    assert fp8.e4m3_encode([1.0625, 1.1875]).tolist() == [0x38, 0x3A]
    # halfway between the two smallest subnormals 2^-9 and 2^-8 -> 2^-8 (m=2 even); half of 2^-9 -> 0
    assert fp8.e4m3_encode([1.5 * 2.0 ** -9, 0.5 * 2.0 ** -9, -0.5 * 2.0 ** -9]).tolist() == [0x02, 0x00, 0x80]
    # beyond the largest finite value: clamped (torch's cast gives NaN there, so this reading is pinned alone)
    assert fp8.e4m3_encode([448.0, 449.0, 464.0, 1e6, -1e30]).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_block_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(1)
    amax = np.concatenate([[448.0, 449.0, 224.0, 224.5, 896.0, 1.0, 2.0 ** -20, 3e5, 7.0 * 2.0 ** 60],
                           np.abs(rng.standard_normal(200)) * 10.0 ** rng.integers(-6, 6, 200)])
    got = fp8.block_scale_exp(amax)
    for a, e in zip(amax, got):
        brute = next(j for j in range(-200, 200) if a / 2.0 ** j <= 448.0)  # smallest integer that fits
        assert e == brute, (a, e, brute)
    assert fp8.block_scale_exp([0.0]).tolist() == [0]


def _bf16_rows(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * scale
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_quantize_rows_error_bound_and_block_maximum():
    x = _bf16_rows((6, 512), 2)
    x[1, 128:256] = 0                                   # an all-zero block
    xv = bf16_bits_to_f64(x)
    codes, scales = fp8.quantize_rows(x)
    assert codes.dtype == np.uint8 and scales.dtype == np.float32 and scales.shape == (6, 4)
    assert scales[1, 1] == 1.0 and np.all(codes[1, 128:256] == 0)
    deq = fp8.dequantize_rows(codes, scales)
    for r in range(6):
        for b in range(4):
            blk = xv[r, b * 128:(b + 1) * 128]
            s = float(scales[r, b])
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            assert 224.0 < amax / s <= 448.0             # the scale puts the block maximum in the top binade
            y = blk / s
            # round-to-nearest error: at most half a quantum (2^(floor(log2|y|) - 4), or 2^-10 below 2^-6)
            half_q = np.where(np.abs(y) >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(y), 1e-300))).astype(int) - 4), 2.0 ** -10)
            assert np.all(np.abs(deq[r, b * 128:(b + 1) * 128] / s - y) <= half_q)


def test_dequantized_rows_are_exact_bf16_values():
    x = _bf16_rows((4, 256), 3, scale=50.0)
    codes, scales = fp8.quantize_rows(x)
    deq = fp8.dequantize_rows(codes, scales)
    assert np.array_equal(bf16_bits_to_f64(fp8.dequantize_rows_bf16(codes, scales)), deq)


def test_quantize_rejects_ragged_blocks():
    with pytest.raises(ValueError):
        fp8.quantize_rows(_bf16_rows((2, 200), 4))


def test_dispatch_fp8_is_dispatch_then_quantize():
    x = _bf16_rows((9, 256), 5)
    ids = np.array([[0, 1], [1, 2], [0, 2], [2, 3], [1, 0], [3, 2], [0, 3], [1, 3], [2, 0]], dtype=np.int32)
    lay, send = dispatch(x, "bf16", ids, 4, 3, 2)
    lay8, codes, scales = fp8.dispatch_fp8(x, ids, 4, 3, 2)
    for nm in ("expert_count", "expert_kept", "expert_overflow", "expert_offset", "row_token", "row_slot",
               "pair_row"):
        assert np.array_equal(getattr(lay, nm), getattr(lay8, nm)), nm
    # every send row is its token's row, quantised on its own
    for i, t in enumerate(lay.row_token):
        c1, s1 = fp8.quantize_rows(x[t:t + 1])
        assert np.array_equal(codes[i], c1[0]) and np.array_equal(scales[i], s1[0])


def test_layer_fp8_equals_bf16_layer_when_rows_are_exact_fp8():
    # rows built from E4M3 values times a power of two per block, each block holding 448 * 2^j: the
    # quantisation is then lossless, so the fp8 layer must give the bf16 layer's output bit for bit
    from oracle.moe import moe_layer
    from oracle.numerics import f64_to_bf16_bits
    rng = np.random.default_rng(7)
    T, H, E, k, F, R, C = 40, 256, 8, 2, 32, 2, 9
    codes = rng.integers(0, 0x7E, size=(T, H))
    codes |= rng.integers(0, 2, size=(T, H)) << 7
    codes[:, ::128] = 0x7E
    j = rng.integers(-12, -4, size=(T, H // 128))
    v = fp8.e4m3_decode(codes).reshape(T, H // 128, 128) * np.ldexp(1.0, j)[:, :, None]
    x = f64_to_bf16_bits(v.reshape(T, H))
    assert np.array_equal(fp8.dequantize_rows(*fp8.quantize_rows(x)), bf16_bits_to_f64(x))
    wr = rng.standard_normal((E, H)).astype(np.float32) * 0.02
    wgu = f64_to_bf16_bits(rng.standard_normal((E // R, 2 * F, H)) * 0.05)
    wdn = f64_to_bf16_bits(rng.standard_normal((E // R, H, F)) * 0.05)
    ref = moe_layer(x, "bf16", wr, None, k, C, R, wgu, wdn, F)
    got = fp8.moe_layer_fp8(x, wr, None, k, C, R, wgu, wdn, F)
    assert ref["layout"].total < T * k                      # some pairs dropped by capacity
    assert np.array_equal(got["y"], ref["y"]) and np.array_equal(got["out_buf"], ref["out_buf"])
    # and with inexact rows the two differ, by no more than the fp8 rounding allows
    x2 = _bf16_rows((T, H), 8)
    a = bf16_bits_to_f64(moe_layer(x2, "bf16", wr, None, k, C, R, wgu, wdn, F)["y"])
    b = bf16_bits_to_f64(fp8.moe_layer_fp8(x2, wr, None, k, C, R, wgu, wdn, F)["y"])
    live = np.linalg.norm(a, axis=1) > 0
    rel = np.linalg.norm(a - b, axis=1)[live] / np.linalg.norm(a, axis=1)[live]
    assert 0 < rel.max() <= 0.1
