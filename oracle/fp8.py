"""fp8 block-scaled token rows for dispatch: OCP FP8 E4M3 codes with one power-of-two scale per block.

TEST INFRASTRUCTURE ONLY: this package is the CPU oracle the HIP path is checked against. Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it; the product path never does.

The pages ship tokens and their block scale factors in dispatch, with fp8 block scaling for dispatch
and bf16 for combine ("Efficient and portable mixture-of-experts communication", section "Dispatch";
"Enabling trillion-parameter models on AWS EFA", section "Оценка"). They fix neither the fp8 format,
the block size nor the scale format; the readings taken here:

* Format: OCP 8-bit floating point, E4M3 -- 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; a
  field e in 1..15 is normal, (-1)^s * 2^(e-7) * (1 + m/8), except e = 15, m = 7, which is NaN; e = 0 is
  subnormal, (-1)^s * 2^-6 * m/8. No infinities. Largest finite 448, smallest normal 2^-6, smallest
  subnormal 2^-9.
* Blocks: 128 consecutive hidden elements of one token row (H a multiple of 128).
* Scale: a power of two 2^E per block, E the smallest integer with max|x| / 2^E <= 448, so dividing by
  the scale is exact; an all-zero block takes E = 0.
* Codes: x / 2^E rounded to the nearest E4M3 value, ties to the even mantissa, clamped to +-448; a value
  that rounds to zero keeps its sign (code 0x80 for -0).
* The consumer (the expert MLP) uses code value * 2^E, which is exactly a bfloat16 value.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_bits_to_f64, f64_to_bf16_bits

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6       # smallest normal 2^-6
E4M3_SUBNORMAL_QUANTUM_EXP = -9  # subnormal quantum 2^-6 * 2^-3
BLOCK = 128


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values, from the field definition; NaN codes give nan."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), E4M3_SUBNORMAL_QUANTUM_EXP),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(v) -> np.ndarray:
    """Real values (float64, finite) -> E4M3 codes (uint8): nearest value, ties to the even mantissa,
    magnitudes above 448 clamped to 448, sign kept for values that round to zero."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, fe = np.frexp(a)                     # a = f * 2^fe, f in [0.5, 1)
    # quantum: 2^(exponent - 3) in the normal range, 2^-9 below 2^-6
    q_exp = np.maximum(fe - 1 - 3, E4M3_SUBNORMAL_QUANTUM_EXP)
    n = np.rint(np.ldexp(a, -q_exp))        # integer count of quanta, half to even
    r = np.ldexp(n, q_exp)                  # the rounded magnitude (may carry into the next binade)
    r = np.minimum(r, E4M3_MAX)
    # back to fields
    _, re = np.frexp(r)
    e_unb = re - 1                          # r in [2^e_unb, 2^(e_unb+1))
    normal = (r > 0) & (e_unb >= E4M3_MIN_NORMAL_EXP)
    e_field = np.where(normal, e_unb + 7, 0)
    m_field = np.where(normal, np.rint(np.ldexp(r, -e_unb) * 8.0 - 8.0),
                       np.rint(np.ldexp(r, -E4M3_SUBNORMAL_QUANTUM_EXP)))
    sign = (np.signbit(v)).astype(np.int64)
    code = (sign << 7) | (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    return code.astype(np.uint8)


def block_scale_exp(amax) -> np.ndarray:
    """Exponent E of the block scale 2^E: the smallest integer with amax / 2^E <= 448 (E = 0 for amax = 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        # amax / 448 = f * 2^fe, f in [0.5, 1): 2^E >= amax / 448 > 2^(E-1) gives E = fe, or fe - 1 when
        # amax / 448 is itself a power of two (f == 0.5)
        f, fe = np.frexp(amax / E4M3_MAX)
    e = np.where(f == 0.5, fe - 1, fe)
    return np.where(amax > 0, e, 0).astype(np.int64)


def quantize_rows(x_bits) -> tuple[np.ndarray, np.ndarray]:
    """bf16 rows [n, H] (uint16 bits) -> (codes [n, H] uint8, scales [n, H/128] float32 = 2^E)."""
    x = bf16_bits_to_f64(x_bits)
    n, H = x.shape
    if H % BLOCK != 0:
        raise ValueError(f"H = {H} is not a multiple of the {BLOCK}-element block")
    xb = x.reshape(n, H // BLOCK, BLOCK)
    E = block_scale_exp(np.abs(xb).max(axis=2))
    scaled = np.ldexp(xb, -E[:, :, None])   # exact: scaling by a power of two
    codes = e4m3_encode(scaled).reshape(n, H)
    scales = np.ldexp(1.0, E).astype(np.float32)
    return codes, scales


def dequantize_rows(codes, scales) -> np.ndarray:
    """(codes [n, H], scales [n, H/128]) -> float64 values code * scale (exact)."""
    codes = np.asarray(codes)
    n, H = codes.shape
    v = e4m3_decode(codes).reshape(n, H // BLOCK, BLOCK) * np.asarray(scales, dtype=np.float64)[:, :, None]
    return v.reshape(n, H)


def dequantize_rows_bf16(codes, scales) -> np.ndarray:
    """The bf16 activation rows the expert MLP consumes (uint16 bits); code * 2^E is exactly a bf16 value."""
    return f64_to_bf16_bits(dequantize_rows(codes, scales))


def dispatch_fp8(x_bits, ids, E: int, C: int, R: int = 1):
    """Dispatch with fp8 block-scaled rows: the layout of moe.dispatch, and the send buffer as codes and
    scales of the kept rows (send row i holds token row_token[i] quantised)."""
    from .moe import dispatch
    layout, send = dispatch(x_bits, "bf16", ids, E, C, R)
    codes, scales = quantize_rows(send.reshape(len(send), -1)) if len(send) else (
        np.zeros((0, np.asarray(x_bits).shape[1]), np.uint8), np.zeros((0, np.asarray(x_bits).shape[1] // BLOCK), np.float32))
    return layout, codes, scales


def moe_layer_fp8(x_bits, w_router, bias, k: int, C: int, R: int, w_gate_up, w_down, F: int, ids=None) -> dict:
    """The layer with fp8 block-scaled dispatch and bf16 combine ("Enabling trillion-parameter models on
    AWS EFA", section "Оценка"): route as moe.moe_layer, dispatch the rows as codes and scales, run the
    expert MLP on the values the codes stand for, combine in bf16. bf16 activations only."""
    from .moe import combine, expert_mlp, router_logits, routing_weights, row_experts, topk_select
    logits = router_logits(x_bits, "bf16", w_router, bias)
    if ids is None:
        ids = topk_select(logits, k)
    ids = np.asarray(ids, dtype=np.int32)
    w = routing_weights(logits, ids)
    E = np.asarray(w_router).shape[0]
    layout, codes, scales = dispatch_fp8(x_bits, ids, E, C, R)
    rows = dequantize_rows_bf16(codes, scales)
    out_buf = expert_mlp(rows, "bf16", row_experts(layout.expert_offset, E), E // R, w_gate_up, w_down, F)
    y = combine(out_buf, "bf16", layout.pair_row, w)
    return dict(logits=logits, ids=ids, weights=w, layout=layout, send_q=codes, send_scale=scales,
                out_buf=out_buf, y=y)
