"""Number formats used by the oracle: bfloat16 carried as uint16 bit patterns, fp32, fp64.

TEST INFRASTRUCTURE ONLY: this package is the CPU oracle the HIP path is checked against. Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it; the product path never does.

bfloat16 is the upper half of an IEEE-754 binary32 word (1 sign, 8 exponent, 7 stored fraction bits),
so widening is exact and narrowing rounds to 8 significant bits. Narrowing here is written from that
definition, in one step from float64, round-to-nearest with ties to even; it is not a bit trick on a
float32 word, so it shares nothing with how a GPU kernel rounds.
"""
from __future__ import annotations

import numpy as np

# Largest finite bfloat16: (2 - 2^-7) * 2^127.
BF16_MAX = float.fromhex("0x1.fep127")
# Exponent of the bfloat16 quantum below the smallest normal (2^-126 * 2^-7).
_BF16_SUBNORMAL_QUANTUM_EXP = -133


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):     # nan patterns widen to nan
        return b.view(np.float32).astype(np.float64)


def round_to_bf16(v) -> np.ndarray:
    """Round real values (float64) to the nearest bfloat16 value, ties to even; returned as float64.

    A normal number a in [2^(e-1), 2^e) keeps 8 significant bits, so its quantum is 2^(e-8); below the
    smallest normal the quantum is fixed at 2^-133. Results above the largest finite value overflow to
    infinity; inf and nan pass through.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                      # a = m * 2^e with m in [0.5, 1)
    q_exp = np.maximum(e - 8, _BF16_SUBNORMAL_QUANTUM_EXP)
    with np.errstate(over="ignore", invalid="ignore"):
        scaled = np.ldexp(a, -q_exp)        # exact: scaling by a power of two
        r = np.ldexp(np.rint(scaled), q_exp)  # np.rint rounds half to even
        r = np.where(r > BF16_MAX, np.inf, r)
    out = np.copysign(r, v)
    return np.where(np.isfinite(v), out, v)


def f64_to_bf16_bits(v) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even) and return the uint16 bit patterns."""
    r = round_to_bf16(v)
    # r is exactly representable in binary32, so this conversion is exact
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_to_f32(v) -> np.ndarray:
    """Round float64 values to the nearest binary32 (ties to even), as float32."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def to_f64(a, dt: str) -> np.ndarray:
    """Activation array in storage form -> float64. dt is "f32" (float32 array) or "bf16" (uint16 bits)."""
    if dt == "bf16":
        return bf16_bits_to_f64(a)
    if dt == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dt!r}")


def from_f64(v, dt: str) -> np.ndarray:
    """float64 -> storage form of dt, one rounding."""
    if dt == "bf16":
        return f64_to_bf16_bits(v)
    if dt == "f32":
        return round_to_f32(v)
    raise ValueError(f"unknown dtype {dt!r}")
