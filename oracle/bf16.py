"""Exact bfloat16 helpers (numpy; no bf16 dtype needed).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

bfloat16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits,
7 stored mantissa bits.  The pages ("KDA Chunk Prefill on Ascend A3",
section "Mathematical definition") round the normalised Q/K to bfloat16 and
emit the output o in bfloat16; the decode page
("flashinfer.kda_decode.packed_kda_decode", section "Parameters") keeps the
recurrent state pool in bfloat16.  The rounding used everywhere is IEEE
round-to-nearest, ties-to-even.
"""

import numpy as np


def bf16_bits(x):
    """float32 array -> uint16 bit patterns, rounded to nearest, ties to even.

    NaN inputs map to a quiet NaN; infinities are preserved.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(x)
    rounded = np.where(nan, (u.astype(np.uint32) >> 16) | 0x40, rounded)
    return rounded.astype(np.uint16)


def bits_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_round(x):
    """Round a float32 array to the nearest bf16 value; returns float32."""
    return bits_to_f32(bf16_bits(x))


def f64_to_bf16_round(x):
    """Round a float64 array straight to the nearest bf16 (one rounding).

    Rounding through float32 first could round twice; this rounds the
    float64 significand directly to 8 bits with ties-to-even.  Values whose
    bf16 result would be subnormal (|x| < 2**-126) are rounded through
    float32, where the two roundings cannot disagree for the magnitudes the
    tests use (documented limitation).  Returns float32.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    u = x.view(np.uint64)
    drop = np.uint64(45)  # 52 stored bits -> 7 stored bits
    lsb = (u >> drop) & np.uint64(1)
    inc = (np.uint64(1) << (drop - np.uint64(1))) - np.uint64(1) + lsb
    r = (u + inc) & ~((np.uint64(1) << drop) - np.uint64(1))
    out = r.view(np.float64).astype(np.float32)
    small = np.abs(x) < 2.0 ** -126
    if np.any(small):
        out = np.where(small, bf16_round(x.astype(np.float32)), out)
    bad = ~np.isfinite(x)
    if np.any(bad):
        out = np.where(bad, x.astype(np.float32), out)
    return out
