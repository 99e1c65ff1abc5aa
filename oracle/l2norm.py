"""Canonical bit-exact Q/K L2 normalisation.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "KDA Chunk Prefill on Ascend A3", section "Mathematical definition":
each row of q and of k (last dimension, length K) is widened to float32,
divided by the square root of (the float32 sum of its squares plus an
epsilon of 1e-6 -- the epsilon sits inside the square root), and the
quotient is rounded to bfloat16.  The decode page
("flashinfer.kda_decode.packed_kda_decode") fixes the same epsilon.

The page writes the sum as a float32 tensor reduction without fixing its
order.  Reading taken here (order-free, and therefore reproducible by any
reduction tree): the sum is the exact sum of the float32 squares, rounded
once to float32 (round-to-nearest-even).  Everything else follows the page
in float32 with IEEE correctly rounded operations:

    sq  = fp32(x * x)                       (exact when x is a bf16 value)
    s   = fp32_rn( exact sum_d sq_d )
    t   = fp32_rn( s + fp32(1e-6) )
    den = fp32_rn( sqrt(t) )
    y   = bf16_rn( fp32_rn(x / den) )
"""

from fractions import Fraction

import numpy as np

from .bf16 import bf16_bits, bits_to_f32

EPS32 = np.float32(1e-6)


def _fraction_to_f32(fr):
    """Correctly rounded (ties-to-even) float32 of an exact rational."""
    if fr == 0:
        return np.float32(0.0)
    c = np.float32(float(fr))
    cands = [c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))]
    best = None
    for cand in cands:
        if not np.isfinite(cand):
            continue
        dist = abs(Fraction(float(cand)) - fr)
        even = (int(np.array(cand, dtype=np.float32).view(np.uint32)) & 1) == 0
        key = (dist, not even)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def exact_sum_f32(sq):
    """Correctly rounded float32 of the exact sum over the last axis.

    ``sq`` is a float32 array of non-negative values.  A float64 sum is
    exact whenever the exact total stays below 2**53 times the finest
    granularity among the terms (then every partial sum is an integer
    multiple of that granularity below 2**53); such rows take the float64
    sum.  Any other row is summed with exact rational arithmetic.
    """
    sq = np.asarray(sq, dtype=np.float32)
    flat = sq.reshape(-1, sq.shape[-1])
    out = np.empty(flat.shape[0], dtype=np.float32)
    block = 1 << 15
    for r0 in range(0, flat.shape[0], block):
        blk = flat[r0:r0 + block].astype(np.float64)
        s64 = blk.sum(axis=-1)
        _, e = np.frexp(blk)
        gran = np.where(blk > 0, np.ldexp(1.0, e - 24), np.inf).min(axis=-1)
        exact = (s64 == 0) | (s64 < np.ldexp(gran, 52))
        res = s64.astype(np.float32)
        for i in np.nonzero(~exact)[0]:
            fr = sum((Fraction(float(v)) for v in blk[i]), Fraction(0))
            res[i] = _fraction_to_f32(fr)
        out[r0:r0 + block] = res
    return out.reshape(sq.shape[:-1])


def l2norm_bf16(x):
    """Normalise rows of ``x`` (float32 values, normally bf16-exact).

    Returns float32 values that are exactly representable in bfloat16.
    """
    xf = np.asarray(x, dtype=np.float32)
    sq = xf * xf
    s = exact_sum_f32(sq)[..., None]
    t = s + EPS32
    den = np.sqrt(t)
    with np.errstate(divide="ignore", invalid="ignore"):
        quo = xf / den
    return bits_to_f32(bf16_bits(quo))
