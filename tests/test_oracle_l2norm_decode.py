"""Pins for the oracle's bf16 helpers, the canonical L2 normalisation and the
decode step.

The L2 normalisation is checked against a brute-force evaluation of its
definition in exact rational arithmetic (independent rounding code), against
closed forms (unit and zero rows, power-of-two scaling), and against the
page's literal float32 torch formula, which it must match except for rare
one-ulp flips caused by torch's unspecified summation order.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.bf16 import bf16_bits, bf16_round, bits_to_f32, f64_to_bf16_round


def round_fraction(fr, p):
    """Independent exact rounding of a rational to p significant bits,
    nearest-even (normal range only)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    unit = Fraction(2) ** (e - p + 1)
    m = a / unit
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * unit


def brute_l2norm_row(x):
    xs = [Fraction(float(v)) for v in x]
    s = round_fraction(sum((v * v for v in xs), Fraction(0)), 24)
    t = round_fraction(s + Fraction(float(np.float32(1e-6))), 24)
    d0 = np.float32(np.sqrt(float(t)))
    cands = [np.nextafter(d0, np.float32(0)), d0, np.nextafter(d0, np.float32(np.inf))]
    d = None
    for i in (1, 0, 2):
        c = cands[i]
        lo = (Fraction(float(np.nextafter(c, np.float32(0)))) + Fraction(float(c))) / 2
        hi = (Fraction(float(c)) + Fraction(float(np.nextafter(c, np.float32(np.inf))))) / 2
        if lo * lo < t < hi * hi:
            d = Fraction(float(c))
            break
    assert d is not None
    return [float(round_fraction(round_fraction(v / d, 24), 8)) for v in xs]


# ---------------------------------------------------------------- bf16


def test_bf16_bits_matches_torch_rounding():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.standard_normal(100000) * 8)).astype(np.float32)
    ties = (rng.integers(0, 2 ** 16, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, np.inf, -np.inf, 3.4e38])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)   # NaN payloads are not part of the method; NaN must stay NaN
    assert np.all(np.isnan(bits_to_f32(bf16_bits(x[nan]))))
    np.testing.assert_array_equal(bf16_bits(x[~nan]), ref[~nan])
    np.testing.assert_array_equal(bf16_round(bits_to_f32(ref)), bits_to_f32(ref))


def test_f64_to_bf16_single_rounding():
    rng = np.random.default_rng(1)
    base = bf16_round(rng.standard_normal(3000).astype(np.float32)).astype(np.float64)
    ulp = np.abs(base) * 2.0 ** -7
    # exact midpoints, and midpoints nudged by far less than a float32 ulp
    mids = base + ulp / 2 * np.where(np.abs(base) >= 2 ** np.floor(np.log2(np.abs(base))), 1, 1)
    x = np.concatenate([mids, mids + ulp * 2.0 ** -30, mids - ulp * 2.0 ** -30,
                        rng.standard_normal(3000)])
    got = f64_to_bf16_round(x)
    for xi, gi in zip(x, got):
        assert Fraction(float(gi)) == round_fraction(Fraction(float(xi)), 8)


# ---------------------------------------------------------------- L2 norm


def test_l2norm_brute_force_exact_arithmetic():
    rng = np.random.default_rng(2)
    rows = []
    for _ in range(12):
        rows.append(np.exp(rng.standard_normal() * 0.6) * rng.standard_normal(16))
    for _ in range(6):   # wide dynamic range: the float64 fast path is not exact
        r = rng.standard_normal(16) * np.exp2(rng.integers(-40, 12, 16))
        rows.append(r)
    for _ in range(4):   # tiny rows, epsilon-dominated
        rows.append(rng.standard_normal(16) * 1e-5)
    x = bf16_round(np.array(rows, dtype=np.float32))
    got = oracle.l2norm_bf16(x)
    for i in range(x.shape[0]):
        assert list(got[i].astype(np.float64)) == brute_l2norm_row(x[i]), i


def test_l2norm_exact_sum_takes_rational_path():
    """A row whose squares span more than float64 can hold exactly."""
    x = np.zeros((1, 8), np.float32)
    x[0, 0] = 1.0
    x[0, 1] = np.float32(2.0 ** -60)
    x[0, 2] = np.float32(1.0 + 2.0 ** -7)
    s = oracle.l2norm.exact_sum_f32(x * x)
    exact = Fraction(1) + Fraction(2) ** -120 + (1 + Fraction(1, 128)) ** 2
    assert Fraction(float(s[0])) == round_fraction(exact, 24)


def test_l2norm_unit_and_zero_rows():
    K = 128
    e0 = np.zeros((2, K), np.float32)
    e0[0, 0] = 1.0
    got = oracle.l2norm_bf16(e0)
    assert np.array_equal(got[0], e0[0]) and np.all(got[1] == 0)
    neg = -e0[:1]
    assert np.array_equal(oracle.l2norm_bf16(neg), neg)


def test_l2norm_power_of_two_scaling_invariance():
    """Once the sum of squares is large enough that the epsilon is absorbed,
    scaling a row by 2**m scales the denominator exactly by 2**m."""
    rng = np.random.default_rng(3)
    x = bf16_round((8 + rng.standard_normal((500, 128))).astype(np.float32))
    assert np.all((x * x).sum(-1) >= 64)
    base = oracle.l2norm_bf16(x)
    for m in (1, 2, 5, 20):
        np.testing.assert_array_equal(oracle.l2norm_bf16(x * np.float32(2.0 ** m)), base)


def test_l2norm_agrees_with_literal_torch_formula():
    """The page's formula evaluated literally in float32 torch ops differs from
    the order-free canonical sum only by rare one-ulp flips."""
    inp = synth.prefill_stress(4, 1, 400, 16, 16, qk_mode="gain")
    x = inp.q.float().reshape(-1, 128)
    lit = (x / torch.sqrt((x * x).sum(-1, keepdim=True) + 1e-6)).to(torch.bfloat16).float().numpy()
    ours = oracle.l2norm_bf16(x.numpy())
    diff = ours != lit
    assert diff.mean() < 1e-3
    if diff.any():
        ub = bf16_bits(ours[diff]).astype(np.int32)
        lb = bf16_bits(lit[diff]).astype(np.int32)
        assert np.all(np.abs(ub - lb) == 1)


# ---------------------------------------------------------------- decode


def test_decode_is_one_recurrent_step():
    inp = synth.decode_config(8, N=32, H=4, HV=4)
    a = synth.to_numpy(inp)
    o, pool = oracle.decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], a["state_indices"])
    for b, idx in enumerate(a["state_indices"]):
        if idx < 0:
            assert np.all(o[b] == 0)
            continue
        r_o, r_S = oracle.recurrent(a["q"][b][None, None], a["k"][b][None, None], a["v"][b][None, None],
                                    a["g"][b][None, None], a["beta"][b][None, None], a["pool"][idx][None])
        np.testing.assert_allclose(o[b], r_o[0, 0], rtol=1e-13, atol=1e-15)
        np.testing.assert_array_equal(pool[idx], f64_to_bf16_round(r_S[0]))
    untouched = np.setdiff1d(np.arange(32), a["state_indices"][a["state_indices"] >= 0])
    np.testing.assert_array_equal(pool[untouched], a["pool"][untouched])


def test_decode_inactive_rows_and_retrieval():
    rng = np.random.default_rng(5)
    B, H, K = 3, 2, 16
    k = np.zeros((B, H, K), np.float32)
    for b in range(B):
        for h in range(H):
            idx = rng.choice(K, 4, replace=False)
            k[b, h, idx] = rng.choice([-0.5, 0.5], 4)
    q = k.copy()
    v = bf16_round(rng.standard_normal((B, H, 8)).astype(np.float32))
    g = -rng.random((B, H, K)).astype(np.float32)
    beta = np.ones((B, H), np.float32)
    pool = bf16_round(rng.standard_normal((4, H, K, 8)).astype(np.float32))
    idx = np.array([2, -1, 0], np.int32)
    o, new = oracle.decode_step(q, k, v, g, beta, pool, idx)
    assert np.all(o[1] == 0)
    np.testing.assert_allclose(o[[0, 2]], K ** -0.5 * v[[0, 2]].astype(np.float64), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(new[[1, 3]], pool[[1, 3]])
