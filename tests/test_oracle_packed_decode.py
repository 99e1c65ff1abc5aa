"""Pins for the oracle's packed decode front-end.

The row extraction and the padding are pinned by composition with the
(independently pinned) decode step at a point where both transforms have
closed forms: raw_gate = -dt_bias gives g = lower_bound / 2 = -2.5 in every
channel and raw_beta = 0 gives beta = 1/2.  The gate transform's formula is
not on the pages ("parity unpinned"); its closed-form properties are pinned:
the midpoint, both limits, monotonicity and the open range (-5, 0).
"""

import numpy as np
import torch

import oracle
import synth
from oracle import packed_decode as pd


def test_beta_sigmoid_closed_forms():
    x = np.array([[0.0, 2.0, -2.0, 40.0, -40.0]])
    b = pd.beta_from_logits(x)
    assert b[0, 0] == 0.5
    np.testing.assert_allclose(b[0, 1] + b[0, 2], 1.0, rtol=0, atol=1e-15)
    assert b[0, 3] == 1.0 and 0 < b[0, 4] < 1e-17


def test_gate_closed_forms():
    H, K = 2, 4
    dt = np.linspace(-1, 1, H * K)
    A_log = np.array([0.0, np.log(8.0)])
    # midpoint: raw + bias = 0 -> sigmoid(0) = 1/2 -> g = -2.5, whatever A_log is
    g = pd.gate(-dt[None, :], A_log, dt)
    assert np.all(g == -2.5)
    # limits: far positive -> lower bound, far negative -> 0 (from below)
    g_hi = pd.gate(np.full((1, H * K), 60.0), A_log, np.zeros(H * K))
    g_lo = pd.gate(np.full((1, H * K), -60.0), A_log, np.zeros(H * K))
    assert np.all(g_hi == -5.0)
    assert np.all(g_lo < 0) and np.all(g_lo > -1e-20)
    # A_log scales the slope: exp(A_log) = 8 -> head 1 at x equals head 0 at 8x
    x = np.array([[0.1, 0.2, 0.3, 0.4, 0.1, 0.2, 0.3, 0.4]])
    g2 = pd.gate(x, A_log, np.zeros(H * K))
    g0 = pd.gate(8 * x, np.zeros(H), np.zeros(H * K))
    np.testing.assert_allclose(g2[0, 1], g0[0, 1], rtol=1e-15)


def test_gate_monotone_and_in_range():
    rng = np.random.default_rng(3)
    x = np.sort(rng.standard_normal(1000) * 5)
    g = pd.gate(x[None, :], np.array([0.5]), np.zeros(1000))[0, 0]
    assert np.all(np.diff(g) <= 0)
    assert np.all(g > -5.0) and np.all(g < 0.0)


def test_extraction_by_composition_with_decode():
    inp = synth.packed_decode_config(16, N=40, H=3, row_pad=24)
    m = inp.mixed_qkv.float().numpy()
    assert np.all(np.isnan(m[:, 3 * 3 * 128:]))          # the padding is poison
    H, K = 3, 128
    dt = inp.dt_bias.numpy()
    raw_gate = -dt[None, :].repeat(16, 0)                  # x = 0 exactly -> g = -2.5
    raw_beta = np.zeros((16, H))                           # beta = 1/2
    pool = inp.pool.float().numpy()
    idx = inp.state_indices.numpy()
    o, new = oracle.packed_decode_step(m, raw_gate, raw_beta, inp.A_log.numpy(), dt, pool, idx)
    q = m[:, :H * K].reshape(16, H, K)
    k = m[:, H * K:2 * H * K].reshape(16, H, K)
    v = m[:, 2 * H * K:3 * H * K].reshape(16, H, K)
    o_ref, new_ref = oracle.decode_step(q, k, v, np.full((16, H, K), -2.5), np.full((16, H), 0.5), pool, idx)
    assert np.all(np.isfinite(o))
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(new, new_ref)


def test_row_order_is_q_k_v():
    # a packed row whose k block is zero leaves the state unchanged by the
    # delta term and gives o = scale * q^T (e^g S); with S = 0, o = 0 and r = v
    H, K = 1, 128
    q = np.zeros((1, 3 * H * K), np.float32)
    q[0, 0] = 1.0                       # q = e0
    q[0, 2 * H * K:] = 0.5              # v = 0.5
    k_block = slice(H * K, 2 * H * K)
    q[0, k_block] = 0.0
    q[0, H * K + 1] = 1.0               # k = e1
    pool = np.zeros((1, H, K, K), np.float32)
    o, new = oracle.packed_decode_step(q, np.zeros((1, K)), np.zeros((1, H)), np.zeros(H), np.zeros(K),
                                       pool, np.array([0]))
    # S' = beta k v^T = 0.5 * e1 (0.5)^T -> row 1 of the state is 0.25; q = e0 reads row 0 -> o = 0
    assert np.all(new[0, 0, 1] == 0.25) and np.all(new[0, 0, [0, 2]] == 0)
    assert np.all(o == 0)
