"""Packed decode front-end: one decode step from the serving-native packed
inputs, float64 arithmetic.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "flashinfer.kda_decode.packed_kda_decode" (its description and the
section "Parameters").  The operator takes the post-convolution packed QKV
row, raw per-channel gate logits and raw beta logits of each batch row,
plus per-head A_log and per-channel dt_bias, and fuses: Q/K extraction and
L2 normalisation, a lower-bound gate transform with lower_bound = -5, a
sigmoid on beta, and one recurrent step against the bf16 state pool (the
step of decode.decode_step).  Shapes: mixed_qkv [B, 3*H*K] (rows may be
padded), raw_gate [B, H*K], raw_beta [B, H], A_log [H], dt_bias [H*K].

Readings where the pages are silent:
  * the packed row is q | k | v, each [H, K] head-major;
  * the gate is g = lower_bound * sigmoid(exp(A_log[h]) * (raw_gate + dt_bias)).
    The page names the transform, its parameters and lower_bound = -5 but
    prints no formula; this is the plainest form built from exactly those
    parameters whose log-decay stays in (lower_bound, 0).  PARITY UNPINNED
    for this formula: the tests pin only its closed-form properties;
  * beta = sigmoid(raw_beta), used unrounded.
"""

import numpy as np

from .decode import decode_step

LOWER_BOUND = -5.0


def _sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gate(raw_gate, A_log, dt_bias):
    """raw_gate [B, H*K]; A_log [H]; dt_bias [H*K] -> g [B, H, K] (float64)."""
    raw = np.asarray(raw_gate, dtype=np.float64)
    B = raw.shape[0]
    H = np.asarray(A_log).shape[0]
    x = (raw + np.asarray(dt_bias, dtype=np.float64)[None, :]).reshape(B, H, -1)
    a = np.exp(np.asarray(A_log, dtype=np.float64))[None, :, None]
    return LOWER_BOUND * _sigmoid(a * x)


def beta_from_logits(raw_beta):
    """raw_beta [B, H] -> beta [B, H] (float64)."""
    return _sigmoid(raw_beta)


def unpack(mixed_qkv, H, K):
    """mixed_qkv [B, >= 3*H*K] -> q, k, v each [B, H, K] (padding ignored)."""
    m = np.asarray(mixed_qkv)
    B = m.shape[0]
    q = m[:, 0 * H * K:1 * H * K].reshape(B, H, K)
    k = m[:, 1 * H * K:2 * H * K].reshape(B, H, K)
    v = m[:, 2 * H * K:3 * H * K].reshape(B, H, K)
    return q, k, v


def packed_decode_step(mixed_qkv, raw_gate, raw_beta, A_log, dt_bias, pool, state_indices):
    """Returns (o [B, H, V] float64, new_pool float32 bf16 values); the input
    pool is not modified."""
    H = np.asarray(A_log).shape[0]
    K = pool.shape[2]
    q, k, v = unpack(mixed_qkv, H, K)
    g = gate(raw_gate, A_log, dt_bias)
    beta = beta_from_logits(raw_beta)
    return decode_step(q, k, v, g, beta, pool, state_indices)
