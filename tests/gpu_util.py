"""Shared helpers for the GPU parity tests (tolerances and comparisons)."""

import numpy as np
import torch

# Tolerances (the parity bar of the forward path, written here so every test uses the same):
#   o:            |o_gpu - o_ref| <= 1e-2 * max(1, |o_ref|) elementwise
#   final state:  ||S_gpu - S_ref||_F / ||S_ref||_F <= 1e-3 per (sequence, head);
#                 an all-zero reference requires an exactly zero result
O_TOL = 1e-2
STATE_TOL = 1e-3


def say(msg):
    print(msg, flush=True)


def bf16_bits_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_o(o_gpu, o_ref, what=""):
    o = o_gpu.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - o_ref) / np.maximum(1.0, np.abs(o_ref))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= O_TOL, f"{what}: o error {worst:.3e} > {O_TOL}"
    return worst


def check_state(s_gpu, s_ref, what=""):
    s = s_gpu.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(s)), f"{what}: non-finite state"
    worst = 0.0
    flat_g = s.reshape(-1, s.shape[-2] * s.shape[-1])
    flat_r = s_ref.reshape(-1, s_ref.shape[-2] * s_ref.shape[-1])
    for i in range(flat_r.shape[0]):
        nr = np.linalg.norm(flat_r[i])
        if nr == 0:
            assert np.all(flat_g[i] == 0), f"{what}: state {i} should be exactly zero"
            continue
        e = np.linalg.norm(flat_g[i] - flat_r[i]) / nr
        worst = max(worst, e)
    assert worst <= STATE_TOL, f"{what}: state rel-Frobenius {worst:.3e} > {STATE_TOL}"
    return worst
