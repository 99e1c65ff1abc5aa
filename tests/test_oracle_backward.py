"""Pins for the oracle's backward (float64 autodiff of the recurrence).

The differentiation is checked against central finite differences of an
independently written float64 forward (plain NumPy loop) on tiny shapes,
with the bf16 rounding of q^, k^ switched off so that the function is
smooth; against the closed form of a single token from a zero state; and
against two structural identities (beta = 0 makes v irrelevant; a shared
Q/K head receives the sum of its value heads' gradients).
"""

import numpy as np
import pytest

import oracle


def _forward_loss(q, k, v, g, beta, s0, do, dht):
    """Independent float64 forward: normalise, run the recurrence, return
    sum(o * do) + sum(S_T * dht).  B = 1, no cu_seqlens."""
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    grp = HV // H
    scale = K ** -0.5
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
    kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + 1e-6)
    loss = 0.0
    S = [s0[0, h].copy() for h in range(HV)]
    for t in range(T):
        for h in range(HV):
            qq, kk = qn[0, t, h // grp], kn[0, t, h // grp]
            Sd = np.exp(g[0, t, h])[:, None] * S[h]
            r = v[0, t, h] - kk @ Sd
            S[h] = Sd + beta[0, t, h] * np.outer(kk, r)
            loss += scale * (qq @ S[h]) @ do[0, t, h]
    for h in range(HV):
        loss += (S[h] * dht[0, h]).sum()
    return loss


def _inputs(rng, T=4, H=1, HV=2, K=6, V=5):
    q = rng.standard_normal((1, T, H, K))
    k = rng.standard_normal((1, T, H, K))
    v = rng.standard_normal((1, T, HV, V))
    g = -0.5 * rng.random((1, T, HV, K))
    beta = rng.random((1, T, HV))
    s0 = 0.3 * rng.standard_normal((1, HV, K, V))
    do = rng.standard_normal((1, T, HV, V))
    dht = rng.standard_normal((1, HV, K, V))
    return q, k, v, g, beta, s0, do, dht


def test_finite_differences():
    rng = np.random.default_rng(1)
    args = _inputs(rng)
    grads = oracle.recurrent_backward(*args[:6], args[6], args[7], round_bf16=False)
    eps = 1e-6
    for which in range(6):
        x = args[which]
        for idx in [tuple(rng.integers(0, n) for n in x.shape) for _ in range(4)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            fd = (_forward_loss(*ap) - _forward_loss(*am)) / (2 * eps)
            ad = grads[which][idx]
            assert abs(fd - ad) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, ad)


def test_single_token_closed_form():
    # one token from a zero state: S = beta k^ v^T, o = K^-1/2 beta (q^.k^) v
    rng = np.random.default_rng(2)
    q, k, v, g, beta, s0, do, dht = _inputs(rng, T=1, H=1, HV=1)
    s0[:] = 0
    dq, dk, dv, dg, db, dh0 = oracle.recurrent_backward(q, k, v, g, beta, s0, do, dht, round_bf16=False)
    K = q.shape[-1]
    qn = q[0, 0, 0] / np.sqrt((q[0, 0, 0] ** 2).sum() + 1e-6)
    kn = k[0, 0, 0] / np.sqrt((k[0, 0, 0] ** 2).sum() + 1e-6)
    b = beta[0, 0, 0]
    dv_ref = K ** -0.5 * b * (qn @ kn) * do[0, 0, 0] + b * (kn @ dht[0, 0])
    db_ref = K ** -0.5 * (qn @ kn) * (v[0, 0, 0] @ do[0, 0, 0]) + kn @ dht[0, 0] @ v[0, 0, 0]
    np.testing.assert_allclose(dv[0, 0, 0], dv_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(db[0, 0, 0], db_ref, rtol=1e-12, atol=1e-14)
    # from a zero state the gate only scales zeros
    np.testing.assert_allclose(dg, 0.0, atol=1e-15)


def test_beta_zero_leaves_v_out():
    rng = np.random.default_rng(3)
    q, k, v, g, beta, s0, do, dht = _inputs(rng)
    beta[:] = 0
    dq, dk, dv, dg, db, dh0 = oracle.recurrent_backward(q, k, v, g, beta, s0, do, dht)
    assert np.all(dv == 0) and np.all(dk == 0)


def test_shared_qk_head_sums_value_heads():
    rng = np.random.default_rng(4)
    q, k, v, g, beta, s0, do, dht = _inputs(rng, H=1, HV=2)
    dq, dk, dv, dg, db, dh0 = oracle.recurrent_backward(q, k, v, g, beta, s0, do, dht)
    qe, ke = np.repeat(q, 2, axis=2), np.repeat(k, 2, axis=2)
    eq, ek, ev, eg, eb, eh = oracle.recurrent_backward(qe, ke, v, g, beta, s0, do, dht)
    np.testing.assert_allclose(dq[:, :, 0], eq.sum(2), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk[:, :, 0], ek.sum(2), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dv, ev, rtol=1e-12, atol=1e-14)


def _segment_loss(q, k, v, g, beta, s0, do, dht, cu):
    """Independent float64 forward over packed sequences: each segment
    [cu[n], cu[n+1]) of the token axis restarts from its own state s0[n]
    (zeros when s0 is None).  Returns the same scalar loss."""
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    grp = HV // H
    scale = K ** -0.5
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
    kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + 1e-6)
    loss = 0.0
    for n in range(len(cu) - 1):
        for h in range(HV):
            S = np.zeros((K, V)) if s0 is None else s0[n, h].copy()
            for t in range(cu[n], cu[n + 1]):
                qq, kk = qn[0, t, h // grp], kn[0, t, h // grp]
                S = np.exp(g[0, t, h])[:, None] * S
                S = S + beta[0, t, h] * np.outer(kk, v[0, t, h] - kk @ S)
                loss += scale * (qq @ S) @ do[0, t, h]
            loss += (S * dht[n, h]).sum()
    return loss


def test_varlen_finite_differences():
    """The cu_seqlens path, an empty sequence included, against central
    finite differences of the independent segmented forward."""
    rng = np.random.default_rng(5)
    cu = [0, 3, 3, 7, 9]
    q, k, v, g, beta, _, do, _ = _inputs(rng, T=9, H=1, HV=2)
    s0 = 0.3 * rng.standard_normal((4, 2, q.shape[-1], v.shape[-1]))
    dht = rng.standard_normal(s0.shape)
    args = [q, k, v, g, beta, s0]
    grads = oracle.recurrent_backward(*args, do, dht, cu_seqlens=np.array(cu), round_bf16=False)
    eps = 1e-6
    for which in range(6):
        x = args[which]
        picks = [tuple(rng.integers(0, n) for n in x.shape) for _ in range(4)]
        if which == 5:
            picks.append((1, 0, 2, 3))            # the empty sequence's state: gradient is dht itself
        for idx in picks:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            fd = (_segment_loss(*ap, do, dht, cu) - _segment_loss(*am, do, dht, cu)) / (2 * eps)
            ad = grads[which][idx]
            assert abs(fd - ad) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, ad)
    # the empty sequence passes its state through untouched
    np.testing.assert_array_equal(grads[5][1], dht[1])


def test_varlen_equals_separate_sequences():
    """Packed sequences give the gradients of separate single-sequence runs."""
    rng = np.random.default_rng(6)
    cu = [0, 4, 4, 9]
    q, k, v, g, beta, _, do, _ = _inputs(rng, T=9, H=1, HV=2)
    s0 = 0.3 * rng.standard_normal((3, 2, q.shape[-1], v.shape[-1]))
    dht = rng.standard_normal(s0.shape)
    packed = oracle.recurrent_backward(q, k, v, g, beta, s0, do, dht, cu_seqlens=np.array(cu))
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        sl = lambda x: x[:, a:b]
        one = oracle.recurrent_backward(sl(q), sl(k), sl(v), sl(g), sl(beta), s0[n:n + 1], sl(do),
                                        dht[n:n + 1])
        for got, want in zip(packed[:5], one[:5]):
            np.testing.assert_allclose(got[:, a:b], want, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(packed[5][n:n + 1], one[5], rtol=1e-12, atol=1e-14)


def test_absent_initial_state_is_zero_state():
    """initial_state None: the token gradients equal those at an explicit
    zero state, and no initial-state gradient is returned; also with
    cu_seqlens and with a batch of two rows."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, s0, do, dht = _inputs(rng, T=6, H=1, HV=2)
    none = oracle.recurrent_backward(q, k, v, g, beta, None, do, dht)
    zero = oracle.recurrent_backward(q, k, v, g, beta, np.zeros_like(s0), do, dht)
    assert none[5] is None and zero[5] is not None
    for a, b in zip(none[:5], zero[:5]):
        np.testing.assert_array_equal(a, b)
    cu = np.array([0, 2, 6])
    dht2 = rng.standard_normal((2,) + s0.shape[1:])
    none = oracle.recurrent_backward(q, k, v, g, beta, None, do, dht2, cu_seqlens=cu)
    zero = oracle.recurrent_backward(q, k, v, g, beta, np.zeros_like(dht2), do, dht2, cu_seqlens=cu)
    assert none[5] is None
    for a, b in zip(none[:5], zero[:5]):
        np.testing.assert_array_equal(a, b)


def test_batch_rows_are_independent():
    """B = 2 without cu_seqlens (the zero-state path the GPU batch case
    uses) equals two single-row runs."""
    rng = np.random.default_rng(8)
    parts = [_inputs(rng, T=5, H=1, HV=2) for _ in range(2)]
    cat = [np.concatenate([p[i] for p in parts], axis=0) for i in range(8)]
    q, k, v, g, beta, s0, do, dht = cat
    both = oracle.recurrent_backward(q, k, v, g, beta, None, do, dht)
    assert both[5] is None
    for b in range(2):
        p = parts[b]
        one = oracle.recurrent_backward(*p[:5], None, p[6], p[7])
        for got, want in zip(both[:5], one[:5]):
            np.testing.assert_allclose(got[b:b + 1], want, rtol=1e-12, atol=1e-14)
        # and the single row itself against finite differences of the zero-state forward
    z = np.zeros_like(parts[0][5])
    grads = oracle.recurrent_backward(*parts[0][:5], None, parts[0][6], parts[0][7], round_bf16=False)
    eps = 1e-6
    for which in range(5):
        x = parts[0][which]
        idx = tuple(rng.integers(0, n) for n in x.shape)
        xp, xm = x.copy(), x.copy()
        xp[idx] += eps
        xm[idx] -= eps
        ap, am = list(parts[0][:5]) + [z], list(parts[0][:5]) + [z]
        ap[which], am[which] = xp, xm
        fd = (_forward_loss(*ap, parts[0][6], parts[0][7]) - _forward_loss(*am, parts[0][6], parts[0][7])) / (2 * eps)
        assert abs(fd - grads[which][idx]) <= 1e-6 * max(1.0, abs(fd)), (which, idx)
