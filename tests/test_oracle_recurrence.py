"""Pins for the fp64 oracle's two forms (recurrent and chunked).

Each check is fixed by the pages or by the mathematics, not by re-typing the
oracle's formulas: the pages' worked example and beta = 0 case, closed forms
that follow from the recurrence, the delta rule's retrieval identity, and the
two independent forms checked against each other, against padding, head
expansion, sequence packing and state carry.
"""

import json
import os

import numpy as np
import pytest

import oracle
import synth
from oracle.bf16 import bf16_round

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FORMS = [oracle.recurrent, oracle.chunked]


def _np(inp):
    a = synth.to_numpy(inp)
    return [a[n] for n in ("q", "k", "v", "g", "beta")], a["initial_state"], a["cu_seqlens"]


def _rand(seed, B, T, H, HV, K, V, *, gate_div=8.0, s0=True):
    rng = np.random.default_rng(seed)
    q = bf16_round(rng.standard_normal((B, T, H, K)).astype(np.float32))
    k = bf16_round(rng.standard_normal((B, T, H, K)).astype(np.float32))
    v = bf16_round(rng.standard_normal((B, T, HV, V)).astype(np.float32))
    g = (np.log(1 / (1 + np.exp(-rng.standard_normal((B, T, HV, K))))) / gate_div).astype(np.float32)
    beta = bf16_round((1 / (1 + np.exp(-rng.standard_normal((B, T, HV))))).astype(np.float32))
    S0 = (0.25 * rng.standard_normal((B, HV, K, V))).astype(np.float32) if s0 else None
    return [q, k, v, g, beta], S0


# ---------------------------------------------------------------- the pages


@pytest.mark.parametrize("form", FORMS)
def test_worked_example(form):
    gold = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    args, S0, _ = _np(synth.worked_example(T=gold["shape"]["T"]))
    o, S = form(*args, S0)
    ob = bf16_round(o.astype(np.float32))
    assert np.all(ob == gold["o_every_element_bf16"])
    assert np.all(S[0, 0, 0] == gold["final_state_row0"])
    assert np.all(S[0, 0, 1:] == gold["final_state_other_rows"])


@pytest.mark.parametrize("form", FORMS)
def test_beta_zero_gives_zero(form):
    gold = json.load(open(os.path.join(GOLDEN, "worked_example.json")))["beta_zero"]
    args, S0, _ = _np(synth.worked_example(beta_value=0.0))
    o, S = form(*args, S0)
    assert np.all(o == gold["o"]) and np.all(S == gold["final_state"])
    # also for random inputs
    args, _ = _rand(3, 1, 150, 2, 2, 16, 16)
    args[4][:] = 0.0
    o, S = form(*args, None)
    assert np.all(o == 0.0) and np.all(S == 0.0)


# ---------------------------------------------------------------- closed forms


@pytest.mark.parametrize("form", FORMS)
def test_beta_zero_pure_decay(form):
    """beta = 0: the state only decays, S_t = exp(sum_{u<=t} g_u) * S0 row-wise
    and o_t = K^-1/2 (q_t * exp(Ghat_t))^T S0, including decay far beyond the
    float range of exp(-G) over a chunk (g = -5 on some channels)."""
    args, S0 = _rand(5, 1, 200, 1, 1, 16, 8, gate_div=1.0)
    q, k, v, g, beta = args
    beta[:] = 0.0
    g[..., :4] = -5.0
    o, S = form(q, k, v, g, beta, S0)
    qn = oracle.l2norm_bf16(q).astype(np.float64)[0, :, 0]
    Ghat = np.cumsum(g[0, :, 0].astype(np.float64), axis=0)       # [T,K]
    expect_o = (qn * np.exp(Ghat)) @ S0[0, 0].astype(np.float64) * 16 ** -0.5
    expect_S = np.exp(Ghat[-1])[:, None] * S0[0, 0]
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o[0, :, 0], expect_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S[0, 0], expect_S, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("form", FORMS)
def test_orthonormal_keys(form):
    """k_t = q_t = e_t, g = 0, beta = 1, S0 = 0: S_t = sum_{u<=t} e_u v_u^T, so
    o_t = K^-1/2 v_t and the final state's rows are the values."""
    T, K, V = 100, 128, 32
    eye = np.eye(K, dtype=np.float32)
    q = eye[:T][None, :, None, :].copy()
    k = q.copy()
    rng = np.random.default_rng(1)
    v = bf16_round(rng.standard_normal((1, T, 1, V)).astype(np.float32))
    g = np.zeros((1, T, 1, K), np.float32)
    beta = np.ones((1, T, 1), np.float32)
    o, S = form(q, k, v, g, beta, None)
    np.testing.assert_allclose(o[0, :, 0], K ** -0.5 * v[0, :, 0].astype(np.float64), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S[0, 0, :T], v[0, :, 0], rtol=1e-13, atol=1e-15)
    assert np.all(S[0, 0, T:] == 0)


@pytest.mark.parametrize("form", FORMS)
def test_repeated_key_overwrites(form):
    """k_t = q_t = e0, beta = 1, g = 0: each write replaces row 0 with v_t (the
    delta rule's overwrite); o_t = K^-1/2 v_t; other rows keep S0."""
    T, K, V = 150, 32, 16
    rng = np.random.default_rng(2)
    q = np.zeros((1, T, 1, K), np.float32)
    q[..., 0] = 1
    k = q.copy()
    v = bf16_round(rng.standard_normal((1, T, 1, V)).astype(np.float32))
    g = np.zeros((1, T, 1, K), np.float32)
    beta = np.ones((1, T, 1), np.float32)
    S0 = rng.standard_normal((1, 1, K, V)).astype(np.float32)
    o, S = form(q, k, v, g, beta, S0)
    np.testing.assert_allclose(o[0, :, 0], K ** -0.5 * v[0, :, 0].astype(np.float64), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S[0, 0, 0], v[0, -1, 0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S[0, 0, 1:], S0[0, 0, 1:], rtol=1e-12)


def _unit_keys(rng, T, K):
    """Keys with four entries of +-0.5: exactly unit norm, unchanged by the
    bf16 normalisation."""
    k = np.zeros((T, K), np.float32)
    for t in range(T):
        idx = rng.choice(K, 4, replace=False)
        k[t, idx] = rng.choice([-0.5, 0.5], 4)
    return k


@pytest.mark.parametrize("form", FORMS)
def test_retrieval_identity(form):
    """For a unit key and beta = 1, the written state retrieves exactly the
    written value: k_T^T S_T = v_T, whatever the decay and prior state; with
    q = k the last output is K^-1/2 v_T."""
    T, K, V = 130, 32, 24
    rng = np.random.default_rng(4)
    k = _unit_keys(rng, T, K)[None, :, None, :]
    assert np.all(oracle.l2norm_bf16(k) == k)
    q = k.copy()
    v = bf16_round(rng.standard_normal((1, T, 1, V)).astype(np.float32))
    g = (-rng.random((1, T, 1, K)) * 2).astype(np.float32)
    beta = np.ones((1, T, 1), np.float32)
    S0 = rng.standard_normal((1, 1, K, V)).astype(np.float32)
    o, S = form(q, k, v, g, beta, S0)
    np.testing.assert_allclose(k[0, -1, 0] @ S[0, 0], v[0, -1, 0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(o[0, -1, 0], K ** -0.5 * v[0, -1, 0].astype(np.float64), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("form", FORMS)
def test_very_negative_gate(form):
    """g = -100: the carried state vanishes each step, so S_t = beta_t k_t v_t^T
    and o_t = K^-1/2 beta_t (q_t . k_t) v_t; no inf*0 anywhere."""
    args, S0 = _rand(6, 1, 140, 1, 1, 16, 8)
    q, k, v, g, beta = args
    g[:] = -100.0
    o, S = form(q, k, v, g, beta, S0)
    qn = oracle.l2norm_bf16(q).astype(np.float64)[0, :, 0]
    kn = oracle.l2norm_bf16(k).astype(np.float64)[0, :, 0]
    b = beta[0, :, 0].astype(np.float64)
    expect = 16 ** -0.5 * (b * np.sum(qn * kn, axis=1))[:, None] * v[0, :, 0].astype(np.float64)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    np.testing.assert_allclose(o[0, :, 0], expect, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(S[0, 0], b[-1] * np.outer(kn[-1], v[0, -1, 0].astype(np.float64)), rtol=1e-10, atol=1e-14)


# ---------------------------------------------------------------- two forms


@pytest.mark.parametrize("T", [1, 2, 15, 63, 64, 65, 127, 130])
@pytest.mark.parametrize("C", [16, 32, 64, 128])
def test_recurrent_equals_chunked(T, C):
    args, S0 = _rand(100 + T, 2, T, 1, 2, 8, 4, gate_div=1.0)
    o1, S1 = oracle.recurrent(*args, S0)
    o2, S2 = oracle.chunked(*args, S0, C=C)
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(S2, S1, rtol=1e-11, atol=1e-13)


def test_recurrent_equals_chunked_full_width_harsh():
    """K = V = 128 with the harsh-decay draw of the T=1000 workload (two heads,
    first 200 tokens): exp(-G) over a chunk would overflow here."""
    inp = synth.config1()
    a = synth.to_numpy(inp)
    sl = (slice(None), slice(0, 200), slice(0, 2))
    args = [a[n][sl] for n in ("q", "k", "v", "g")] + [a["beta"][:, :200, :2]]
    S0 = a["initial_state"][:, :2]
    o1, S1 = oracle.recurrent(*args, S0)
    o2, S2 = oracle.chunked(*args, S0)
    assert np.all(np.isfinite(o2))
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(S2, S1, rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("form", FORMS)
def test_zero_padding_invariance(form):
    """Tokens with q = k = v = 0, g = 0, beta = 0 leave the state alone and emit
    zeros (the page pads the last partial chunk this way)."""
    args, S0 = _rand(7, 1, 70, 1, 1, 16, 8)
    o1, S1 = form(*args, S0)
    padded = [np.concatenate([x, np.zeros((1, 30) + x.shape[2:], x.dtype)], axis=1) for x in args]
    o2, S2 = form(*padded, S0)
    np.testing.assert_allclose(o2[:, :70], o1, rtol=1e-12, atol=1e-15)
    assert np.all(o2[:, 70:] == 0)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("form", FORMS)
def test_gqa_head_mapping(form):
    """H=2, HV=4 equals H=HV=4 with each Q/K head repeated for its two value
    heads (value head h reads Q/K head h // (HV // H))."""
    args, S0 = _rand(8, 1, 90, 2, 4, 16, 8)
    o1, S1 = form(*args, S0)
    q, k, v, g, beta = args
    q4 = q[:, :, [0, 0, 1, 1]]
    k4 = k[:, :, [0, 0, 1, 1]]
    o2, S2 = form(q4, k4, v, g, beta, S0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


@pytest.mark.parametrize("form", FORMS)
def test_varlen_equals_separate(form):
    lens = [70, 0, 1, 129, 64]
    T = sum(lens)
    args, _ = _rand(9, 1, T, 1, 2, 16, 8)
    rng = np.random.default_rng(10)
    S0 = rng.standard_normal((len(lens), 2, 16, 8)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, S = form(*args, S0, cu_seqlens=cu)
    for n, L in enumerate(lens):
        sl = slice(cu[n], cu[n + 1])
        part = [x[:, sl] for x in args]
        o1, S1 = form(*part, S0[n:n + 1])
        np.testing.assert_allclose(o[:, sl], o1, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(S[n:n + 1], S1, rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(S[1], S0[1])  # empty sequence keeps its state


@pytest.mark.parametrize("form", FORMS)
def test_state_carry_split(form):
    args, S0 = _rand(11, 1, 200, 1, 1, 16, 8)
    o, S = form(*args, S0)
    first = [x[:, :128] for x in args]
    second = [x[:, 128:] for x in args]
    oa, Sa = form(*first, S0)
    ob, Sb = form(*second, Sa.astype(np.float64))
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(Sb, S, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("form", FORMS)
def test_value_linearity(form):
    """With S0 = 0 the outputs and state are linear in v."""
    args, _ = _rand(12, 1, 100, 1, 1, 16, 8)
    q, k, v1, g, beta = args
    v2 = np.random.default_rng(13).standard_normal(v1.shape)
    oa, Sa = form(q, k, 3.0 * v1 + v2, g, beta, None)
    o1, S1 = form(q, k, v1, g, beta, None)
    o2, S2 = form(q, k, v2, g, beta, None)
    np.testing.assert_allclose(oa, 3.0 * o1 + o2, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(Sa, 3.0 * S1 + S2, rtol=1e-10, atol=1e-13)


def test_parallel_runner_equals_recurrent():
    """The multi-process runner reassembles exactly what the serial
    recurrence computes (varlen with an empty sequence, GQA)."""
    from oracle.parallel import recurrent_parallel
    cu = np.array([0, 40, 40, 95, 130])
    args, _ = _rand(21, 1, 130, 2, 4, 16, 8)
    S0 = 0.25 * np.random.default_rng(22).standard_normal((4, 4, 16, 8))
    o1, s1 = oracle.recurrent(*args, S0, cu)
    o2, s2 = recurrent_parallel(*args, S0, cu, workers=3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)
