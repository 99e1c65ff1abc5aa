"""Chunk construction of the KDA recurrence in float64 (oracle form 2).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "KDA Chunk Prefill on Ascend A3", section "Mathematical definition",
the equivalent construction for a chunk of C tokens (zero-based indices,
ordered by token position), for one value head:

    G_i     = sum_{u <= i} g_u                                (per channel)
    L_ij    = beta_i * sum_d k_id k_jd exp(G_id - G_jd)   for j <  i, else 0
    A       = solve(I + L, diag(beta))
    W       = A @ (exp(G) * k)
    U       = A @ v
    Qg_i    = K**-0.5 * q_i * exp(G_i)
    Kg_i    = k_i * exp(G_last - G_i)
    Aqk_ij  = K**-0.5 * sum_d q_id k_jd exp(G_id - G_jd)  for j <= i, else 0
    Vnew    = U - W @ S_in
    O       = Qg @ S_in + Aqk @ Vnew
    S_out   = exp(G_last)[:, None] * S_in + Kg^T @ Vnew

The page's golden uses C = 64 and zero-pads q, k, v, g and beta of the last
partial chunk, trims the output and keeps the state.  This module follows
that, with C a parameter.  It shares nothing with ``recurrent`` except the
L2 normalisation, so agreement between the two pins both.

The exponent differences G_i - G_j are formed only where j <= i (masked to
-inf elsewhere before exp), so no positive exponent is ever evaluated.
"""

import numpy as np

from .l2norm import l2norm_bf16
from .recurrent import _segments


def _chunk(qc, kc, vc, gc, bc, S, scale):
    """One chunk for all heads. qc,kc,gc [C,HV,K]; vc [C,HV,V]; bc [C,HV];
    S [HV,K,V].  Returns (O [C,HV,V], S_out)."""
    C = qc.shape[0]
    G = np.cumsum(gc, axis=0)                                  # [C,HV,K]
    diff = G[:, None] - G[None, :]                             # [i,j,HV,K]
    lower_incl = np.tril(np.ones((C, C), dtype=bool))          # j <= i
    lower_strict = np.tril(np.ones((C, C), dtype=bool), -1)    # j <  i
    E = np.exp(np.where(lower_incl[:, :, None, None], diff, -np.inf))
    kk = np.einsum("ihd,jhd,ijhd->hij", kc, kc, E)
    qk = np.einsum("ihd,jhd,ijhd->hij", qc, kc, E)
    L = np.where(lower_strict[None], bc.T[:, :, None] * kk, 0.0)   # [HV,i,j]
    Aqk = np.where(lower_incl[None], scale * qk, 0.0)
    eye = np.eye(C)[None]
    A = np.linalg.solve(eye + L, eye * bc.T[:, None, :])      # solve(I+L, diag(beta))
    eG = np.exp(G).transpose(1, 0, 2)                          # [HV,C,K]
    kT = kc.transpose(1, 0, 2)
    qT = qc.transpose(1, 0, 2)
    vT = vc.transpose(1, 0, 2)
    W = A @ (eG * kT)
    U = A @ vT
    Qg = scale * qT * eG
    Glast = G[-1]                                              # [HV,K]
    Kg = kT * np.exp(Glast[:, None, :] - G.transpose(1, 0, 2))
    Vnew = U - W @ S
    O = Qg @ S + Aqk @ Vnew
    S_out = np.exp(Glast)[:, :, None] * S + Kg.transpose(0, 2, 1) @ Vnew
    return O.transpose(1, 0, 2), S_out


def chunked(q, k, v, g, beta, initial_state=None, cu_seqlens=None, C=64, normalize=True):
    """Same contract as ``oracle.recurrent.recurrent``; chunk size C."""
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if HV % H:
        raise ValueError("HV must be a multiple of H")
    if normalize:
        q = l2norm_bf16(q)
        k = l2norm_bf16(k)
    group = HV // H
    qh = np.repeat(q.astype(np.float64), group, axis=2)
    kh = np.repeat(k.astype(np.float64), group, axis=2)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    scale = K ** -0.5

    segs = _segments(B, T, cu_seqlens)
    o = np.zeros((B, T, HV, V), dtype=np.float64)
    final = np.zeros((len(segs), HV, K, V), dtype=np.float64)
    for n, (b, t0, t1) in enumerate(segs):
        if initial_state is None:
            S = np.zeros((HV, K, V), dtype=np.float64)
        else:
            S = np.array(initial_state[n], dtype=np.float64)
        for c0 in range(t0, t1, C):
            c1 = min(c0 + C, t1)
            pad = C - (c1 - c0)

            def take(x):
                xc = x[b, c0:c1]
                if pad:
                    xc = np.concatenate([xc, np.zeros((pad,) + xc.shape[1:])], axis=0)
                return xc

            Oc, S = _chunk(take(qh), take(kh), take(v), take(g), take(beta), S, scale)
            o[b, c0:c1] = Oc[: c1 - c0]
        final[n] = S
    return o, final
