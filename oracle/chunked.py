"""Chunk-parallel form of the KDA recurrence in float64 (oracle form 2).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "KDA Chunk Prefill on Ascend A3", section "Mathematical definition".
The page states the token recurrence and says an equivalent chunk-local
construction with an inter-chunk state carry computes the same result; the
golden uses 64-token chunks with the last partial chunk zero-padded (q, k, v,
g and beta all zero), the output trimmed and the state kept.  This module
does not restate the page's construction.  It derives the chunk form afresh
from the recurrence, as follows, and computes it that way.

Derivation (one value head; state S is [K, V]; inside a chunk the tokens are
numbered 1..C and S_0 is the state entering the chunk).  A token first
decays every key row of the state by exp(g_t) and then writes the rank-one
correction k_t u_t^T, where the "write" u_t = beta_t (v_t - k_t^T S') is the
delta-rule residual against the decayed state S'.  Let P_t be the running
per-channel decay exp(g_1 + ... + g_t) (a diagonal matrix).  Unrolling the
recurrence,

    state before token i's write = P_i S_0 + sum_{j<i} P_i P_j^-1 k_j u_j^T

(the product P_i P_j^-1 = exp(sum of g over tokens j+1..i) is at most 1, so
it is evaluated as one exponential of that partial sum, never as a ratio).
Substituting into the definition of u_i gives a unit lower-triangular system
for the writes of the whole chunk,

    u_i + beta_i sum_{j<i} M_ij u_j = beta_i (v_i - (P_i k_i)^T S_0),
    M_ij = sum_d k_id k_jd exp(G_id - G_jd),  G = running sum of g,

which is solved here by explicit forward substitution, one token at a time.
The outputs and the exiting state then follow from the same unrolling:

    o_i   = K^-1/2 [ (P_i q_i)^T S_0 + sum_{j<=i} N_ij u_j ],
            N_ij = sum_d q_id k_jd exp(G_id - G_jd)
    S_out = P_C S_0 + sum_j (P_C P_j^-1 k_j) u_j^T.

Nothing here is shared with ``recurrent`` except the L2 normalisation and
the sequence segmentation, so agreement between the two pins both.  The
exponent differences are formed only for j <= i (masked to -inf before the
exponential), so no positive exponent is ever evaluated.
"""

import numpy as np

from .l2norm import l2norm_bf16
from .recurrent import _segments


def _chunk(qc, kc, vc, gc, bc, S0, scale):
    """One chunk for all value heads.  qc, kc, gc [C,HV,K]; vc [C,HV,V];
    bc [C,HV]; S0 [HV,K,V].  Returns (o [C,HV,V], S_out [HV,K,V])."""
    C = qc.shape[0]
    G = np.cumsum(gc, axis=0)                                    # running log-decay [C,HV,K]
    incl = np.tril(np.ones((C, C), dtype=bool))                  # j <= i
    # pair decay exp(G_i - G_j) per channel, only where j <= i
    dec = np.exp(np.where(incl[:, :, None, None], G[:, None] - G[None, :], -np.inf))   # [i,j,HV,K]
    M = np.einsum("ihd,jhd,ijhd->hij", kc, kc, dec)             # key-key decayed overlaps
    N = np.einsum("ihd,jhd,ijhd->hij", qc, kc, dec)             # query-key decayed overlaps
    P = np.exp(G)                                                # decay since the chunk start
    # right-hand side: the residual of each token against the decayed entering state
    rhs = bc[:, :, None] * (vc - np.einsum("ihk,hkv->ihv", P * kc, S0))   # [C,HV,V]
    # forward substitution for the writes u
    u = np.zeros_like(rhs)
    for i in range(C):
        acc = np.einsum("hj,jhv->hv", M[:, i, :i], u[:i]) if i else 0.0
        u[i] = rhs[i] - bc[i][:, None] * acc
    o = scale * (np.einsum("ihk,hkv->ihv", P * qc, S0) + np.einsum("hij,jhv->ihv", N, u))
    # exiting state: decayed entering state plus every write, decayed to the chunk end
    tail = np.exp(G[-1][None] - G)                               # [C,HV,K], each <= 1
    S_out = P[-1][:, :, None] * S0 + np.einsum("jhk,jhv->hkv", tail * kc, u)
    return o, S_out


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
