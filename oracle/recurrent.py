"""Token-by-token KDA recurrence in float64 (oracle form 1).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "KDA Chunk Prefill on Ascend A3", section "Mathematical definition",
the recurrent semantics for one batch row and one value head with a [K, V]
state.  Each token first multiplies key row d of the state by exp(g_t[d]);
it then measures the residual between its value and what the decayed state
already returns for its key, and adds the outer product of the key with
beta_t times that residual (the delta-rule write); its output is the scaled
query (K**-0.5 q_t) read against the updated state.

q and k enter already L2-normalised and rounded to bfloat16 (section
"Mathematical definition": the normalised bf16 values are widened for the
rest of the computation).  Section "Function and tensor contract": value
head h reads Q/K head h // (HV // H).

Readings where the page is silent:
  * g is [B, T, HV, K] and beta is [B, T, HV]: the gate and the write
    strength belong to the value head whose state they act on.
  * cu_seqlens (int [N+1], B == 1) packs N independent sequences along T,
    each with its own initial and final state; a length-0 sequence returns
    its initial state unchanged.
  * initial_state None means zeros, and the final state is still returned.
"""

import numpy as np

from .l2norm import l2norm_bf16


def _segments(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    if B != 1:
        raise ValueError("cu_seqlens requires B == 1")
    cu = [int(c) for c in np.asarray(cu_seqlens).tolist()]
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def recurrent(q, k, v, g, beta, initial_state=None, cu_seqlens=None, normalize=True):
    """Run the recurrence.

    Shapes: q, k [B,T,H,K]; v [B,T,HV,V]; g [B,T,HV,K]; beta [B,T,HV];
    initial_state [N,HV,K,V] or None; cu_seqlens int [N+1] or None (N = B).
    Values are float arrays (bf16 inputs passed as their exact float32
    values).  Returns (o [B,T,HV,V] float64, final_state [N,HV,K,V] float64).
    """
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
    # value head h reads Q/K head h // group
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
        for t in range(t0, t1):
            S = np.exp(g[b, t])[:, :, None] * S
            kt = kh[b, t]
            r = v[b, t] - np.einsum("hk,hkv->hv", kt, S)
            S = S + beta[b, t][:, None, None] * kt[:, :, None] * r[:, None, :]
            o[b, t] = scale * np.einsum("hk,hkv->hv", qh[b, t], S)
        final[n] = S
    return o, final
