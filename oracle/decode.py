"""One decode step against a bf16 state pool, float64 arithmetic.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Sources:
  * "flashinfer.kda_decode.packed_kda_decode", section "Parameters": the
    state is a caller-owned bfloat16 pool [N, HV, K, V] updated in place at
    the slot that state_indices names for each batch row; -1 marks an
    inactive row, which produces zero output and neither reads nor writes
    the pool.  The fixed numerical contract is scale 1/sqrt(128) and L2
    epsilon 1e-6.
  * "KDA Chunk Prefill on Ascend A3", section "Mathematical definition":
    the recurrent step itself and the Q/K normalisation.

Readings where the pages are silent: the pool's axes are [slot, HV, K, V] with V
innermost (the same [K, V] orientation as the prefill state); o is formed
from the unrounded updated state, and the stored state is that state
rounded once to bf16 (nearest, ties to even).  The decode front-end of the
page (packed QKV extraction, gate transform, beta sigmoid) is not part of
this step: q, k, v, g and beta arrive already separated.
"""

import numpy as np

from .bf16 import f64_to_bf16_round
from .l2norm import l2norm_bf16


def decode_step(q, k, v, g, beta, pool, state_indices):
    """q, k [B,H,K]; v [B,HV,V]; g [B,HV,K]; beta [B,HV]; pool float32
    [N,HV,K,V] holding bf16 values; state_indices int [B].

    Returns (o [B,HV,V] float64, new_pool float32 bf16 values).  The input
    pool is not modified.
    """
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    B, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    group = HV // H
    qn = np.repeat(l2norm_bf16(q).astype(np.float64), group, axis=1)
    kn = np.repeat(l2norm_bf16(k).astype(np.float64), group, axis=1)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    scale = K ** -0.5
    new_pool = np.array(pool, dtype=np.float32, copy=True)
    o = np.zeros((B, HV, V), dtype=np.float64)
    for b in range(B):
        idx = int(state_indices[b])
        if idx < 0:
            continue
        S = np.asarray(pool[idx], dtype=np.float64)
        S = np.exp(g[b])[:, :, None] * S
        r = v[b] - np.einsum("hk,hkv->hv", kn[b], S)
        S = S + beta[b][:, None, None] * kn[b][:, :, None] * r[:, None, :]
        o[b] = scale * np.einsum("hk,hkv->hv", qn[b], S)
        new_pool[idx] = f64_to_bf16_round(S)
    return o, new_pool
