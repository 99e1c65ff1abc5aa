"""Backward of the KDA forward: gradients by float64 automatic
differentiation of the token-by-token recurrence.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "KDA Chunk Prefill on Ascend A3" -- section "Mathematical
definition" (the recurrence and the Q/K normalisation) and the page's
optional backward: gradients of o and final_state with respect to q, k, v,
g, beta and initial_state (None when the initial state is absent).

Definition.  With upstream gradients do (shape of o) and dht (shape of
final_state), the gradients are those of the scalar
    sum(o * do) + sum(final_state * dht)
through the same recurrence as recurrent.recurrent, in float64.  Reading
(the page gives no backward formula): the normalised q^, k^ enter the recurrence rounded to
bf16 exactly as in the forward, and the rounding passes gradients through
unchanged (its derivative is taken as the identity), so dq and dk are the
gradients of the unrounded x / sqrt(sum(x*x) + 1e-6).  The pins in
tests/test_oracle_backward.py check the differentiation itself with the
rounding switched off (central finite differences) and closed forms.
"""

import numpy as np

from .l2norm import l2norm_bf16


def _norm(x, round_bf16):
    """x / sqrt(sum(x^2) + 1e-6) per row.  With round_bf16 the value is the
    canonical bf16 normalisation of the forward (l2norm_bf16) and the
    gradient is that of the unrounded expression."""
    import torch
    n = torch.sqrt((x * x).sum(-1, keepdim=True) + 1e-6)
    y = x / n
    if round_bf16:
        yr = torch.from_numpy(l2norm_bf16(x.detach().numpy().astype(np.float32)).astype(np.float64))
        y = y + (yr - y).detach()
    return y


def recurrent_backward(q, k, v, g, beta, initial_state, do, dht, cu_seqlens=None, round_bf16=True):
    """Shapes as recurrent.recurrent; do [B,T,HV,V]; dht [N,HV,K,V].

    Returns (dq, dk, dv, dg, dbeta, dh0) as float64 arrays; dh0 is None when
    initial_state is None.
    """
    import torch
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    q, k, v, g, beta = t(q), t(k), t(v), t(g), t(beta)
    s0 = None if initial_state is None else t(initial_state)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    group = HV // H
    scale = K ** -0.5
    qn = _norm(q, round_bf16).repeat_interleave(group, dim=2)
    kn = _norm(k, round_bf16).repeat_interleave(group, dim=2)
    if cu_seqlens is None:
        segs = [(b, 0, T) for b in range(B)]
    else:
        cu = [int(c) for c in np.asarray(cu_seqlens).tolist()]
        segs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    do = torch.from_numpy(np.asarray(do, dtype=np.float64))
    dht = torch.from_numpy(np.asarray(dht, dtype=np.float64))
    loss = torch.zeros((), dtype=torch.float64)
    for n, (b, t0, t1) in enumerate(segs):
        S = torch.zeros(HV, K, V, dtype=torch.float64) if s0 is None else s0[n]
        for tt in range(t0, t1):
            S = torch.exp(g[b, tt])[:, :, None] * S
            kt = kn[b, tt]
            r = v[b, tt] - torch.einsum("hk,hkv->hv", kt, S)
            S = S + beta[b, tt][:, None, None] * kt[:, :, None] * r[:, None, :]
            o = scale * torch.einsum("hk,hkv->hv", qn[b, tt], S)
            loss = loss + (o * do[b, tt]).sum()
        loss = loss + (S * dht[n]).sum()
    loss.backward()
    out = [x.grad.numpy() if x.grad is not None else np.zeros(x.shape) for x in (q, k, v, g, beta)]
    out.append(None if s0 is None else s0.grad.numpy())
    return tuple(out)
