"""Seeded synthetic inputs for the KDA forward path.

Shared by the tests, the benchmark and the oracle checks.  This module only
draws random numbers and shapes them into the input tensors; it holds none
of the method's arithmetic (no normalisation, no recurrence, no chunk math).

Distributions follow the input generator described on "KDA Chunk Prefill on
Ascend A3" (section "Public examples and full evaluation"): normal q/k with
optional per-row gains exp(0.6 N), tiny and zero-row modes, standard-normal
v, gates logsigmoid(N)/divisor, beta = sigmoid(N) with edge modes, and
states 0.25 N / zero / None.  The named workloads below are the fixed
synthetic configurations this repository is measured and checked on.

All draws use a CPU ``torch.Generator`` seeded per workload, in the order
q, k, v, g, beta, initial_state, extras.  bf16 tensors come from float32
draws rounded to nearest-even by ``Tensor.to(torch.bfloat16)``.
"""

import math
from dataclasses import dataclass
from typing import Optional

import torch
import torch.nn.functional as F

K_DIM = 128
V_DIM = 128


@dataclass
class PrefillInputs:
    q: torch.Tensor            # [B,T,H,K] bf16
    k: torch.Tensor            # [B,T,H,K] bf16
    v: torch.Tensor            # [B,T,HV,V] bf16
    g: torch.Tensor            # [B,T,HV,K] fp32
    beta: torch.Tensor         # [B,T,HV] bf16
    initial_state: Optional[torch.Tensor]   # [N,HV,K,V] fp32 or None
    cu_seqlens: Optional[torch.Tensor]      # [N+1] int32 or None
    name: str = ""

    @property
    def shape(self):
        B, T, H, K = self.q.shape
        return B, T, H, self.v.shape[2], K, self.v.shape[3]

    def num_seqs(self):
        if self.cu_seqlens is not None:
            return self.cu_seqlens.numel() - 1
        return self.q.shape[0]


@dataclass
class DecodeInputs:
    q: torch.Tensor            # [B,H,K] bf16
    k: torch.Tensor            # [B,H,K] bf16
    v: torch.Tensor            # [B,HV,V] bf16
    g: torch.Tensor            # [B,HV,K] fp32
    beta: torch.Tensor         # [B,HV] bf16
    pool: torch.Tensor         # [N,HV,K,V] bf16
    state_indices: torch.Tensor  # [B] int32
    name: str = ""


def _gen(seed):
    return torch.Generator().manual_seed(seed)


def _randn(gen, *shape):
    return torch.randn(*shape, generator=gen, dtype=torch.float32)


def _logsig_gate(gen, shape, mean=3.0):
    """g = log(sigmoid(x)) with x ~ N(mean, 1), fp32."""
    return F.logsigmoid(_randn(gen, *shape) + mean)


def prefill_basic(seed, B, T, H, HV, *, init="none", cu_seqlens=None, name=""):
    """q,k,v ~ N(0,1) bf16; g = logsigmoid(N(3,1)) fp32; beta = sigmoid(N(0,1))
    bf16.  init: 'none' | 'zero' | 'normal0.1' (fp32 0.1*N(0,1))."""
    gen = _gen(seed)
    q = _randn(gen, B, T, H, K_DIM).to(torch.bfloat16)
    k = _randn(gen, B, T, H, K_DIM).to(torch.bfloat16)
    v = _randn(gen, B, T, HV, V_DIM).to(torch.bfloat16)
    g = _logsig_gate(gen, (B, T, HV, K_DIM))
    beta = torch.sigmoid(_randn(gen, B, T, HV)).to(torch.bfloat16)
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if init == "none":
        s0 = None
    elif init == "zero":
        s0 = torch.zeros(N, HV, K_DIM, V_DIM, dtype=torch.float32)
    elif init == "normal0.1":
        s0 = 0.1 * _randn(gen, N, HV, K_DIM, V_DIM)
    else:
        raise ValueError(init)
    return PrefillInputs(q, k, v, g, beta, s0, cu_seqlens, name)


# --------------------------------------------------------------------------
# Named workloads


def config0():
    """Single chunk pair: B=1, H=HV=1, T=128, K=V=128, no initial state."""
    return prefill_basic(0, 1, 128, 1, 1, init="none", name="cfg0_b1_h1_t128")


def config1():
    """B=2, H=HV=8, T=1000 (15 full chunks of 64 plus a 40-token tail), harsh
    decay: g clamped at >= -5 with 10% of (b, hv, k) channels pinned to -5 for
    every token; initial state fp32 0.1*N(0,1)."""
    B, T, H, HV = 2, 1000, 8, 8
    gen = _gen(1)
    q = _randn(gen, B, T, H, K_DIM).to(torch.bfloat16)
    k = _randn(gen, B, T, H, K_DIM).to(torch.bfloat16)
    v = _randn(gen, B, T, HV, V_DIM).to(torch.bfloat16)
    g = _logsig_gate(gen, (B, T, HV, K_DIM)).clamp_min(-5.0)
    beta = torch.sigmoid(_randn(gen, B, T, HV)).to(torch.bfloat16)
    s0 = 0.1 * _randn(gen, B, HV, K_DIM, V_DIM)
    nch = B * HV * K_DIM
    pick = torch.randperm(nch, generator=gen)[: math.ceil(0.1 * nch)]
    gflat = g.permute(0, 2, 3, 1).reshape(nch, T)     # (b, hv, k) x t
    gflat[pick] = -5.0
    g = gflat.reshape(B, HV, K_DIM, T).permute(0, 3, 1, 2).contiguous()
    return PrefillInputs(q, k, v, g, beta, s0, None, "cfg1_b2_h8_t1000_harsh")


def config2(T=8192, H=96):
    """At scale: B=1, H=HV=96, T=8192; explicit zero fp32 initial state."""
    return prefill_basic(2, 1, T, H, H, init="zero", name=f"cfg2_b1_h{H}_t{T}")


def config3_lengths(num=16, max_len=4096, seed=3):
    gen = _gen(seed)
    lens = torch.randint(1, max_len + 1, (num,), generator=gen)
    return lens


def config3(num=16, max_len=4096):
    """Packed variable-length batch: 16 sequences with lengths ~U[1,4096],
    GQA with H=16 Q/K heads and HV=32 value heads; per-sequence fp32 initial
    states 0.1*N(0,1)."""
    lens = config3_lengths(num, max_len)
    cu = torch.zeros(num + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    T = int(cu[-1])
    inp = prefill_basic(33, 1, T, 16, 32, init="normal0.1", cu_seqlens=cu,
                        name=f"cfg3_varlen{num}_t{T}_h16_hv32")
    return inp


def decode_config(B, N=1024, H=12, HV=12, seed=4):
    """Single-token decode: q,k,v,g,beta as the prefill draws with T=1; bf16
    pool 0.1*N(0,1) [N,HV,K,V]; unique slots from a permutation with rows
    r % 8 == 7 set to -1."""
    gen = _gen(seed * 1000 + B)
    q = _randn(gen, B, H, K_DIM).to(torch.bfloat16)
    k = _randn(gen, B, H, K_DIM).to(torch.bfloat16)
    v = _randn(gen, B, HV, V_DIM).to(torch.bfloat16)
    g = _logsig_gate(gen, (B, HV, K_DIM))
    beta = torch.sigmoid(_randn(gen, B, HV)).to(torch.bfloat16)
    pool = (0.1 * _randn(gen, N, HV, K_DIM, V_DIM)).to(torch.bfloat16)
    idx = torch.randperm(N, generator=gen)[:B].to(torch.int32)
    rows = torch.arange(B)
    idx[rows % 8 == 7] = -1
    return DecodeInputs(q, k, v, g, beta, pool, idx, f"decode_b{B}_h{HV}")


@dataclass
class PackedDecodeInputs:
    mixed_qkv: torch.Tensor    # [B, 3*H*K + row_pad] bf16 (rows q | k | v, then padding)
    raw_gate: torch.Tensor     # [B, H*K] bf16
    raw_beta: torch.Tensor     # [B, H] bf16
    A_log: torch.Tensor        # [H] fp32
    dt_bias: torch.Tensor      # [H*K] fp32
    pool: torch.Tensor         # [N,H,K,V] bf16
    state_indices: torch.Tensor  # [B] int32
    H: int
    name: str = ""


def packed_decode_config(B, N=1024, H=12, row_pad=0, seed=7):
    """Packed decode inputs: q,k,v ~ N(0,1) packed in one bf16 row per batch
    row (row_pad trailing elements of each row hold NaN, which must never be
    read); raw gate and beta logits ~ N(0,1) bf16; A_log = log U(1,16) per
    head and dt_bias ~ N(0,1) per channel (fp32); bf16 pool 0.1*N(0,1);
    unique slots from a permutation with rows r % 8 == 7 set to -1."""
    gen = _gen(seed * 1000 + B)
    qkv = _randn(gen, B, 3 * H * K_DIM)
    mixed = torch.full((B, 3 * H * K_DIM + row_pad), float("nan"))
    mixed[:, : 3 * H * K_DIM] = qkv
    raw_gate = _randn(gen, B, H * K_DIM).to(torch.bfloat16)
    raw_beta = _randn(gen, B, H).to(torch.bfloat16)
    A_log = torch.log(1.0 + 15.0 * torch.rand(H, generator=gen))
    dt_bias = _randn(gen, H * K_DIM)
    pool = (0.1 * _randn(gen, N, H, K_DIM, V_DIM)).to(torch.bfloat16)
    idx = torch.randperm(N, generator=gen)[:B].to(torch.int32)
    idx[torch.arange(B) % 8 == 7] = -1
    return PackedDecodeInputs(mixed.to(torch.bfloat16), raw_gate, raw_beta, A_log, dt_bias, pool, idx, H,
                              f"packed_decode_b{B}_h{H}_pad{row_pad}")


def handoff_config(N, slots=1024, HV=12, seed=6):
    """Prefill-to-decode handoff: N fp32 states 0.25*N(0,1) [N,HV,K,V] (the
    pages' nonzero state), a bf16 pool 0.1*N(0,1) [slots,HV,K,V] and unique
    slots from a permutation with rows r % 8 == 7 set to -1."""
    gen = _gen(seed * 1000 + N)
    state = 0.25 * _randn(gen, N, HV, K_DIM, V_DIM)
    pool = (0.1 * _randn(gen, slots, HV, K_DIM, V_DIM)).to(torch.bfloat16)
    idx = torch.randperm(slots, generator=gen)[:N].to(torch.int32)
    idx[torch.arange(N) % 8 == 7] = -1
    return state, pool, idx


def worked_example(T=128, beta_value=1.0):
    """The pages' worked example: B=H=HV=1, K=V=128, q=k=e0, v=1, g=0,
    beta=1 (or beta_value), no initial state."""
    q = torch.zeros(1, T, 1, K_DIM)
    q[..., 0] = 1.0
    k = q.clone()
    v = torch.ones(1, T, 1, V_DIM)
    g = torch.zeros(1, T, 1, K_DIM)
    beta = torch.full((1, T, 1), beta_value)
    return PrefillInputs(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16),
                         g, beta.to(torch.bfloat16), None, None, f"worked_example_beta{beta_value}")


# --------------------------------------------------------------------------
# Stress modes (the page's generator, shapes chosen by the caller)


def prefill_stress(seed, B, T, H, HV, *, qk_mode="gain", gate="moderate",
                   beta_mode="sigmoid", state="normal"):
    """qk_mode: 'gain' | 'tiny' | 'zero_rows'; gate: 'weak' | 'moderate' |
    'strong' | 'zero'; beta_mode: 'sigmoid' | 'zero' | 'one' | 'edge';
    state: 'normal' | 'zero' | 'none'."""
    gen = _gen(seed)
    gq = torch.exp(_randn(gen, B, T, H, 1) * 0.6)
    q = gq * _randn(gen, B, T, H, K_DIM)
    gk = torch.exp(_randn(gen, B, T, H, 1) * 0.6)
    k = gk * _randn(gen, B, T, H, K_DIM)
    q = q.to(torch.bfloat16)
    k = k.to(torch.bfloat16)
    if qk_mode == "tiny":
        q = (q.float() * 1e-5).to(torch.bfloat16)
        k = (k.float() * 1e-5).to(torch.bfloat16)
    elif qk_mode == "zero_rows":
        q[:, ::3] = 0
        k[:, 1::3] = 0
    elif qk_mode != "gain":
        raise ValueError(qk_mode)
    v = _randn(gen, B, T, HV, V_DIM).to(torch.bfloat16)
    div = {"weak": 128.0, "moderate": 8.0, "strong": 1.0}
    if gate == "zero":
        g = torch.zeros(B, T, HV, K_DIM)
    else:
        g = F.logsigmoid(_randn(gen, B, T, HV, K_DIM)) / div[gate]
    beta = torch.sigmoid(_randn(gen, B, T, HV))
    if beta_mode == "zero":
        beta = torch.zeros_like(beta)
    elif beta_mode == "one":
        beta = torch.ones_like(beta)
    elif beta_mode == "edge":
        edge = torch.tensor([0.0, 1.0, 1e-4, 1.0 - 1e-4])
        beta = edge[torch.arange(T) % 4].view(1, T, 1).expand(B, T, HV).clone()
    elif beta_mode != "sigmoid":
        raise ValueError(beta_mode)
    beta = beta.to(torch.bfloat16)
    if state == "normal":
        s0 = 0.25 * _randn(gen, B, HV, K_DIM, V_DIM)
    elif state == "zero":
        s0 = torch.zeros(B, HV, K_DIM, V_DIM)
    elif state == "none":
        s0 = None
    else:
        raise ValueError(state)
    return PrefillInputs(q, k, v, g, beta, s0, None,
                         f"stress_{qk_mode}_{gate}_{beta_mode}_{state}")


def upstream_grads(inp, seed=11):
    """Upstream gradients for a backward call on a prefill workload: d_out
    ~ N(0,1) as bf16 [B,T,HV,V] (the dtype of o) and d_final_state ~ N(0,1)
    fp32 [N,HV,K,V]."""
    gen = _gen(seed)
    B, T, HV = inp.v.shape[0], inp.v.shape[1], inp.v.shape[2]
    N = B if inp.cu_seqlens is None else inp.cu_seqlens.numel() - 1
    d_out = _randn(gen, B, T, HV, V_DIM).to(torch.bfloat16)
    d_final = _randn(gen, N, HV, K_DIM, V_DIM)
    return d_out, d_final


def to_numpy(inp):
    """float32 numpy copies of every tensor field (bf16 values are exact)."""
    out = {}
    for name in ("q", "k", "v", "g", "beta"):
        out[name] = getattr(inp, name).float().numpy()
    s0 = inp.initial_state if isinstance(inp, PrefillInputs) else None
    out["initial_state"] = None if s0 is None else s0.float().numpy()
    if isinstance(inp, PrefillInputs):
        out["cu_seqlens"] = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    else:
        out["pool"] = inp.pool.float().numpy()
        out["state_indices"] = inp.state_indices.numpy()
    return out
