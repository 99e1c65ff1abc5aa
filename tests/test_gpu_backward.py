"""kda_chunk_backward on the GPU against the oracle's backward (float64
automatic differentiation of the token recurrence, oracle/backward.py).

Bars (float32 arithmetic throughout the GPU path; the float32 outputs are
compared):
  * elementwise, for every gradient tensor,
        |grad_gpu - grad_ref| <= 1e-4 * (|grad_ref| + rms(grad_ref)),
    rms taken over the tensor (per (sequence, head) for d_initial_state), so
    an error confined to a few tokens, channels or one head fails;
  * per tensor, ||grad_gpu - grad_ref||_F <= 1e-5 ||grad_ref||_F (per
    (sequence, head) for d_initial_state), reported beside it.
Cases cover several chunks with a ragged tail, GQA, varlen batches
(including an empty sequence and one shorter than a chunk), a missing
initial state and a missing final-state gradient, harsh gates and
beta = 0.  The bf16 outputs (the default, gradients in their inputs'
dtypes) are checked to be the nearest-even rounding of the float32 ones,
bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import say

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-5        # relative Frobenius, per tensor
ELEM_TOL = 1e-4         # elementwise, relative to |ref| + rms(ref)
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _rel(a, b):
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.abs(a).max(initial=0.0))


def _run(kda, inp, d_out, d_final, use_dht=True):
    say(f"backward {inp.name} shape={tuple(inp.q.shape)} HV={inp.v.shape[2]} "
        f"cu={None if inp.cu_seqlens is None else inp.cu_seqlens.tolist()} dht={use_dht}")
    dev = "cuda"
    s0 = None if inp.initial_state is None else inp.initial_state.to(dev)
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.to(dev)
    got = kda.chunk_backward(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev),
                             inp.beta.to(dev), s0, d_out.to(dev),
                             d_final.to(dev) if use_dht else None, cu_seqlens=cu, grad_dtype="float32",
                             want_d_initial_state=True)
    torch.cuda.synchronize()
    got = [None if x is None else x.cpu().numpy().astype(np.float64) for x in got]
    a = synth.to_numpy(inp)
    dht = d_final.numpy() if use_dht else np.zeros(d_final.shape)
    ref = oracle.recurrent_backward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["initial_state"],
                                    d_out.float().numpy(), dht, cu_seqlens=a["cu_seqlens"])
    return got, ref


def _elem(x, r):
    """max over elements of |x - r| / (|r| + rms(r)); 0 for an all-zero
    reference matched exactly, inf if it is not matched."""
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    if rms == 0.0:
        return 0.0 if np.all(x == 0) else float("inf")
    return float(np.max(np.abs(x - r) / (np.abs(r) + rms)))


def _check(got, ref, what):
    errs, elems = {}, {}
    for name, x, r in zip(NAMES, got, ref):
        if r is None:
            continue
        assert x is not None and np.all(np.isfinite(x)), f"{what}: {name} missing or non-finite"
        assert x.shape == r.shape, f"{what}: {name} shape {x.shape} vs {r.shape}"
        if name == "dh0":
            flat_x = x.reshape(-1, x.shape[-2] * x.shape[-1])
            flat_r = r.reshape(-1, r.shape[-2] * r.shape[-1])
            e = max(_rel(flat_x[i], flat_r[i]) for i in range(flat_r.shape[0]))
            el = max(_elem(flat_x[i], flat_r[i]) for i in range(flat_r.shape[0]))
        else:
            e = _rel(x, r)
            el = _elem(x, r)
        errs[name] = e
        elems[name] = el
    say(f"  {what}: frob " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    say(f"  {what}: elem " + " ".join(f"{k} {v:.2e}" for k, v in elems.items()))
    for name, e in errs.items():
        assert e <= GRAD_TOL, f"{what}: {name} rel-Frobenius {e:.3e} > {GRAD_TOL}"
    for name, e in elems.items():
        assert e <= ELEM_TOL, f"{what}: {name} elementwise {e:.3e} > {ELEM_TOL}"


CASES = [
    ("gqa_tail", dict(seed=30, B=1, T=150, H=1, HV=2, init="normal0.1")),
    ("batch_noinit", dict(seed=31, B=2, T=70, H=2, HV=2, init="none")),
    ("one_chunk", dict(seed=32, B=1, T=64, H=1, HV=1, init="normal0.1")),
    ("short", dict(seed=33, B=1, T=5, H=1, HV=1, init="normal0.1")),
    ("sixteen_chunks", dict(seed=34, B=1, T=1000, H=2, HV=4, init="normal0.1")),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_backward_vs_oracle(gpu_lib, name, kw):
    seed = kw.pop("seed")
    inp = synth.prefill_basic(seed, **kw, name=name)
    d_out, d_final = synth.upstream_grads(inp, seed + 100)
    got, ref = _run(gpu_lib, inp, d_out, d_final)
    _check(got, ref, name)


def test_backward_varlen(gpu_lib):
    cu = torch.tensor([0, 37, 37, 120, 200], dtype=torch.int32)
    inp = synth.prefill_basic(35, 1, 200, 1, 2, init="normal0.1", cu_seqlens=cu, name="varlen")
    d_out, d_final = synth.upstream_grads(inp, 135)
    got, ref = _run(gpu_lib, inp, d_out, d_final)
    _check(got, ref, "varlen")


def test_backward_no_final_grad(gpu_lib):
    inp = synth.prefill_basic(36, 1, 130, 1, 1, init="none", name="no_dht")
    d_out, d_final = synth.upstream_grads(inp, 136)
    got, ref = _run(gpu_lib, inp, d_out, d_final, use_dht=False)
    _check(got, ref, "no_dht")


def test_backward_harsh_gates(gpu_lib):
    inp = synth.config1()
    B, T = 1, 300
    inp = synth.PrefillInputs(inp.q[:B, :T, :2].contiguous(), inp.k[:B, :T, :2].contiguous(),
                              inp.v[:B, :T, :2].contiguous(), inp.g[:B, :T, :2].contiguous(),
                              inp.beta[:B, :T, :2].contiguous(), inp.initial_state[:B, :2].contiguous(),
                              None, "harsh")
    d_out, d_final = synth.upstream_grads(inp, 137)
    got, ref = _run(gpu_lib, inp, d_out, d_final)
    _check(got, ref, "harsh")


def test_backward_beta_zero(gpu_lib):
    inp = synth.prefill_basic(38, 1, 100, 1, 1, init="normal0.1", name="beta0")
    inp.beta.zero_()
    d_out, d_final = synth.upstream_grads(inp, 138)
    got, ref = _run(gpu_lib, inp, d_out, d_final)
    assert np.all(got[2] == 0), "beta = 0: v must get exactly zero gradient"
    _check(got, ref, "beta0")


def test_backward_full_size_sampled_head(gpu_lib):
    """The bench workload (B=1, H=HV=96, T=8192, zero initial state) in one
    call; heads are independent (H == HV), so one sampled head is checked
    against the oracle run on that head alone (37 s of CPU), and every
    output is checked to be finite."""
    inp = synth.config2()
    d_out, d_final = synth.upstream_grads(inp)
    say(f"backward full size {inp.name}")
    dev = "cuda"
    got = gpu_lib.chunk_backward(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev),
                                 inp.beta.to(dev), inp.initial_state.to(dev), d_out.to(dev),
                                 d_final.to(dev), grad_dtype="float32")
    torch.cuda.synchronize()
    for name, x in zip(NAMES, got):
        assert bool(torch.isfinite(x).all()), f"full size: {name} non-finite"
    h = 37
    sl = lambda t: t[:, :, h:h + 1].float().numpy()
    ref = oracle.recurrent_backward(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g), sl(inp.beta),
                                    inp.initial_state[:, h:h + 1].numpy(), sl(d_out),
                                    d_final[:, h:h + 1].numpy())
    mine = [x[:, :, h:h + 1] if x.dim() >= 3 and name != "dh0" else x[:, h:h + 1]
            for name, x in zip(NAMES, got)]
    mine = [x.cpu().numpy().astype(np.float64) for x in mine]
    _check(mine, ref, f"full size head {h}")


def test_backward_varlen_gqa_full_size_sampled(gpu_lib):
    """The 16-sequence varlen GQA batch (H=16, HV=32, about 37.5k tokens)
    in one call; the longest sequence's Q/K head 3 with its two value heads
    is checked against the oracle run on that sequence and head group."""
    inp = synth.config3()
    d_out, d_final = synth.upstream_grads(inp, 77)
    cu = inp.cu_seqlens
    say(f"backward full size {inp.name}")
    dev = "cuda"
    got = gpu_lib.chunk_backward(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev),
                                 inp.beta.to(dev), inp.initial_state.to(dev), d_out.to(dev),
                                 d_final.to(dev), cu_seqlens=cu.to(dev), grad_dtype="float32")
    torch.cuda.synchronize()
    for name, x in zip(NAMES, got):
        assert bool(torch.isfinite(x).all()), f"varlen full size: {name} non-finite"
    lens = (cu[1:] - cu[:-1]).tolist()
    n = int(np.argmax(lens))
    t0, t1 = int(cu[n]), int(cu[n + 1])
    h = 3
    hv0, hv1 = 2 * h, 2 * h + 2
    qk = lambda t: t[:, t0:t1, h:h + 1].float().numpy()
    vh = lambda t: t[:, t0:t1, hv0:hv1].float().numpy()
    ref = oracle.recurrent_backward(qk(inp.q), qk(inp.k), vh(inp.v), vh(inp.g), vh(inp.beta),
                                    inp.initial_state[n:n + 1, hv0:hv1].numpy(), vh(d_out),
                                    d_final[n:n + 1, hv0:hv1].numpy())
    dq, dk, dv, dg, db, dh0 = got
    mine = [dq[:, t0:t1, h:h + 1], dk[:, t0:t1, h:h + 1], dv[:, t0:t1, hv0:hv1], dg[:, t0:t1, hv0:hv1],
            db[:, t0:t1, hv0:hv1], dh0[n:n + 1, hv0:hv1]]
    mine = [x.cpu().numpy().astype(np.float64) for x in mine]
    _check(mine, ref, f"varlen full size sequence {n} ({t1 - t0} tokens) head {h}")


def test_backward_empty_sequence_axis(gpu_lib):
    """T = 0: nothing flows through the recurrence, so d_initial_state is
    d_final_state exactly and the token gradients are empty."""
    dev = "cuda"
    B, H, HV = 2, 1, 2
    inp = synth.prefill_basic(40, B, 0, H, HV, init="normal0.1", name="t0")
    d_out, d_final = synth.upstream_grads(inp, 140)
    got = gpu_lib.chunk_backward(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev),
                                 inp.beta.to(dev), inp.initial_state.to(dev), d_out.to(dev), d_final.to(dev),
                                 grad_dtype="float32")
    torch.cuda.synchronize()
    assert all(x.numel() == 0 for x in got[:5])
    assert torch.equal(got[5].cpu(), d_final)


def test_backward_deterministic_and_inputs_untouched(gpu_lib):
    """Two calls give bitwise equal gradients (no atomics: every sum has a
    fixed order) and leave every input unchanged."""
    dev = "cuda"
    inp = synth.prefill_basic(41, 1, 300, 2, 4, init="normal0.1", name="det")
    d_out, d_final = synth.upstream_grads(inp, 141)
    args = [t.to(dev) for t in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.initial_state, d_out, d_final)]
    before = [t.clone() for t in args]
    a = gpu_lib.chunk_backward(*args, grad_dtype="float32")
    b = gpu_lib.chunk_backward(*args, grad_dtype="float32")
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for x, y in zip(args, before):
        assert torch.equal(x, y)


def test_backward_input_dtypes_and_absent_state(gpu_lib):
    """The default output follows the page's contract: gradients in their
    inputs' dtypes (dq, dk, dv, dbeta bf16; dg float32) and None for an
    absent initial state.  The bf16 gradients are the nearest-even rounding
    of the float32 ones bit for bit (the same kernels; only the final store
    differs), on a GQA case (the separate normalisation kernel) and an
    H == HV case (the normalisation fused into the gradient kernel)."""
    dev = "cuda"
    for seed, H, HV in ((42, 1, 2), (43, 2, 2)):
        inp = synth.prefill_basic(seed, 1, 150, H, HV, init="none", name="dtypes")
        d_out, d_final = synth.upstream_grads(inp, seed + 100)
        args = [t.to(dev) for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
        lo = gpu_lib.chunk_backward(*args, None, d_out.to(dev), d_final.to(dev))
        hi = gpu_lib.chunk_backward(*args, None, d_out.to(dev), d_final.to(dev), grad_dtype="float32")
        torch.cuda.synchronize()
        assert lo[5] is None and hi[5] is None
        for i, name in enumerate(NAMES[:5]):
            want = torch.bfloat16 if name != "dg" else torch.float32
            assert lo[i].dtype == want, (name, lo[i].dtype)
            ref = hi[i].to(torch.bfloat16) if name != "dg" else hi[i]
            assert torch.equal(lo[i].view(torch.int16) if name != "dg" else lo[i],
                               ref.view(torch.int16) if name != "dg" else ref), name
        # asking for the zero-state gradient still works without an initial state
        z = gpu_lib.chunk_backward(*args, None, d_out.to(dev), d_final.to(dev), grad_dtype="float32",
                                   want_d_initial_state=True)
        torch.cuda.synchronize()
        assert z[5] is not None and z[5].dtype == torch.float32
