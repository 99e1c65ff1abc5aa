"""A seeded sweep of small random configurations: shapes, GQA layouts,
packed variable-length batches (empty and one-token sequences included),
initial states present or absent.  Each prefill runs through
kda_chunk_prefill (whichever partition it picks), kda_chunk_prefill_split
and kda_chunk_prefill_fused, which must agree bit for bit, and is checked in
full against the oracle; each decode batch against the oracle's step."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_o, check_state, say

pytestmark = pytest.mark.gpu


def _prefill_case(seed):
    rng = np.random.default_rng(seed)
    H = int(rng.choice([1, 2, 3, 4]))
    HV = H * int(rng.choice([1, 2, 3, 5]))
    init = str(rng.choice(["none", "zero", "normal0.1"]))
    if rng.random() < 0.5:
        lens = rng.integers(0, 300, size=int(rng.integers(1, 7)))
        cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
        inp = synth.prefill_basic(1000 + seed, 1, int(cu[-1]), H, HV, init=init, cu_seqlens=cu,
                                  name=f"rand{seed}_varlen{len(lens)}")
    else:
        B = int(rng.integers(1, 4))
        T = int(rng.integers(1, 400))
        inp = synth.prefill_basic(1000 + seed, B, T, H, HV, init=init, name=f"rand{seed}")
    return inp


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill(gpu_lib, seed):
    kda = gpu_lib
    inp = _prefill_case(seed)
    dev = "cuda"
    a = [None if t is None else t.to(dev) for t in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.initial_state,
                                                     inp.cu_seqlens)]
    say(f"random prefill {inp.name} shape={inp.shape} init={'none' if inp.initial_state is None else 'given'}")
    oa, sa = kda.chunk_prefill(*a)
    osp, ssp = kda.chunk_prefill_split(*a)
    ofu, sfu = kda.chunk_prefill_fused(*a)
    torch.cuda.synchronize()
    for what, (o, s) in (("split", (osp, ssp)), ("fused", (ofu, sfu))):
        assert torch.equal(oa.view(torch.int16), o.view(torch.int16)), f"{inp.name}: o differs from {what}"
        assert torch.equal(sa, s), f"{inp.name}: state differs from {what}"
    n = synth.to_numpy(inp)
    o_ref, s_ref = oracle.recurrent(n["q"], n["k"], n["v"], n["g"], n["beta"], n["initial_state"], n["cu_seqlens"])
    eo = check_o(oa, o_ref, inp.name) if oa.numel() else 0.0
    es = check_state(sa, s_ref, inp.name)
    say(f"  o_err={eo:.2e} state_err={es:.2e}")


@pytest.mark.parametrize("seed", range(8))
def test_random_decode(gpu_lib, seed):
    rng = np.random.default_rng(500 + seed)
    H = int(rng.choice([1, 2, 4, 12]))
    HV = H * int(rng.choice([1, 2, 3]))
    B = int(rng.choice([1, 2, 3, 5, 7, 33, 100]))
    inp = synth.decode_config(B, N=B + int(rng.integers(0, 20)), H=H, HV=HV, seed=600 + seed)
    # a random extra share of inactive rows
    drop = torch.from_numpy(rng.random(B) < 0.2)
    inp.state_indices[drop] = -1
    dev = "cuda"
    say(f"random decode B={B} H={H} HV={HV} active={int((inp.state_indices >= 0).sum())}")
    pool = inp.pool.to(dev)
    before = pool.clone()
    o = gpu_lib.decode(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev), inp.beta.to(dev), pool,
                       inp.state_indices.to(dev))
    torch.cuda.synchronize()
    n = synth.to_numpy(inp)
    idx = n["state_indices"]
    N = n["pool"].shape[0]
    act = [int(i) for i in idx if 0 <= i < N]
    sub = n["pool"][act] if act else n["pool"][:0]
    remap = np.array([act.index(int(i)) if 0 <= i < N else -1 for i in idx], np.int32)
    o_ref, sub_new = oracle.decode_step(n["q"], n["k"], n["v"], n["g"], n["beta"], sub, remap)
    check_o(o[:, 0], o_ref, "random decode")
    og = o[:, 0].float().cpu().numpy()
    assert np.all(og[remap < 0] == 0)
    if act:
        got = pool.float().cpu().numpy()[act]
        assert np.all(np.abs(got - sub_new) <= np.abs(sub_new) * 2.0 ** -7 + 1e-6 * np.abs(sub_new).max())
    others = np.setdiff1d(np.arange(N), act)
    assert torch.equal(pool[torch.from_numpy(others).to(dev)], before[torch.from_numpy(others).to(dev)])
