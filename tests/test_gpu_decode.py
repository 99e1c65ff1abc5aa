"""kda_decode on the GPU against the oracle's decode step (fp64):
output within the parity bar, written slots within one bf16 step of the
oracle's rounded state, every other slot and every inactive row untouched."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_o, say

pytestmark = pytest.mark.gpu


def _run(kda, inp, pool_stride_pad=0):
    B = inp.q.shape[0]
    N, HV, K, V = inp.pool.shape
    if pool_stride_pad:
        store = torch.zeros(N, HV * K * V + pool_stride_pad, dtype=torch.bfloat16, device="cuda")
        store[:, : HV * K * V] = inp.pool.reshape(N, -1).cuda()
        pool = torch.as_strided(store, (N, HV, K, V), (HV * K * V + pool_stride_pad, K * V, V, 1))
    else:
        pool = inp.pool.cuda()
    before = pool.clone()
    o = kda.decode(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.g.cuda(), inp.beta.cuda(),
                   pool, inp.state_indices.cuda())
    torch.cuda.synchronize()
    return o, pool, before


def _check(kda, inp, pad=0):
    say(f"decode {inp.name} pad={pad}")
    o, pool, before = _run(kda, inp, pad)
    a = synth.to_numpy(inp)
    idx = a["state_indices"]
    N = a["pool"].shape[0]
    act = [int(i) for i in idx if 0 <= i < N]
    # oracle on the referenced slots only (sub-pool with remapped indices)
    sub = a["pool"][act] if act else a["pool"][:0]
    remap = np.array([act.index(int(i)) if 0 <= i < N else -1 for i in idx], np.int32)
    o_ref, sub_new = oracle.decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], sub, remap)
    check_o(o[:, 0], o_ref, inp.name)
    og = o[:, 0].float().cpu().numpy()
    for b, i in enumerate(idx):
        if not (0 <= i < N):
            assert np.all(og[b] == 0), f"inactive row {b} not zero"
    got = pool.float().cpu().numpy()
    if act:
        ref = sub_new
        g = got[act]
        ulp = np.abs(ref) * 2.0 ** -7
        err = np.abs(g - ref)
        assert np.all(err <= ulp + 1e-6 * np.abs(ref).max()), "state differs by more than one bf16 step"
        assert np.count_nonzero(g != ref) <= 1e-3 * g.size + 1
    others = np.setdiff1d(np.arange(N), act)
    assert torch.equal(pool[torch.from_numpy(others).cuda()], before[torch.from_numpy(others).cuda()])


@pytest.mark.parametrize("B", [1, 4, 8, 32, 256])
def test_decode_workload(gpu_lib, B):
    _check(gpu_lib, synth.decode_config(B))


def test_decode_padded_slot_stride(gpu_lib):
    _check(gpu_lib, synth.decode_config(32, N=64), pad=136)


def test_decode_gqa_and_all_inactive(gpu_lib):
    inp = synth.decode_config(16, N=40, H=4, HV=12)
    _check(gpu_lib, inp)
    one = synth.decode_config(1, N=8)
    one.state_indices[:] = -1
    _check(gpu_lib, one)


def test_decode_out_of_range_index_is_inactive(gpu_lib):
    inp = synth.decode_config(8, N=16)
    inp.state_indices[2] = 16        # == num_slots: treated as inactive, no access
    inp.state_indices[3] = -7
    _check(gpu_lib, inp)


def test_decode_deterministic(gpu_lib):
    inp = synth.decode_config(32, N=64)
    o1, p1, _ = _run(gpu_lib, inp)
    o2, p2, _ = _run(gpu_lib, inp)
    assert torch.equal(o1, o2) and torch.equal(p1, p2)


def test_decode_batch_invariant(gpu_lib):
    """Small batches (4 B HV at most the compute units: B <= 5 at 12 value
    heads on MI355X) run the column-quarter kernel, larger ones the row
    kernel; both take the same arithmetic in the same order, so a row's
    output and its new state must not depend on the batch it is decoded in:
    rows of a 256-row batch decoded alone and in batches of 5, 6, 31 and 32
    rows give the same bits."""
    inp = synth.decode_config(256, N=1024, seed=12)
    dev = "cuda"
    a = [t.to(dev) for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
    idx = inp.state_indices.to(dev)
    pool_full = inp.pool.to(dev)
    o_full = gpu_lib.decode(*a, pool_full, idx)
    torch.cuda.synchronize()
    for lo, hi in ((0, 31), (31, 63), (100, 101), (255, 256), (7, 8), (40, 45), (50, 56)):
        say(f"decode rows {lo}..{hi - 1} alone (B={hi - lo})")
        pool = inp.pool.to(dev)
        o = gpu_lib.decode(*(t[lo:hi] for t in a), pool, idx[lo:hi])
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_full[lo:hi].view(torch.int16)), f"rows {lo}..{hi}: o differs"
        act = idx[lo:hi][idx[lo:hi] >= 0].long()
        assert torch.equal(pool[act].view(torch.int16), pool_full[act].view(torch.int16)), \
            f"rows {lo}..{hi}: state differs"


def test_decode_max_batch(gpu_lib):
    """The largest batch kda_decode accepts (B = 65535, the launch grid's
    limit), one head, a 2 GiB pool generated on the device: 256 sampled rows
    against the oracle, their inactive rows zero, and every slot no row
    addresses left untouched."""
    B, N = 65535, 65535 + 17
    dev = "cuda"
    gen = torch.Generator().manual_seed(30)
    q = torch.randn(B, 1, 128, generator=gen).to(torch.bfloat16)
    k = torch.randn(B, 1, 128, generator=gen).to(torch.bfloat16)
    v = torch.randn(B, 1, 128, generator=gen).to(torch.bfloat16)
    g = torch.nn.functional.logsigmoid(torch.randn(B, 1, 128, generator=gen) + 3.0)
    beta = torch.sigmoid(torch.randn(B, 1, generator=gen)).to(torch.bfloat16)
    idx = torch.randperm(N, generator=gen)[:B].to(torch.int32)
    idx[torch.arange(B) % 8 == 7] = -1
    dgen = torch.Generator(device=dev).manual_seed(31)
    pool = (0.1 * torch.randn(N, 1, 128, 128, generator=dgen, device=dev)).to(torch.bfloat16)
    rows = torch.randperm(B, generator=gen)[:256].sort().values
    used = torch.zeros(N, dtype=torch.bool)
    used[idx[idx >= 0].long()] = True
    free_slots = torch.nonzero(~used).flatten().to(dev)
    act = [int(r) for r in rows if idx[r] >= 0]
    before_rows = pool[idx[act].long().to(dev)].float().cpu().numpy()
    before_free = pool[free_slots].clone()
    say(f"decode B={B}: {len(act)} sampled active rows, {free_slots.numel()} unaddressed slots")
    o = gpu_lib.decode(q.to(dev), k.to(dev), v.to(dev), g.to(dev), beta.to(dev), pool, idx.to(dev))
    torch.cuda.synchronize()
    sub = lambda t: t[rows].float().numpy()
    remap = np.array([act.index(int(r)) if idx[r] >= 0 else -1 for r in rows], np.int32)
    o_ref, new_ref = oracle.decode_step(sub(q), sub(k), sub(v), sub(g), sub(beta), before_rows, remap)
    check_o(o[rows.to(dev), 0], o_ref, "decode max batch")
    og = o[rows.to(dev), 0].float().cpu().numpy()
    assert np.all(og[remap < 0] == 0), "inactive rows not zero"
    got = pool[idx[act].long().to(dev)].float().cpu().numpy()
    assert np.all(np.abs(got - new_ref) <= np.abs(new_ref) * 2.0 ** -7 + 1e-6 * np.abs(new_ref).max())
    assert torch.equal(pool[free_slots], before_free), "an unaddressed slot changed"


@pytest.mark.parametrize("B,H,HV", [(3, 1, 12), (50, 4, 20), (2, 5, 5)], ids=["group12", "group5", "odd"])
def test_decode_head_layouts(gpu_lib, B, H, HV):
    """GQA groups and odd head counts on both decode kernels (B=3 and B=2
    take the column-quarter kernel, B=50 the row kernel)."""
    _check(gpu_lib, synth.decode_config(B, N=3 * B + 5, H=H, HV=HV, seed=50 + HV))
