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


@pytest.mark.parametrize("B", [1, 8, 32, 256])
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
