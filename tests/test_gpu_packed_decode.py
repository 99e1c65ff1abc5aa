"""kda_packed_decode on the GPU against the oracle's packed decode step
(fp64): output within the parity bar, written slots within one bf16 step of
the oracle's rounded state, every other slot and every inactive row
untouched; row padding (filled with NaN) never read.  At the point where the
gate and beta transforms have closed forms the packed path must equal
kda_decode bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_o, say

pytestmark = pytest.mark.gpu


def _run(kda, inp, pool_stride_pad=0):
    N, H, K, V = inp.pool.shape
    if pool_stride_pad:
        store = torch.zeros(N, H * K * V + pool_stride_pad, dtype=torch.bfloat16, device="cuda")
        store[:, : H * K * V] = inp.pool.reshape(N, -1).cuda()
        pool = torch.as_strided(store, (N, H, K, V), (H * K * V + pool_stride_pad, K * V, V, 1))
    else:
        pool = inp.pool.cuda()
    before = pool.clone()
    m = inp.mixed_qkv.cuda()
    qkv = m[:, : 3 * H * K]          # a view: rows keep the padded stride
    o = kda.packed_decode(qkv, inp.raw_gate.cuda(), inp.raw_beta.cuda(), inp.A_log.cuda(), inp.dt_bias.cuda(),
                          pool, inp.state_indices.cuda())
    torch.cuda.synchronize()
    return o, pool, before


def _check(kda, inp, pad=0):
    say(f"packed decode {inp.name} pool pad={pad}")
    o, pool, before = _run(kda, inp, pad)
    idx = inp.state_indices.numpy()
    N = inp.pool.shape[0]
    act = [int(i) for i in idx if 0 <= i < N]
    pool_np = inp.pool.float().numpy()
    sub = pool_np[act] if act else pool_np[:0]
    remap = np.array([act.index(int(i)) if 0 <= i < N else -1 for i in idx], np.int32)
    o_ref, sub_new = oracle.packed_decode_step(inp.mixed_qkv.float().numpy(), inp.raw_gate.float().numpy(),
                                               inp.raw_beta.float().numpy(), inp.A_log.numpy(),
                                               inp.dt_bias.numpy(), sub, remap)
    check_o(o[:, 0], o_ref, inp.name)
    og = o[:, 0].float().cpu().numpy()
    for b, i in enumerate(idx):
        if not (0 <= i < N):
            assert np.all(og[b] == 0), f"inactive row {b} not zero"
    got = pool.float().cpu().numpy()
    if act:
        g = got[act]
        ulp = np.abs(sub_new) * 2.0 ** -7
        assert np.all(np.abs(g - sub_new) <= ulp + 1e-6 * np.abs(sub_new).max()), "state off by more than one bf16 step"
        assert np.count_nonzero(g != sub_new) <= 1e-3 * g.size + 1
    others = np.setdiff1d(np.arange(N), act)
    assert torch.equal(pool[torch.from_numpy(others).cuda()], before[torch.from_numpy(others).cuda()])


@pytest.mark.parametrize("B", [1, 4, 8, 32, 256])
def test_packed_decode_workload(gpu_lib, B):
    _check(gpu_lib, synth.packed_decode_config(B))


def test_packed_decode_padded_rows_and_slots(gpu_lib):
    _check(gpu_lib, synth.packed_decode_config(32, N=64, row_pad=24), pad=136)


def test_packed_decode_other_head_counts_and_index_edges(gpu_lib):
    inp = synth.packed_decode_config(16, N=40, H=4, row_pad=8)
    inp.state_indices[2] = 40        # == num_slots: inactive, no access
    inp.state_indices[3] = -9
    _check(gpu_lib, inp)


def test_packed_equals_split_decode_at_closed_form_point(gpu_lib):
    """raw_gate = -dt_bias and raw_beta = 0 make g = -2.5 and beta = 1/2
    exactly, so the packed path and kda_decode on the extracted q, k, v must
    agree bit for bit, output and pool."""
    inp = synth.packed_decode_config(24, N=48, H=12, row_pad=16)
    say("packed vs split decode at g=-2.5, beta=1/2")
    H, K = 12, 128
    raw_gate = inp.raw_gate
    dt_bias = -raw_gate[0].float()                     # exact: bf16 values are fp32 values
    raw_gate = raw_gate[0:1].expand(24, -1).contiguous()
    raw_beta = torch.zeros(24, H, dtype=torch.bfloat16)
    m = inp.mixed_qkv.cuda()
    pool_a = inp.pool.cuda()
    pool_b = pool_a.clone()
    idx = inp.state_indices.cuda()
    oa = gpu_lib.packed_decode(m[:, : 3 * H * K], raw_gate.cuda(), raw_beta.cuda(), inp.A_log.cuda(),
                               dt_bias.cuda(), pool_a, idx)
    q = m[:, : H * K].reshape(24, H, K).contiguous()
    k = m[:, H * K: 2 * H * K].reshape(24, H, K).contiguous()
    v = m[:, 2 * H * K: 3 * H * K].reshape(24, H, K).contiguous()
    g = torch.full((24, H, K), -2.5, device="cuda")
    beta = torch.full((24, H), 0.5, dtype=torch.bfloat16, device="cuda")
    ob = gpu_lib.decode(q, k, v, g, beta, pool_b, idx)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
    assert torch.equal(pool_a.view(torch.int16), pool_b.view(torch.int16))


def test_packed_decode_batch_invariant(gpu_lib):
    """As for kda_decode: the small-batch and the large-batch kernel give the
    same bits, so rows of a 256-row batch decoded alone or in 5-, 6-, 31-
    and 32-row batches equal the full batch's rows."""
    inp = synth.packed_decode_config(256, row_pad=24)
    dev = "cuda"
    H, K = inp.H, 128
    qkv = inp.mixed_qkv.to(dev)[:, : 3 * H * K]
    a = [t.to(dev) for t in (inp.raw_gate, inp.raw_beta)]
    A_log, dt_bias = inp.A_log.to(dev), inp.dt_bias.to(dev)
    idx = inp.state_indices.to(dev)
    pool_full = inp.pool.to(dev)
    o_full = gpu_lib.packed_decode(qkv, *a, A_log, dt_bias, pool_full, idx)
    torch.cuda.synchronize()
    for lo, hi in ((0, 31), (31, 63), (200, 201), (10, 15), (20, 26)):
        say(f"packed decode rows {lo}..{hi - 1} alone (B={hi - lo})")
        pool = inp.pool.to(dev)
        o = gpu_lib.packed_decode(qkv[lo:hi], *(t[lo:hi] for t in a), A_log, dt_bias, pool, idx[lo:hi])
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_full[lo:hi].view(torch.int16)), f"rows {lo}..{hi}: o differs"
        act = idx[lo:hi][idx[lo:hi] >= 0].long()
        assert torch.equal(pool[act].view(torch.int16), pool_full[act].view(torch.int16)), \
            f"rows {lo}..{hi}: state differs"
