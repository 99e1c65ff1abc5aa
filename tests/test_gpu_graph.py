"""The library under HIP graph capture: kda_decode (the page's -1 rows are
"graph padding", so the decode is meant to be captured) and
kda_chunk_prefill with a caller-owned workspace (in both of the forms it
picks between: split at a few units, fused at 256) are captured once, then
replayed on new inputs copied into the captured buffers; every replay must
equal a direct call on the same inputs bit for bit.  Eager work and host
synchronisations run between the replays.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_decode_graph_replay(gpu_lib):
    kda = gpu_lib
    dev = "cuda"
    B = 32
    base = synth.decode_config(B, N=64, seed=40)
    static = {n: getattr(base, n).to(dev) for n in ("q", "k", "v", "g", "beta", "state_indices")}
    pool0 = base.pool.to(dev)
    pool = pool0.clone()
    out = torch.empty((B, 1, 12, 128), dtype=torch.bfloat16, device=dev)
    args = lambda d, p: (d["q"], d["k"], d["v"], d["g"], d["beta"], p, d["state_indices"])
    kda.decode(*args(static, pool), out=out)          # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.decode(*args(static, pool), out=out)
    torch.cuda.synchronize()
    for r in range(4):
        nxt = synth.decode_config(B, N=64, seed=41 + r)
        for n in static:
            static[n].copy_(getattr(nxt, n).to(dev))
        pool.copy_(pool0)
        graph.replay()
        torch.cuda.synchronize()
        ref_pool = pool0.clone()
        ref_out = kda.decode(*args(static, ref_pool))
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref_out)), f"replay {r}: o differs"
        assert torch.equal(_bits(pool), _bits(ref_pool)), f"replay {r}: pool differs"
        say(f"decode graph replay {r}: identical to the direct call")


@pytest.mark.parametrize("B,T,H,HV", [(1, 300, 2, 4), (4, 300, 16, 64)], ids=["split", "fused"])
def test_prefill_graph_replay(gpu_lib, B, T, H, HV):
    kda = gpu_lib
    dev = "cuda"
    assert kda.prefill_partition(B, HV) == ("split" if B * HV < 192 else "fused")
    first = synth.prefill_basic(50, B, T, H, HV, init="normal0.1")
    names = ("q", "k", "v", "g", "beta", "initial_state")
    static = {n: getattr(first, n).to(dev) for n in names}
    ws = torch.empty(kda.workspace_size(B, T, H, HV), dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, HV, 128), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((B, HV, 128, 128), dtype=torch.float32, device=dev)
    call = lambda d, **kw: kda.chunk_prefill(*(d[n] for n in names), **kw)
    call(static, out=out, final_state=fin, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static, out=out, final_state=fin, workspace=ws)
    torch.cuda.synchronize()
    for r in range(4):
        nxt = synth.prefill_basic(51 + r, B, T, H, HV, init="normal0.1")
        for n in names:
            static[n].copy_(getattr(nxt, n).to(dev))
        graph.replay()
        torch.cuda.synchronize()
        ref_o, ref_s = call(static)                        # its own workspace and outputs
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref_o)), f"replay {r}: o differs"
        assert torch.equal(fin, ref_s), f"replay {r}: final state differs"
        say(f"prefill graph replay {r}: identical to the direct call")


@pytest.mark.parametrize("B,T,H,HV", [(1, 700, 2, 4), (4, 300, 16, 64)], ids=["split", "fused"])
def test_prefill_noalloc_graph_replay(gpu_lib, B, T, H, HV):
    """The allocation-free prefill (its workspace a static device array, so
    nothing is allocated inside the capture), captured once and replayed on
    new inputs: every replay equals a direct call bit for bit."""
    kda = gpu_lib
    dev = "cuda"
    first = synth.prefill_basic(60, B, T, H, HV, init="normal0.1")
    names = ("q", "k", "v", "g", "beta", "initial_state")
    static = {n: getattr(first, n).to(dev) for n in names}
    out = torch.empty((B, T, HV, 128), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((B, HV, 128, 128), dtype=torch.float32, device=dev)
    kda.chunk_prefill_noalloc(*(static[n] for n in names), out=out, final_state=fin)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.chunk_prefill_noalloc(*(static[n] for n in names), out=out, final_state=fin)
    torch.cuda.synchronize()
    for r in range(4):
        nxt = synth.prefill_basic(61 + r, B, T, H, HV, init="normal0.1")
        for n in names:
            static[n].copy_(getattr(nxt, n).to(dev))
        graph.replay()
        torch.cuda.synchronize()
        ref_o, ref_s = kda.chunk_prefill_split(*(static[n] for n in names))
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref_o)), f"replay {r}: o differs"
        assert torch.equal(fin, ref_s), f"replay {r}: final state differs"
        say(f"noalloc prefill graph replay {r} ({kda.prefill_partition(B, HV)} form): identical to the direct call")


def test_packed_decode_graph_replay(gpu_lib):
    kda = gpu_lib
    dev = "cuda"
    B = 32
    base = synth.packed_decode_config(B, N=64, row_pad=8, seed=42)
    H = base.H
    names = ("mixed_qkv", "raw_gate", "raw_beta", "A_log", "dt_bias", "state_indices")
    static = {n: getattr(base, n).to(dev) for n in names}
    pool0 = base.pool.to(dev)
    pool = pool0.clone()
    out = torch.empty((B, 1, H, 128), dtype=torch.bfloat16, device=dev)
    qkv = lambda d: d["mixed_qkv"][:, : 3 * H * 128]
    call = lambda d, p, **kw: kda.packed_decode(qkv(d), d["raw_gate"], d["raw_beta"], d["A_log"], d["dt_bias"], p,
                                                d["state_indices"], **kw)
    call(static, pool, out=out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static, pool, out=out)
    torch.cuda.synchronize()
    for r in range(4):
        nxt = synth.packed_decode_config(B, N=64, row_pad=8, seed=43 + r)
        for n in names:
            static[n].copy_(getattr(nxt, n).to(dev))
        pool.copy_(pool0)
        graph.replay()
        torch.cuda.synchronize()
        ref_pool = pool0.clone()
        ref_out = call(static, ref_pool)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref_out)), f"replay {r}: o differs"
        assert torch.equal(_bits(pool), _bits(ref_pool)), f"replay {r}: pool differs"
        say(f"packed decode graph replay {r}: identical to the direct call")
