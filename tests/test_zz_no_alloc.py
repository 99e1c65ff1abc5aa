"""kda_chunk_prefill_noalloc (static workspace, nothing allocated) against
kda_chunk_prefill_split with a caller workspace: the same kernels on the
same inputs give bitwise equal results (the window size does not change the
arithmetic, and the fused form the allocation-free call picks from 192
units equals the split form bit for bit), on two calls in a row (the second
with a smaller input, so it meets the first call's leftovers in the shared
array), varlen included."""

import numpy as np
import pytest
import torch

import synth
from gpu_util import say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _pair(kda, inp):
    dev = "cuda"
    a = [None if t is None else t.to(dev) for t in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.initial_state,
                                                     inp.cu_seqlens)]
    B, T = inp.q.shape[:2]
    HV = inp.v.shape[2]
    N = inp.cu_seqlens.numel() - 1 if inp.cu_seqlens is not None else B
    o = torch.full((B, T, HV, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    s = torch.full((N, HV, 128, 128), float("nan"), dtype=torch.float32, device=dev)
    kda.chunk_prefill_noalloc(*a, out=o, final_state=s)
    ro, rs = kda.chunk_prefill_split(*a)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o), _bits(ro)), f"{inp.name}: o differs"
    assert torch.equal(s, rs), f"{inp.name}: final state differs"
    say(f"noalloc {inp.name} ({kda.prefill_partition(B, HV, N if inp.cu_seqlens is not None else 0)} form): "
        "bitwise equal to kda_chunk_prefill_split")


def test_noalloc_matches_prefill_twice(gpu_lib):
    # 96 value heads x 8192 tokens: 13 windows of the static workspace
    # (10 slots per head each) against one caller-workspace window of 130
    _pair(gpu_lib, synth.config2())
    _pair(gpu_lib, synth.prefill_basic(61, 2, 300, 2, 4, init="none", name="small"))


def test_noalloc_fused_form_then_split_form(gpu_lib):
    # 4 x 64 = 256 units take the fused form (the array untouched), then a
    # smaller split-form call
    _pair(gpu_lib, synth.prefill_basic(64, 4, 300, 16, 64, init="normal0.1", name="units256"))
    _pair(gpu_lib, synth.prefill_basic(65, 1, 200, 2, 4, init="normal0.1", name="units4"))


def test_noalloc_varlen_after_larger(gpu_lib):
    _pair(gpu_lib, synth.config1())
    lens = [70, 0, 1, 129, 64, 33]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    _pair(gpu_lib, synth.prefill_basic(62, 1, int(cu[-1]), 2, 4, init="normal0.1", cu_seqlens=cu,
                                       name="varlen"))


def test_noalloc_rejects_too_many_heads(gpu_lib):
    inp = synth.prefill_basic(63, 1, 2, 1, 1024, init="none")
    with pytest.raises(gpu_lib.KDAError, match="WORKSPACE"):
        gpu_lib.chunk_prefill_noalloc(*(t.cuda() for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)))
