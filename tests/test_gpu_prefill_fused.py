"""The two prefill partitions on the GPU: kda_chunk_prefill_fused,
kda_chunk_prefill_split and kda_chunk_prefill, which picks one of them.

Both partitions run the same per-chunk arithmetic with the same operand
precisions and the same MFMA accumulation orders; the split form only
passes the chunk-local matrices through the workspace, which stores exactly
the values the fused form reads from LDS.  So the fused results must equal
the split results bit for bit, and the automatic entry point must equal
both, which is checked on every workload shape the prefill is tested on
(kda_chunk_prefill itself is checked against the oracle in
test_gpu_prefill.py); a few cases are also compared with the oracle
directly.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_o, check_state, say

pytestmark = pytest.mark.gpu


def _args(inp):
    dev = "cuda"
    s0 = None if inp.initial_state is None else inp.initial_state.to(dev)
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.to(dev)
    return (inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev), inp.beta.to(dev), s0, cu)


def _bitwise(kda, inp):
    a = _args(inp)
    N = inp.cu_seqlens.numel() - 1 if inp.cu_seqlens is not None else 0
    say(f"fused vs split vs automatic ({kda.prefill_partition(inp.q.shape[0], inp.v.shape[2], N)}) "
        f"{inp.name} shape={inp.shape}")
    of, sf = kda.chunk_prefill_fused(*a)
    os_, ss = kda.chunk_prefill_split(*a)
    oa, sa = kda.chunk_prefill(*a)
    torch.cuda.synchronize()
    for what, (o, s) in (("split", (os_, ss)), ("automatic", (oa, sa))):
        assert torch.equal(of.view(torch.int16), o.view(torch.int16)), f"{inp.name}: o differs ({what})"
        assert torch.equal(sf, s), f"{inp.name}: final state differs ({what})"
    return of, sf


def _oracle(inp):
    a = synth.to_numpy(inp)
    return oracle.recurrent(a["q"], a["k"], a["v"], a["g"], a["beta"], a["initial_state"], a["cu_seqlens"])


def test_fused_small_against_oracle(gpu_lib):
    inp = synth.config0()
    of, sf = _bitwise(gpu_lib, inp)
    o_ref, s_ref = _oracle(inp)
    check_o(of, o_ref, inp.name)
    check_state(sf, s_ref, inp.name)


def test_fused_harsh_decay_ragged_tail(gpu_lib):
    inp = synth.config1()
    of, sf = _bitwise(gpu_lib, inp)
    o_ref, s_ref = _oracle(inp)
    say(f"  o_err={check_o(of, o_ref, inp.name):.2e} state_err={check_state(sf, s_ref, inp.name):.2e}")


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 129, 200])
def test_fused_ragged_lengths(gpu_lib, T):
    _bitwise(gpu_lib, synth.prefill_basic(50 + T, 2, T, 2, 2, init="normal0.1"))


def test_fused_worked_example_exact(gpu_lib):
    inp = synth.worked_example()
    of, sf = _bitwise(gpu_lib, inp)
    assert torch.all(of.float() == 0.08837890625)


@pytest.mark.parametrize("mode", [("gain", "strong", "edge", "normal"), ("zero_rows", "zero", "edge", "none"),
                                  ("tiny", "moderate", "sigmoid", "zero")], ids=lambda m: "-".join(m))
def test_fused_stress(gpu_lib, mode):
    qk, gate, bm, st = mode
    _bitwise(gpu_lib, synth.prefill_stress(70, 2, 300, 2, 4, qk_mode=qk, gate=gate, beta_mode=bm, state=st))


def test_fused_extreme_gates(gpu_lib):
    inp = synth.prefill_basic(80, 1, 200, 2, 2, init="normal0.1")
    inp.g[..., :8] = -15.0
    inp.g[:, 100:110, :, 8:16] = -40.0
    _bitwise(gpu_lib, inp)


def test_fused_gqa_and_varlen(gpu_lib):
    lens = [70, 0, 1, 129, 64, 33]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    inp = synth.prefill_basic(90, 1, int(cu[-1]), 2, 4, init="normal0.1", cu_seqlens=cu, name="varlen_small")
    _bitwise(gpu_lib, inp)
    _bitwise(gpu_lib, synth.prefill_basic(91, 1, 150, 2, 4, init="none"))


def test_fused_zero_length(gpu_lib):
    inp = synth.prefill_basic(94, 2, 0, 2, 2, init="normal0.1")
    of, sf = gpu_lib.chunk_prefill_fused(*_args(inp))
    torch.cuda.synchronize()
    assert of.numel() == 0 and torch.equal(sf.cpu(), inp.initial_state)


def test_fused_full_scale(gpu_lib):
    """The bench workload (H=HV=96, T=8192), fused == split bitwise."""
    _bitwise(gpu_lib, synth.config2())


def test_fused_many_units_varlen(gpu_lib):
    """The packed 16-sequence GQA batch (512 units, more than the compute
    units), fused == split bitwise."""
    _bitwise(gpu_lib, synth.config3())


def test_partition_choice_on_device(gpu_lib):
    """On MI355X (256 compute units) the automatic entry point runs the
    split form at the 96-unit workload and the fused form from 192 units."""
    kda = gpu_lib
    assert kda.prefill_partition(1, 96) == "split"
    assert kda.prefill_partition(1, 191) == "split"
    assert kda.prefill_partition(1, 192) == "fused"
    assert kda.prefill_partition(1, 32, 16) == "fused"
    assert kda.prefill_partition(16, 64) == "fused"


def test_fused_crossover_shapes(gpu_lib):
    """Either side of the crossover (191 and 192 units), all three equal."""
    _bitwise(gpu_lib, synth.prefill_basic(95, 1, 130, 1, 191, init="normal0.1", name="units191"))
    _bitwise(gpu_lib, synth.prefill_basic(96, 1, 130, 1, 192, init="normal0.1", name="units192"))


def test_fused_longest_first_order_ties_and_empties(gpu_lib):
    """Packed sequences are taken longest first (ties by index); lengths with
    equal chunk counts, empty and one-token sequences, 9 x 24 = 216 units."""
    lens = [64, 130, 0, 1, 129, 65, 64, 200, 0]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    _bitwise(gpu_lib, synth.prefill_basic(97, 1, int(cu[-1]), 8, 24, init="normal0.1", cu_seqlens=cu,
                                          name="varlen_ties"))


def test_fused_more_sequences_than_threads(gpu_lib):
    """600 packed sequences (more than the 512 a workgroup ranks): index order."""
    rng = np.random.default_rng(98)
    lens = rng.integers(0, 40, size=600)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    _bitwise(gpu_lib, synth.prefill_basic(98, 1, int(cu[-1]), 1, 1, init="normal0.1", cu_seqlens=cu,
                                          name="varlen_600"))
