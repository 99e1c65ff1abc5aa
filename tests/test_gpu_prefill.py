"""kda_chunk_prefill on the GPU against the fp64 oracle.

Small workloads are compared in full; the full-size workloads (H=96, T=8192
and the packed variable-length GQA batch) run in the launch configuration
the benchmark times and are compared on sampled heads and sequences, which
the oracle computes independently.  Invariants that must hold bit for bit
(determinism, GQA expansion, packing, state carry) are checked GPU vs GPU.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_o, check_state, say

pytestmark = pytest.mark.gpu


def _gpu(kda, inp):
    dev = "cuda"
    s0 = None if inp.initial_state is None else inp.initial_state.to(dev)
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.to(dev)
    o, s = kda.chunk_prefill(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev),
                             inp.beta.to(dev), s0, cu)
    torch.cuda.synchronize()
    return o, s


def _ref(inp, heads=None, seq=None):
    a = synth.to_numpy(inp)
    q, k, v, g, beta, s0, cu = (a["q"], a["k"], a["v"], a["g"], a["beta"],
                                a["initial_state"], a["cu_seqlens"])
    return oracle.recurrent(q, k, v, g, beta, s0, cu)


def _full_check(kda, inp):
    say(f"prefill {inp.name} shape={inp.shape}")
    o, s = _gpu(kda, inp)
    o_ref, s_ref = _ref(inp)
    eo = check_o(o, o_ref, inp.name)
    es = check_state(s, s_ref, inp.name)
    say(f"  o_err={eo:.2e} state_err={es:.2e}")


def test_small_single_head(gpu_lib):
    _full_check(gpu_lib, synth.config0())


def test_worked_example_exact(gpu_lib):
    inp = synth.worked_example()
    o, s = _gpu(gpu_lib, inp)
    assert torch.all(o.float() == 0.08837890625)
    sf = s.cpu()
    assert torch.all(sf[0, 0, 0] == 1.0) and torch.all(sf[0, 0, 1:] == 0.0)


def test_beta_zero_exact(gpu_lib):
    inp = synth.worked_example(beta_value=0.0)
    o, s = _gpu(gpu_lib, inp)
    assert torch.all(o == 0) and torch.all(s == 0)
    inp = synth.config0()
    inp.beta.zero_()
    o, s = _gpu(gpu_lib, inp)
    assert torch.all(o == 0) and torch.all(s == 0)


def test_harsh_decay_ragged_tail(gpu_lib):
    _full_check(gpu_lib, synth.config1())


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 129, 200])
def test_ragged_lengths(gpu_lib, T):
    _full_check(gpu_lib, synth.prefill_basic(50 + T, 2, T, 2, 2, init="normal0.1"))


def test_many_units_wide_tile(gpu_lib):
    """(sequence, head) units >= 256 select the 128-column tile."""
    _full_check(gpu_lib, synth.prefill_basic(61, 2, 130, 128, 128, init="normal0.1"))


STRESS = [
    ("gain", "moderate", "sigmoid", "normal"),
    ("gain", "strong", "edge", "normal"),
    ("gain", "weak", "one", "none"),
    ("tiny", "moderate", "sigmoid", "zero"),
    ("zero_rows", "strong", "sigmoid", "normal"),
    ("zero_rows", "zero", "edge", "none"),
    ("gain", "zero", "zero", "normal"),
    ("tiny", "strong", "one", "normal"),
]


@pytest.mark.parametrize("mode", STRESS, ids=["-".join(m) for m in STRESS])
def test_stress_modes(gpu_lib, mode):
    qk, gate, bm, st = mode
    _full_check(gpu_lib, synth.prefill_stress(70, 2, 300, 2, 4, qk_mode=qk, gate=gate, beta_mode=bm, state=st))


def test_extreme_gate_fallback(gpu_lib):
    """Gates of -15 on some channels push the split decay factors of diagonal
    blocks past float range; those blocks are evaluated pair by pair."""
    inp = synth.prefill_basic(80, 1, 200, 2, 2, init="normal0.1")
    inp.g[..., :8] = -15.0
    inp.g[:, 100:110, :, 8:16] = -40.0
    _full_check(gpu_lib, inp)


def test_full_scale_sampled_heads(gpu_lib):
    """H=HV=96, T=8192 as timed; heads 0, 47 and 95 against the oracle."""
    inp = synth.config2()
    say("prefill cfg2 full size")
    o, s = _gpu(gpu_lib, inp)
    for h in (0, 47, 95):
        sub = synth.PrefillInputs(inp.q[:, :, h:h + 1], inp.k[:, :, h:h + 1], inp.v[:, :, h:h + 1],
                                  inp.g[:, :, h:h + 1], inp.beta[:, :, h:h + 1],
                                  inp.initial_state[:, h:h + 1], None, f"cfg2_head{h}")
        o_ref, s_ref = _ref(sub)
        eo = check_o(o[:, :, h:h + 1], o_ref, sub.name)
        es = check_state(s[:, h:h + 1], s_ref, sub.name)
        say(f"  head {h}: o_err={eo:.2e} state_err={es:.2e}")


def test_varlen_gqa_sampled(gpu_lib):
    """Packed 16-sequence batch, H=16, HV=32: sampled (sequence, Q/K head)
    pairs against the oracle run on that sequence and head pair alone."""
    inp = synth.config3()
    say(f"prefill {inp.name}")
    o, s = _gpu(gpu_lib, inp)
    cu = inp.cu_seqlens.tolist()
    lens = [cu[i + 1] - cu[i] for i in range(16)]
    picks = [(int(np.argmax(lens)), 0), (int(np.argmin(lens)), 5), (3, 15), (9, 7)]
    for n, hq in picks:
        t0, t1 = cu[n], cu[n + 1]
        hv = slice(2 * hq, 2 * hq + 2)
        sub = synth.PrefillInputs(inp.q[:, t0:t1, hq:hq + 1], inp.k[:, t0:t1, hq:hq + 1],
                                  inp.v[:, t0:t1, hv], inp.g[:, t0:t1, hv], inp.beta[:, t0:t1, hv],
                                  inp.initial_state[n:n + 1, hv], None, f"cfg3_seq{n}_qk{hq}")
        o_ref, s_ref = _ref(sub)
        eo = check_o(o[:, t0:t1, hv], o_ref, sub.name)
        es = check_state(s[n:n + 1, hv], s_ref, sub.name)
        say(f"  seq {n} (len {t1 - t0}) qk-head {hq}: o_err={eo:.2e} state_err={es:.2e}")


def test_varlen_small_full(gpu_lib):
    lens = [70, 0, 1, 129, 64, 33]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    inp = synth.prefill_basic(90, 1, int(cu[-1]), 2, 4, init="normal0.1", cu_seqlens=cu, name="varlen_small")
    _full_check(gpu_lib, inp)


# ------------------------------------------------------------ invariants (GPU vs GPU)


def test_deterministic_and_inputs_untouched(gpu_lib):
    inp = synth.config1()
    dev = [t.cuda() for t in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.initial_state)]
    keep = [t.clone() for t in dev]
    o1, s1 = gpu_lib.chunk_prefill(*dev)
    o2, s2 = gpu_lib.chunk_prefill(*dev)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    for a, b in zip(dev, keep):
        assert torch.equal(a, b)


def test_gqa_equals_expanded_heads(gpu_lib):
    inp = synth.prefill_basic(91, 1, 150, 2, 4, init="normal0.1")
    o1, s1 = _gpu(gpu_lib, inp)
    idx = torch.tensor([0, 0, 1, 1])
    exp = synth.PrefillInputs(inp.q[:, :, idx].contiguous(), inp.k[:, :, idx].contiguous(), inp.v, inp.g,
                              inp.beta, inp.initial_state, None, "expanded")
    o2, s2 = _gpu(gpu_lib, exp)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_packed_equals_separate(gpu_lib):
    lens = [100, 64, 1, 77]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    inp = synth.prefill_basic(92, 1, int(cu[-1]), 2, 2, init="normal0.1", cu_seqlens=cu)
    o, s = _gpu(gpu_lib, inp)
    for n in range(len(lens)):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        part = synth.PrefillInputs(inp.q[:, t0:t1], inp.k[:, t0:t1], inp.v[:, t0:t1], inp.g[:, t0:t1],
                                   inp.beta[:, t0:t1], inp.initial_state[n:n + 1], None, "part")
        o1, s1 = _gpu(gpu_lib, part)
        assert torch.equal(o[:, t0:t1], o1) and torch.equal(s[n:n + 1], s1)


def test_state_carry_split_bitwise(gpu_lib):
    inp = synth.prefill_basic(93, 1, 320, 2, 2, init="normal0.1")
    o, s = _gpu(gpu_lib, inp)
    a = synth.PrefillInputs(*(t[:, :192] for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)),
                            inp.initial_state, None, "a")
    oa, sa = _gpu(gpu_lib, a)
    b = synth.PrefillInputs(*(t[:, 192:].contiguous() for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)),
                            sa.cpu(), None, "b")
    ob, sb = _gpu(gpu_lib, b)
    assert torch.equal(torch.cat([oa, ob], dim=1), o) and torch.equal(sb, s)


def test_zero_length(gpu_lib):
    inp = synth.prefill_basic(94, 2, 0, 2, 2, init="normal0.1")
    o, s = _gpu(gpu_lib, inp)
    assert o.numel() == 0 and torch.equal(s.cpu(), inp.initial_state)
    inp = synth.prefill_basic(95, 2, 0, 2, 2, init="none")
    o, s = _gpu(gpu_lib, inp)
    assert torch.all(s == 0)
