"""kda_chunk_prefill on the GPU against the fp64 oracle.

Every workload is compared in full, the full-size ones (H=96, T=8192 and
the packed variable-length GQA batch) in the launch configuration the
benchmark times, with the oracle spread over the host's cores.  Invariants that must hold bit for bit
(determinism, GQA expansion, packing, state carry) are checked GPU vs GPU.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_o, check_state, say
from oracle.parallel import recurrent_parallel

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
    """256 (sequence, value head) units: more than one per compute unit."""
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


def test_full_scale_all_heads(gpu_lib):
    """H=HV=96, T=8192 in the launch the benchmark times; every head's o
    and final state against the oracle (run over the host's cores, one
    process per head)."""
    inp = synth.config2()
    say("prefill cfg2 full size")
    o, s = _gpu(gpu_lib, inp)
    a = synth.to_numpy(inp)
    o_ref, s_ref = recurrent_parallel(a["q"], a["k"], a["v"], a["g"], a["beta"], a["initial_state"])
    eo = check_o(o, o_ref, inp.name)
    es = check_state(s, s_ref, inp.name)
    say(f"  all 96 heads: o_err={eo:.2e} state_err={es:.2e}")


def test_varlen_gqa_all(gpu_lib):
    """Packed 16-sequence batch, H=16, HV=32, in one call; every sequence
    and head against the oracle (one process per sequence and Q/K head)."""
    inp = synth.config3()
    say(f"prefill {inp.name}")
    o, s = _gpu(gpu_lib, inp)
    a = synth.to_numpy(inp)
    o_ref, s_ref = recurrent_parallel(a["q"], a["k"], a["v"], a["g"], a["beta"], a["initial_state"],
                                      a["cu_seqlens"])
    eo = check_o(o, o_ref, inp.name)
    es = check_state(s, s_ref, inp.name)
    say(f"  all sequences and heads: o_err={eo:.2e} state_err={es:.2e}")


def test_state_near_domain_bound(gpu_lib):
    """Initial states up to the prefill's documented bound (|state| < 2^14)
    and values in the thousands: finite results, the final state within the
    1e-3 relative bar, and o within 1e-2 of the oracle relative to o's
    scale (the recurrence is linear in (v, state), so absolute errors grow
    with them; the elementwise o bar is stated for unit-scale values)."""
    inp = synth.prefill_basic(96, 1, 300, 2, 2, init="normal0.1", name="state_bound")
    s0 = inp.initial_state
    inp.initial_state = s0 * (16000.0 / float(s0.abs().max()))
    inp.v = (inp.v.float() * 1000.0).to(torch.bfloat16)
    o, s = _gpu(gpu_lib, inp)
    o_ref, s_ref = _ref(inp)
    of = o.float().cpu().numpy()
    assert np.all(np.isfinite(of))
    eo = float(np.abs(of - o_ref).max() / np.abs(o_ref).max())
    es = check_state(s, s_ref, inp.name)
    say(f"  state bound: max|S0|={float(inp.initial_state.abs().max()):.0f} max|S|={np.abs(s_ref).max():.0f} "
        f"o_err/max|o|={eo:.2e} state_err={es:.2e}")
    assert eo <= 1e-2


def test_many_windows_varlen(gpu_lib):
    """A workspace of one chunk slot per value head makes the split form's
    windows one slot long, so sequences span many windows (the state
    crossing them through final_state) and empty and one-token sequences
    sit inside later windows; compared in full against the oracle, and
    bitwise against the single-window split call, the allocation-free call
    and the automatic call (both fused here: 7 x 512 units)."""
    lens = [100, 0, 1, 64, 200, 0, 37]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    inp = synth.prefill_basic(97, 1, int(cu[-1]), 256, 512, init="normal0.1", cu_seqlens=cu,
                              name="varlen_512heads")
    dev = "cuda"
    a = [t.to(dev) for t in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.initial_state, inp.cu_seqlens)]
    one_slot = torch.empty(512 * gpu_lib.PREFILL_SLOT_BYTES, dtype=torch.uint8, device=dev)
    o, s = gpu_lib.chunk_prefill_split(*a, workspace=one_slot)
    runs = {"split, one window": gpu_lib.chunk_prefill_split(*a),
            "allocation-free": gpu_lib.chunk_prefill_noalloc(*a),
            "automatic": gpu_lib.chunk_prefill(*a)}
    torch.cuda.synchronize()
    assert gpu_lib.prefill_partition(1, 512, len(lens)) == "fused"
    for what, (o1, s1) in runs.items():
        assert torch.equal(o.view(torch.int16), o1.view(torch.int16)) and torch.equal(s, s1), what
    o_ref, s_ref = _ref(inp)
    eo = check_o(o, o_ref, inp.name)
    es = check_state(s, s_ref, inp.name)
    say(f"  512 heads, one-slot windows: o_err={eo:.2e} state_err={es:.2e}")


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


# ---------------------------------------------------------------------------
# The normalisation fused into the prefill equals the canonical one bit for
# bit.  With g = 0 every decay factor is exactly 1, so the workspace block Qg
# holds fp16(fp32(K^-1/2 * fp16(q^))) and Kg^T holds fp16(k^): a q^ or k^ off
# by one bf16 step changes them (unless both round to zero in fp16).  This reads the chunk slots back through
# their documented layout (slot = W | Qg | Kg^T | Aqk | A | gamma; rows of
# 16-byte pieces stored at piece ^ (row % 8); contraction indices permuted
# within each group of 32 as 4g+e -> 8g+e, 16+4g+e -> 8g+4+e).

_WS_SLOT, _WS_QG, _WS_KGT = 66048, 16384, 32768


def _perm32(c):
    cp = c & 31
    return (c & ~31) + 8 * ((cp & 15) >> 2) + 4 * (cp >> 4) + (cp & 3)


def _read_block(slot, off, rows, cols):
    """Logical [rows][cols] fp16 block (cols permuted, pieces swizzled) as uint16."""
    raw = slot[off:off + rows * cols * 2].view(np.uint16).reshape(rows, cols)
    out = np.empty((rows, cols), np.uint16)
    for r in range(rows):
        for c in range(cols):
            pos = _perm32(c)
            piece, e = pos // 8, pos % 8
            out[r, c] = raw[r, (piece ^ (r & 7)) * 8 + e]
    return out


def _crafted_rows(rng, n):
    rows = []
    e0 = np.zeros(128, np.float32)
    e0[0] = 1
    rows += [e0, -e0, np.zeros(128, np.float32), np.full(128, 3.0, np.float32)]
    for span in (10, 15, 16, 17, 30, 38, 60, 120):      # fast path and both sides of its limit
        for _ in range(4):
            r = rng.standard_normal(128) * np.exp2(rng.integers(-span // 2, span // 2 + 1, 128))
            rows.append(r.astype(np.float32))
    rows.append((rng.standard_normal(128) * 1e-5).astype(np.float32))
    while len(rows) < n:
        rows.append((rng.standard_normal(128) * np.exp(0.6 * rng.standard_normal())).astype(np.float32))
    rows = np.stack(rows[:n])
    return rows[rng.permutation(n)]


def test_fused_normalisation_bit_exact(gpu_lib):
    kda = gpu_lib
    rng = np.random.default_rng(11)
    B, T, H = 1, 256, 2
    q = torch.from_numpy(_crafted_rows(rng, T * H).reshape(B, T, H, 128)).to(torch.bfloat16)
    k = torch.from_numpy(_crafted_rows(rng, T * H).reshape(B, T, H, 128)).to(torch.bfloat16)
    v = torch.randn(B, T, H, 128, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    g = torch.zeros(B, T, H, 128)
    beta = torch.full((B, T, H), 0.5).to(torch.bfloat16)
    dev = "cuda"
    ws = torch.zeros(kda.workspace_size(B, T, H, H), dtype=torch.uint8, device=dev)
    kda.chunk_prefill(q.to(dev), k.to(dev), v.to(dev), g.to(dev), beta.to(dev), None, None, workspace=ws)
    torch.cuda.synchronize()
    wsn = ws.cpu().numpy()
    nslots = wsn.size // (_WS_SLOT * H)
    qhat = oracle.l2norm_bf16(q.float().numpy())          # exact bf16 values as float32
    khat = oracle.l2norm_bf16(k.float().numpy())
    scale = np.float32(0.08838834764831845)
    bad_q = bad_k = 0
    for hv in range(H):
        for c in range(T // 64):
            slot = wsn[(hv * nslots + c) * _WS_SLOT:(hv * nslots + c + 1) * _WS_SLOT]
            qg = _read_block(slot, _WS_QG, 64, 128)
            kgt = _read_block(slot, _WS_KGT, 128, 64)
            qh = qhat[0, 64 * c:64 * c + 64, hv].astype(np.float16)
            kh = khat[0, 64 * c:64 * c + 64, hv].astype(np.float16)
            want_q = (qh.astype(np.float32) * scale).astype(np.float16)
            want_k = kh.T
            # Compared as values: the kernel forms these products with a fused
            # multiply-add whose zero addend turns -0 into +0, which no MFMA
            # sum can see; every nonzero value must match bit for bit.
            bad_q += np.count_nonzero(qg.view(np.float16) != want_q)
            bad_k += np.count_nonzero(kgt.view(np.float16) != want_k)
    say(f"fused normalisation: q mismatches {bad_q}, k mismatches {bad_k} of {T * H * 128} each")
    assert bad_q == 0 and bad_k == 0


def test_long_sequence_full(gpu_lib):
    """One 131,072-token sequence (2,048 chunks per head), H=HV=8, with an
    initial state: every output and final state against the oracle."""
    inp = synth.prefill_basic(99, 1, 131072, 8, 8, init="normal0.1", name="t131072")
    say(f"prefill {inp.name} shape={inp.shape}")
    o, s = _gpu(gpu_lib, inp)
    a = synth.to_numpy(inp)
    o_ref, s_ref = recurrent_parallel(a["q"], a["k"], a["v"], a["g"], a["beta"], a["initial_state"])
    eo = check_o(o, o_ref, inp.name)
    es = check_state(s, s_ref, inp.name)
    say(f"  o_err={eo:.2e} state_err={es:.2e}")


@pytest.mark.parametrize("B,T,H,HV", [(1, 200, 1, 64), (1, 130, 2, 200), (3, 77, 7, 21)],
                         ids=["group64-split", "group100-fused", "odd-heads"])
def test_large_gqa_groups_full(gpu_lib, B, T, H, HV):
    """Large GQA groups (up to 100 value heads per Q/K head) and odd head
    counts, on both partitions: every output and state against the oracle."""
    inp = synth.prefill_basic(100 + HV, B, T, H, HV, init="normal0.1", name=f"gqa_h{H}_hv{HV}")
    say(f"prefill {inp.name} shape={inp.shape} ({gpu_lib.prefill_partition(B, HV)} form)")
    o, s = _gpu(gpu_lib, inp)
    a = synth.to_numpy(inp)
    o_ref, s_ref = recurrent_parallel(a["q"], a["k"], a["v"], a["g"], a["beta"], a["initial_state"])
    eo = check_o(o, o_ref, inp.name)
    es = check_state(s, s_ref, inp.name)
    say(f"  o_err={eo:.2e} state_err={es:.2e}")
