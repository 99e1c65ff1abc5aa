"""The split prefill's overlapped schedule against its sequential schedule.

With sequences of equal length (no cu_seqlens; or one packed sequence), 48
to CUs - 32 (sequence, value head) units, at least 48 chunk rows (24 when
twice the units exceed the compute units) and a workspace with room for the
ready flags (the size kda_chunk_prefill_workspace_size returns),
kda_chunk_prefill_split runs the chunk-parallel kernel over the first chunk
rows on every compute unit and over the rest on the workgroups that stay,
while the carry (one workgroup per unit, 32 state columns per wave) runs on
a second stream on the compute units of those that leave, waiting for each
of its slots to be flagged.  The arithmetic of every
column is the one the sequential schedule performs, so both schedules (and
the fused form) must agree bit for bit; a workspace without the flag room
forces the sequential schedule on the same inputs.  That the overlapped
schedule ran is read back from the flags it leaves set in the workspace.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_o, check_state, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t


def _args(inp):
    dev = "cuda"
    s0 = None if inp.initial_state is None else inp.initial_state.to(dev)
    return (inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev), inp.beta.to(dev), s0, None)


def _flag_bytes(nslots, HV, nseq=1):
    # ready flags per (slot, value head), then a status word per unit
    return ((nslots + nseq) * HV * 4 + 255) // 256 * 256


def _run(kda, args, B, T, H, HV, overlapped):
    """kda_chunk_prefill_split with the full workspace (overlapped) or the
    slots alone (sequential, one window); returns o, final state and the
    flag region (None for the sequential run)."""
    need = kda.workspace_size(B, T, H, HV)
    nslots = (B * T) // 64 + B + 1
    fb = _flag_bytes(nslots, HV, B)
    assert need == nslots * HV * kda.PREFILL_SLOT_BYTES + fb
    ws = torch.zeros(need if overlapped else need - fb, dtype=torch.uint8, device="cuda")
    o, s = kda.chunk_prefill_split(*args, workspace=ws)
    torch.cuda.synchronize()
    return o, s, (ws[need - fb:].view(torch.int32) if overlapped else None)


def _compare(kda, inp, name):
    B, T, H = inp.q.shape[:3]
    HV = inp.v.shape[2]
    a = _args(inp)
    oo, so, flags = _run(kda, a, B, T, H, HV, True)
    os_, ss, _ = _run(kda, a, B, T, H, HV, False)
    nslots = (B * T) // 64 + B + 1
    set_flags = int((flags[:nslots * HV] != 0).sum())
    gave_up = int((flags[nslots * HV:nslots * HV + B * HV] != 0).sum())
    assert set_flags > 0, f"{name}: the overlapped schedule did not run"
    # one flag per (chunk, value head) of every sequence, each set once its slot is stored
    assert set_flags == B * ((T + 63) // 64) * HV, f"{name}: {set_flags} slots flagged"
    assert gave_up == 0, f"{name}: {gave_up} units gave up waiting"
    assert torch.equal(_bits(oo), _bits(os_)), f"{name}: o differs between the schedules"
    assert torch.equal(so, ss), f"{name}: final state differs between the schedules"
    say(f"overlapped == sequential bitwise, {name} (B={B} T={T} H={H} HV={HV}; {set_flags} slots flagged)")
    return oo, so


def test_overlap_bench_workload(gpu_lib):
    """The bench workload (B=1, H=HV=96, T=8192): both schedules, the fused
    form and the automatic entry point agree bit for bit."""
    kda = gpu_lib
    inp = synth.config2()
    oo, so = _compare(kda, inp, "B=1 H=HV=96 T=8192")
    of, sf = kda.chunk_prefill_fused(*_args(inp))
    torch.cuda.synchronize()
    assert torch.equal(_bits(oo), _bits(of)) and torch.equal(so, sf), "fused form differs"
    # the automatic entry point with its default workspace takes the same path
    oa, sa = kda.chunk_prefill(*_args(inp))
    torch.cuda.synchronize()
    assert torch.equal(_bits(oo), _bits(oa)) and torch.equal(so, sa), "automatic entry point differs"


def test_overlap_ragged_gqa_against_oracle(gpu_lib):
    """48 value heads over 24 Q/K heads, a ragged last chunk and an initial
    state; sampled heads against the fp64 oracle."""
    kda = gpu_lib
    inp = synth.prefill_basic(120, 1, 3085, 24, 48, init="normal0.1", name="ragged_gqa48")
    oo, so = _compare(kda, inp, "ragged GQA")
    a = synth.to_numpy(inp)
    for hv in (0, 17, 47):
        hq = hv // 2
        o_ref, s_ref = oracle.recurrent(a["q"][:, :, hq:hq + 1], a["k"][:, :, hq:hq + 1], a["v"][:, :, hv:hv + 1],
                                        a["g"][:, :, hv:hv + 1], a["beta"][:, :, hv:hv + 1],
                                        a["initial_state"][:, hv:hv + 1], None)
        e_o = check_o(oo[:, :, hv:hv + 1], o_ref, f"head {hv}")
        e_s = check_state(so[:, hv:hv + 1], s_ref, f"head {hv}")
        say(f"  value head {hv}: o_err={e_o:.2e} state_err={e_s:.2e}")


def test_overlap_smallest_qualifying_shape(gpu_lib):
    """48 value heads and 48 chunk rows (the fewest units and rows the
    schedule takes), no initial state; the most units it takes on 256
    compute units (224); 191 units, whose leaving workgroups are rounded up
    to 192; and 24 chunk rows with 160 units (twice the units above the
    compute units)."""
    _compare(gpu_lib, synth.prefill_basic(121, 1, 3072, 48, 48, init="none", name="min48"), "smallest")
    _compare(gpu_lib, synth.prefill_basic(122, 1, 3072, 32, 224, init="normal0.1", name="max224"), "most heads")
    _compare(gpu_lib, synth.prefill_basic(126, 1, 3072, 191, 191, init="normal0.1", name="u191"), "191 units")
    _compare(gpu_lib, synth.prefill_basic(127, 1, 1536, 80, 160, init="normal0.1", name="r24u160"), "24 rows")


@pytest.mark.parametrize("T,H,HV", [(3008, 48, 48), (3072, 47, 47), (3072, 75, 225), (1472, 160, 160),
                                    (1536, 128, 128)],
                         ids=["47rows", "47heads", "225heads", "23rows160heads", "24rows128heads"])
def test_overlap_boundaries_run_sequential(gpu_lib, T, H, HV):
    """Just outside the schedule's range (47 chunk rows, 47 or 225 units on
    256 compute units; 23 rows with 160 units; 24 rows with 128 units, whose
    sequential carry fits the compute units) the split form runs
    sequentially even with the flag room: the flags stay untouched."""
    kda = gpu_lib
    inp = synth.prefill_basic(123, 1, T, H, HV, init="none")
    oo, so, flags = _run(kda, _args(inp), 1, T, H, HV, True)
    assert int((flags != 0).sum()) == 0, "the overlapped schedule ran outside its range"


def test_overlap_several_sequences(gpu_lib):
    """Several equal-length sequences: the chunk kernel takes its items
    chunk-major across the sequences, the carry waits by chunk row.  Two
    sequences of 48 heads with a ragged tail and an initial state (sampled
    heads of the second sequence against the oracle), and three sequences
    of 32 value heads over 16 Q/K heads."""
    kda = gpu_lib
    inp = synth.prefill_basic(124, 2, 3100, 48, 48, init="normal0.1", name="b2_h48")
    oo, so = _compare(kda, inp, "two sequences")
    a = synth.to_numpy(inp)
    for hv in (5, 40):
        o_ref, s_ref = oracle.recurrent(a["q"][1:2, :, hv:hv + 1], a["k"][1:2, :, hv:hv + 1],
                                        a["v"][1:2, :, hv:hv + 1], a["g"][1:2, :, hv:hv + 1],
                                        a["beta"][1:2, :, hv:hv + 1], a["initial_state"][1:2, hv:hv + 1], None)
        e_o = check_o(oo[1:2, :, hv:hv + 1], o_ref, f"sequence 1 head {hv}")
        e_s = check_state(so[1:2, hv:hv + 1], s_ref, f"sequence 1 head {hv}")
        say(f"  sequence 1, value head {hv}: o_err={e_o:.2e} state_err={e_s:.2e}")
    _compare(kda, synth.prefill_basic(125, 3, 4096, 16, 32, init="normal0.1", name="b3_gqa"), "three sequences")


def test_overlap_packed_sequences_run_sequential(gpu_lib):
    """Two packed sequences (cu_seqlens) take the sequential schedule: their
    chunk rows are not formed, and the flags stay untouched."""
    kda = gpu_lib
    lens = [3100, 3300]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    T = int(cu[-1])
    inp = synth.prefill_basic(126, 1, T, 48, 48, init="normal0.1", cu_seqlens=cu, name="packed2")
    a = _args(inp)[:6] + (cu.cuda(),)
    need = kda.workspace_size(1, T, 48, 48, 2)
    nslots = T // 64 + 2 + 1
    fb = _flag_bytes(nslots, 48, 2)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    o, s = kda.chunk_prefill_split(*a, workspace=ws)
    torch.cuda.synchronize()
    assert int((ws[need - fb:].view(torch.int32) != 0).sum()) == 0
    of, sf = kda.chunk_prefill_fused(*a)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o), _bits(of)) and torch.equal(s, sf)


def test_overlap_single_packed_sequence(gpu_lib):
    """One packed sequence (cu_seqlens holding a single sequence) keeps the
    slot order as its chunk rows: 1,580 tokens (25 chunks, the last ragged,
    26 slot rows) with 160 value heads over 80 Q/K heads takes the
    overlapped schedule (24 rows suffice with twice the units above the
    compute units).  Bitwise equal to the sequential schedule and to the
    fused form, every chunk flagged, no unit gave up; one head against the
    oracle."""
    kda = gpu_lib
    T, H, HV = 1580, 80, 160
    cu = torch.tensor([0, T], dtype=torch.int32)
    inp = synth.prefill_basic(128, 1, T, H, HV, init="normal0.1", cu_seqlens=cu, name="packed1_u160")
    a = _args(inp)[:6] + (cu.cuda(),)
    need = kda.workspace_size(1, T, H, HV, 1)
    nslots = T // 64 + 2
    fb = _flag_bytes(nslots, HV, 1)
    assert need == nslots * HV * kda.PREFILL_SLOT_BYTES + fb
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    oo, so = kda.chunk_prefill_split(*a, workspace=ws)
    torch.cuda.synchronize()
    flags = ws[need - fb:].view(torch.int32)
    assert int((flags[:nslots * HV] != 0).sum()) == ((T + 63) // 64) * HV, "the overlapped schedule did not run"
    assert int((flags[nslots * HV:nslots * HV + HV] != 0).sum()) == 0, "a unit gave up waiting"
    ws2 = torch.zeros(need - fb, dtype=torch.uint8, device="cuda")
    os_, ss = kda.chunk_prefill_split(*a, workspace=ws2)
    of, sf = kda.chunk_prefill_fused(*a)
    torch.cuda.synchronize()
    assert torch.equal(_bits(oo), _bits(os_)) and torch.equal(so, ss), "overlapped differs from sequential"
    assert torch.equal(_bits(oo), _bits(of)) and torch.equal(so, sf), "overlapped differs from the fused form"
    x = synth.to_numpy(inp)
    hv = 131
    hq = hv // (HV // H)
    o_ref, s_ref = oracle.recurrent(x["q"][:, :, hq:hq + 1], x["k"][:, :, hq:hq + 1], x["v"][:, :, hv:hv + 1],
                                    x["g"][:, :, hv:hv + 1], x["beta"][:, :, hv:hv + 1],
                                    x["initial_state"][:, hv:hv + 1], x["cu_seqlens"])
    e_o = check_o(oo[:, :, hv:hv + 1], o_ref, f"value head {hv}")
    e_s = check_state(so[:, hv:hv + 1], s_ref, f"value head {hv}")
    say(f"single packed sequence, value head {hv}: o_err={e_o:.2e} state_err={e_s:.2e}")


def test_overlap_repeated_calls_one_workspace(gpu_lib):
    """Three calls in a row on one workspace: each call clears the flags it
    waits for, so a previous call's flags never release a slot early."""
    kda = gpu_lib
    B, T, H, HV = 1, 4096, 64, 64
    need = kda.workspace_size(B, T, H, HV)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for r in range(3):
        inp = synth.prefill_basic(130 + r, B, T, H, HV, init="normal0.1", name=f"rep{r}")
        a = _args(inp)
        o, s = kda.chunk_prefill_split(*a, workspace=ws)
        ro, rs, _ = _run(kda, a, B, T, H, HV, False)
        assert torch.equal(_bits(o), _bits(ro)) and torch.equal(s, rs), f"call {r} differs"
        say(f"call {r} on a reused workspace: identical to the sequential schedule")


def test_overlap_graph_replay(gpu_lib):
    """The overlapped schedule captured in a HIP graph (its second stream
    forks from and joins the captured stream), replayed on new inputs with
    eager work between the replays; every replay equals a direct call."""
    kda = gpu_lib
    dev = "cuda"
    B, T, H, HV = 1, 3085, 24, 48
    names = ("q", "k", "v", "g", "beta", "initial_state")
    first = synth.prefill_basic(140, B, T, H, HV, init="normal0.1")
    static = {n: getattr(first, n).to(dev) for n in names}
    need = kda.workspace_size(B, T, H, HV)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, HV, 128), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((B, HV, 128, 128), dtype=torch.float32, device=dev)
    call = lambda d, **kw: kda.chunk_prefill_split(*(d[n] for n in names), **kw)
    call(static, out=out, final_state=fin, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static, out=out, final_state=fin, workspace=ws)
    torch.cuda.synchronize()
    for r in range(3):
        nxt = synth.prefill_basic(141 + r, B, T, H, HV, init="normal0.1")
        for n in names:
            static[n].copy_(getattr(nxt, n).to(dev))
        graph.replay()
        torch.cuda.synchronize()
        ref_o, ref_s, _ = _run(kda, tuple(static[n] for n in names) + (None,), B, T, H, HV, False)
        assert torch.equal(_bits(out), _bits(ref_o)), f"replay {r}: o differs"
        assert torch.equal(fin, ref_s), f"replay {r}: final state differs"
        say(f"overlapped prefill graph replay {r}: identical to the sequential schedule")


_FIRST_CALL_CAPTURED = r'''
import sys, torch
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
import kda_gated_delta_amd as kda, synth
dev = "cuda"
B, T, H, HV = 1, 3085, 24, 48
names = ("q", "k", "v", "g", "beta", "initial_state")
static = {n: getattr(synth.prefill_basic(150, B, T, H, HV, init="normal0.1"), n).to(dev) for n in names}
need = kda.workspace_size(B, T, H, HV)
ws = torch.zeros(need, dtype=torch.uint8, device=dev)
out = torch.empty((B, T, HV, 128), dtype=torch.bfloat16, device=dev)
fin = torch.empty((B, HV, 128, 128), dtype=torch.float32, device=dev)
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):
    kda.chunk_prefill_split(*(static[n] for n in names), out=out, final_state=fin, workspace=ws)
torch.cuda.synchronize()
nslots = T // 64 + 2
fb = ((nslots + 1) * HV * 4 + 255) // 256 * 256
ws[need - fb:].zero_()
graph.replay()
torch.cuda.synchronize()
captured_flags = int((ws[need - fb:].view(torch.int32) != 0).sum())
ref_o, ref_s = kda.chunk_prefill_split(*(static[n] for n in names))
torch.cuda.synchronize()
same = torch.equal(out.view(torch.int16), ref_o.view(torch.int16)) and torch.equal(fin, ref_s)
print(f"RESULT captured_flags={captured_flags} same={same}", flush=True)
'''


def test_overlap_first_call_under_capture():
    """In a fresh process whose first overlapped-size call is captured into a
    graph, the library makes no stream during the capture: the captured call
    runs the sequential schedule (its replay leaves the flags untouched) and
    equals a direct call made afterwards (which runs overlapped)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _FIRST_CALL_CAPTURED, root], capture_output=True, text=True,
                       timeout=300)
    line = [l for l in r.stdout.splitlines() if l.startswith("RESULT")]
    assert r.returncode == 0 and line, f"subprocess failed: {r.stdout[-2000:]} {r.stderr[-2000:]}"
    say(line[0])
    assert line[0] == "RESULT captured_flags=0 same=True"


def test_overlap_carry_gives_up_and_is_repaired(gpu_lib):
    """With the carry's wait limit at 0, every wait for a flag that is not
    yet set gives up at once: the unit marks its status word, writes no
    final state, and the sequential carry launched after the join redoes it.
    The results still equal the sequential schedule's bit for bit.  (One
    split row here, so each unit waits on its second chunk almost at once.)"""
    kda = gpu_lib
    B, T, H, HV = 2, 3100, 12, 24
    inp = synth.prefill_basic(127, B, T, H, HV, init="normal0.1", name="give_up")
    a = _args(inp)
    prev = kda.prefill_overlap_wait_limit(0)
    try:
        oo, so, flags = _run(kda, a, B, T, H, HV, True)
    finally:
        kda.prefill_overlap_wait_limit(-1)
    assert prev > 0
    nslots = (B * T) // 64 + B + 1
    gave_up = int((flags[nslots * HV:nslots * HV + B * HV] != 0).sum())
    os_, ss, _ = _run(kda, a, B, T, H, HV, False)
    assert torch.equal(_bits(oo), _bits(os_)) and torch.equal(so, ss), "repaired results differ"
    say(f"{gave_up} of {B * HV} units gave up waiting and were redone; results bitwise equal")
    assert gave_up > 0


_SERIALISED = r'''
import sys, torch
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
import kda_gated_delta_amd as kda, synth
dev = "cuda"
B, T, H, HV = 1, 3085, 24, 48
inp = synth.prefill_basic(151, B, T, H, HV, init="normal0.1")
a = [x.to(dev) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.initial_state)] + [None]
need = kda.workspace_size(B, T, H, HV)
nslots = T // 64 + 2
fb = ((nslots + 1) * HV * 4 + 255) // 256 * 256
ws = torch.zeros(need, dtype=torch.uint8, device=dev)
o, s = kda.chunk_prefill_split(*a, workspace=ws)
torch.cuda.synchronize()
flags = ws[need - fb:].view(torch.int32)
ran = int((flags[:nslots * HV] != 0).sum())
gave_up = int((flags[nslots * HV:nslots * HV + HV] != 0).sum())
ws2 = torch.zeros(need - fb, dtype=torch.uint8, device=dev)
ro, rs = kda.chunk_prefill_split(*a, workspace=ws2)
torch.cuda.synchronize()
same = torch.equal(o.view(torch.int16), ro.view(torch.int16)) and torch.equal(s, rs)
print(f"RESULT overlapped={ran > 0} same={same} gave_up={gave_up}", flush=True)
'''


def test_overlap_under_serialised_kernels():
    """In a process where the runtime runs every kernel to completion before
    the next (AMD_SERIALIZE_KERNEL=3) the two kernels cannot overlap: the
    carry runs either after the chunk kernel (it finds every slot flagged;
    the order this runtime takes) or before it (every unit gives up after
    its bounded wait and the sequential carry after the join redoes it).
    Either way the results equal the sequential schedule's bit for bit."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, AMD_SERIALIZE_KERNEL="3")
    r = subprocess.run([sys.executable, "-c", _SERIALISED, root], capture_output=True, text=True, timeout=300,
                       env=env)
    line = [l for l in r.stdout.splitlines() if l.startswith("RESULT")]
    assert r.returncode == 0 and line, f"subprocess failed: {r.stdout[-2000:]} {r.stderr[-2000:]}"
    say(line[0])
    assert line[0].startswith("RESULT overlapped=True same=True")


def _overlap_expected(units, rows, cus):
    """The schedule's range: 48 to CUs - 32 units and at least 48 chunk rows,
    or at least 24 where twice the units exceed the compute units."""
    if units < 48 or units > cus - 32:
        return False
    return rows >= 48 or (rows >= 24 and 2 * units > cus)


@pytest.mark.parametrize("seed", range(6))
def test_overlap_random_shapes(gpu_lib, seed):
    """Seeded random shapes around the overlapped schedule's range: several
    equal-length sequences or one packed sequence, GQA groups, ragged tails,
    initial state present or absent.  The schedule runs exactly where its
    rule says (every chunk flagged, no unit gave up; otherwise the flags stay
    untouched); the split form's two schedules and the fused form agree bit
    for bit; two random heads against the oracle."""
    kda = gpu_lib
    rng = np.random.default_rng(7000 + seed)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    group = int(rng.choice([1, 2, 4]))
    units_target = int(rng.integers(40, 233))
    packed = bool(rng.random() < 0.3)
    B = 1 if packed else int(rng.choice([1, 1, 2, 3]))
    HV = max(group, (units_target // B) // group * group)
    H = HV // group
    T = int(rng.integers(1400, 3300))
    init = str(rng.choice(["none", "normal0.1"]))
    if packed:
        cu = torch.tensor([0, T], dtype=torch.int32)
        inp = synth.prefill_basic(7100 + seed, 1, T, H, HV, init=init, cu_seqlens=cu, name=f"ovl_rand{seed}_packed")
        a = _args(inp)[:6] + (cu.cuda(),)
        nseq, nslots, rows = 1, T // 64 + 2, T // 64 + 2
    else:
        inp = synth.prefill_basic(7100 + seed, B, T, H, HV, init=init, name=f"ovl_rand{seed}")
        a = _args(inp)
        nseq, nslots, rows = B, (B * T) // 64 + B + 1, (T + 63) // 64
    units = nseq * HV
    expect = _overlap_expected(units, rows, cus)
    say(f"random overlap case {inp.name}: B={B} T={T} H={H} HV={HV} units={units} rows={rows} "
        f"packed={packed} init={init} overlapped={expect}")
    need = kda.workspace_size(B, T, H, HV, nseq if packed else 0)
    fb = _flag_bytes(nslots, HV, nseq)
    assert need == nslots * HV * kda.PREFILL_SLOT_BYTES + fb
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    oo, so = kda.chunk_prefill_split(*a, workspace=ws)
    torch.cuda.synchronize()
    flags = ws[need - fb:].view(torch.int32)
    set_flags = int((flags[:nslots * HV] != 0).sum())
    gave_up = int((flags[nslots * HV:nslots * HV + units] != 0).sum())
    if expect:
        assert set_flags == nseq * ((T + 63) // 64) * HV, f"{inp.name}: {set_flags} slots flagged"
        assert gave_up == 0, f"{inp.name}: {gave_up} units gave up waiting"
    else:
        assert set_flags == 0 and gave_up == 0, f"{inp.name}: the overlapped schedule ran outside its range"
    ws2 = torch.zeros(need - fb, dtype=torch.uint8, device="cuda")
    os_, ss = kda.chunk_prefill_split(*a, workspace=ws2)
    of, sf = kda.chunk_prefill_fused(*a)
    torch.cuda.synchronize()
    assert torch.equal(_bits(oo), _bits(os_)) and torch.equal(so, ss), f"{inp.name}: schedules differ"
    assert torch.equal(_bits(oo), _bits(of)) and torch.equal(so, sf), f"{inp.name}: fused form differs"
    x = synth.to_numpy(inp)
    for hv in sorted(set(int(h) for h in rng.integers(0, HV, size=2))):
        hq = hv // group
        n = int(rng.integers(0, B))
        s0 = None if x["initial_state"] is None else x["initial_state"][n:n + 1, hv:hv + 1]
        o_ref, s_ref = oracle.recurrent(x["q"][n:n + 1, :, hq:hq + 1], x["k"][n:n + 1, :, hq:hq + 1],
                                        x["v"][n:n + 1, :, hv:hv + 1], x["g"][n:n + 1, :, hv:hv + 1],
                                        x["beta"][n:n + 1, :, hv:hv + 1], s0, x["cu_seqlens"])
        e_o = check_o(oo[n:n + 1, :, hv:hv + 1], o_ref, f"{inp.name} sequence {n} head {hv}")
        e_s = check_state(so[n:n + 1, hv:hv + 1], s_ref, f"{inp.name} sequence {n} head {hv}")
        say(f"  sequence {n}, value head {hv}: o_err={e_o:.2e} state_err={e_s:.2e}")
