"""kda_qk_l2norm on the GPU against the oracle's canonical normalisation:
bit-exact on every workload's q and k and on crafted rows."""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.bf16 import bf16_bits
from gpu_util import say

pytestmark = pytest.mark.gpu


def _gpu_bits(kda, x_bf16):
    y = kda.qk_l2norm(x_bf16.cuda())
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle_bits(x_bf16):
    return bf16_bits(oracle.l2norm_bf16(x_bf16.float().numpy()))


def _compare(kda, x, what):
    say(f"l2norm {what} rows={x.numel() // 128}")
    got = _gpu_bits(kda, x)
    ref = _oracle_bits(x)
    bad = np.count_nonzero(got != ref)
    assert bad == 0, f"{what}: {bad} of {ref.size} bf16 values differ"


@pytest.mark.parametrize("which", ["cfg0", "cfg1", "cfg3"])
def test_l2norm_workloads(gpu_lib, which):
    inp = {"cfg0": synth.config0, "cfg1": synth.config1, "cfg3": synth.config3}[which]()
    _compare(gpu_lib, inp.q, which + ".q")
    _compare(gpu_lib, inp.k, which + ".k")


def test_l2norm_full_scale_q(gpu_lib):
    inp = synth.config2()
    _compare(gpu_lib, inp.q, "cfg2.q")
    _compare(gpu_lib, inp.k[:, :2048], "cfg2.k[:2048]")


@pytest.mark.parametrize("mode", ["gain", "tiny", "zero_rows"])
def test_l2norm_stress(gpu_lib, mode):
    inp = synth.prefill_stress(21, 2, 333, 4, 4, qk_mode=mode)
    _compare(gpu_lib, inp.q, mode + ".q")
    _compare(gpu_lib, inp.k, mode + ".k")


def test_l2norm_crafted_rows(gpu_lib):
    rng = np.random.default_rng(7)
    rows = []
    e0 = np.zeros(128, np.float32)
    e0[0] = 1
    rows += [e0, -e0, np.zeros(128, np.float32), np.full(128, 3.0, np.float32)]
    for span in (10, 15, 16, 17, 30, 38, 60, 120):     # straddles the exact float64 window
        for _ in range(6):
            r = rng.standard_normal(128) * np.exp2(rng.integers(-span // 2, span // 2 + 1, 128))
            rows.append(r.astype(np.float32))
    sub = np.zeros(128, np.float32)                     # bf16 subnormal magnitudes
    sub[:5] = [1e-39, -2e-39, 5e-40, 3e-39, 1e-38]
    rows.append(sub)
    for tiny_val in (1e-39, -3e-39, 5e-40, 2e-38, 1e-40):   # quotients below float32's normal range
        r = np.zeros(128, np.float32)
        r[0] = 1.0
        r[1:6] = tiny_val * np.arange(1, 6)
        rows.append(r)
    big = (rng.standard_normal(128) * 1e18).astype(np.float32)
    rows.append(big)
    tiny = (rng.standard_normal(128) * 1e-5).astype(np.float32)
    rows.append(tiny)
    x = torch.from_numpy(np.stack(rows)).to(torch.bfloat16)
    x = torch.cat([x, x.flip(0)])        # different row positions within a wave
    _compare(gpu_lib, x, "crafted")


def test_l2norm_odd_row_counts(gpu_lib):
    for rows in (1, 3, 15, 17, 1000):
        x = torch.randn(rows, 128, generator=torch.Generator().manual_seed(rows)).to(torch.bfloat16)
        _compare(gpu_lib, x, f"rows{rows}")
