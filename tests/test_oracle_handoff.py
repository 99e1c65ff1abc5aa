"""Pins for the oracle's prefill-to-decode handoff (state_to_pool).

Rounding is pinned by values worked out by hand (ties to even at both
parities, overflow to infinity, the subnormal range) and against torch's own
float32 -> bfloat16 conversion, an independent round-to-nearest-even
implementation; the slot logic by an explicit layout of active, inactive and
out-of-range indices.
"""

import numpy as np
import torch

import oracle
from oracle.bf16 import bits_to_f32


def f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


def test_hand_worked_roundings():
    # (float32 bit pattern in, bf16 bit pattern out), each derived by hand:
    cases = [
        (0x3F808000, 0x3F80),   # 1 + 2^-8: midway between 1 and 1 + 2^-7 -> even (1)
        (0x3F818000, 0x3F82),   # 1 + 3*2^-8: midway, odd below -> rounds up to 1 + 2^-6
        (0x3F808001, 0x3F81),   # just above the midway point -> up
        (0x3F807FFF, 0x3F80),   # just below -> down
        (0xBF808000, 0xBF80),   # negative midway -> even, sign kept
        (0x7F7FFFFF, 0x7F80),   # largest float32 is beyond the largest bf16 + half a step -> inf
        (0x7F800000, 0x7F80),   # inf stays inf
        (0x00000001, 0x0000),   # 2^-149 is far below half of bf16's smallest subnormal 2^-133
        (0x00018000, 0x0002),   # 1.5 * 2^-133: midway between 2^-133 (odd) and 2^-132 -> 2^-132
        (0x00010000, 0x0001),   # 2^-133 itself is exact
        (0x80000000, 0x8000),   # -0 stays -0
    ]
    x = f32([c[0] for c in cases]).reshape(len(cases), 1, 1, 1)
    pool = np.zeros((len(cases), 1, 1, 1), np.float32)
    got = oracle.state_to_pool(x, pool, np.arange(len(cases)))
    want = bits_to_f32(np.array([c[1] for c in cases], np.uint16))
    np.testing.assert_array_equal(got.reshape(-1).view(np.uint32), want.view(np.uint32))


def test_nan_stays_nan():
    x = f32([0x7FC00000, 0xFF800001, 0x7F800001]).reshape(3, 1, 1, 1)
    got = oracle.state_to_pool(x, np.zeros((3, 1, 1, 1), np.float32), np.arange(3))
    assert np.all(np.isnan(got))


def test_matches_torch_bf16_conversion():
    rng = np.random.default_rng(11)
    # the pages' nonzero state: standard normal times 0.25, plus a wide spread of scales
    s = (0.25 * rng.standard_normal((3, 2, 16, 16))).astype(np.float32)
    s[2] *= np.float32(2.0) ** rng.integers(-140, 120, s[2].shape).astype(np.float32)
    got = oracle.state_to_pool(s, np.zeros_like(s), np.arange(3))
    ref = torch.from_numpy(s).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_slot_layout_and_untouched_slots():
    rng = np.random.default_rng(12)
    s = rng.standard_normal((5, 2, 4, 4)).astype(np.float32)
    pool = torch.from_numpy(rng.standard_normal((6, 2, 4, 4)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    idx = np.array([3, -1, 0, 7, 5], np.int32)       # 7 >= 6 slots: skipped like -1
    got = oracle.state_to_pool(s, pool, idx)
    r = torch.from_numpy(s).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(got[3], r[0])
    np.testing.assert_array_equal(got[0], r[2])
    np.testing.assert_array_equal(got[5], r[4])
    np.testing.assert_array_equal(got[[1, 2, 4]], pool[[1, 2, 4]])
    # the input pool is not modified
    assert not np.array_equal(pool[3], r[0])


def test_bf16_states_pass_unchanged():
    rng = np.random.default_rng(13)
    s = torch.from_numpy(rng.standard_normal((2, 3, 8, 8)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    got = oracle.state_to_pool(s, np.zeros((4, 3, 8, 8), np.float32), np.array([1, 2]))
    np.testing.assert_array_equal(got[1:3], s)
