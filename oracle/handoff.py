"""Prefill-to-decode handoff: states stored into the bf16 decode pool.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Sources:
  * "KDA Chunk Prefill on Ascend A3", section "Function and tensor
    contract": the prefill returns one fp32 final state [HV, K, V] per
    sequence.
  * "flashinfer.kda_decode.packed_kda_decode", section "Parameters": the
    decode keeps states in a bf16 pool [slots, HV, K, V], addressed by an
    int32 slot index per row, -1 meaning no state access.

Reading (the pages are silent here): handing a state to the decode stores it in
its slot rounded once to bf16, nearest-even -- the rounding the decode
itself applies when it writes a slot back.  An index outside
[0, slots) skips its state.
"""

import numpy as np

from .bf16 import bf16_round


def state_to_pool(state, pool, state_indices):
    """state [N,HV,K,V] (float32 values); pool float32 [slots,HV,K,V]
    holding bf16 values; state_indices int [N].

    Returns the new pool (float32 array of bf16 values); the input pool is
    not modified.
    """
    state = np.asarray(state, dtype=np.float32)
    new_pool = np.array(pool, dtype=np.float32, copy=True)
    slots = new_pool.shape[0]
    for n in range(state.shape[0]):
        idx = int(state_indices[n])
        if 0 <= idx < slots:
            new_pool[idx] = bf16_round(state[n])
    return new_pool
