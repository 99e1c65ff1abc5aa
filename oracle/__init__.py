"""CPU fp64 oracle for the Kimi Delta Attention (KDA) forward path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call,
link or execute this package: only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library under ``kda_gated_delta_amd``; the two meet only through the seeded
input generators in ``synth``, which hold none of the method's arithmetic.

Sources (titles of the pages the method is specified on):
  * "KDA Chunk Prefill on Ascend A3" -- section "Mathematical definition"
    (Q/K normalisation, recurrent semantics, chunk construction) and the
    section "Example" (worked example and the beta = 0 case).
  * "flashinfer.kda_decode.packed_kda_decode" -- section "Parameters"
    (bf16 state pool, -1 slot indices, in-place update).

Modules
  bf16       exact bf16 <-> float conversions with round-to-nearest-even
  l2norm     the canonical bit-exact Q/K L2 normalisation
  recurrent  the token-by-token recurrence, fp64
  chunked    the chunk construction (G, L, A, W, U, Qg, Kg, Aqk, carry), fp64
  decode     one recurrent step against a bf16 state pool
  handoff    prefill final states stored into the bf16 decode pool
  packed_decode  the decode step from packed QKV and raw gate/beta logits
  backward   gradients of the forward by float64 autodiff of the recurrence

Pinning status: every public function here is pinned by tests that do not
re-type its formula (closed forms, the pages' worked example, invariants,
brute force against exact rational arithmetic, and the two independent
forms checked against each other).  See tests/test_oracle_*.py.  The one
exception is the packed decode's gate transform, whose formula the pages do
not give: "parity unpinned" -- only its closed-form properties are pinned.
"""

from .bf16 import bf16_round, bf16_bits, bits_to_f32, f64_to_bf16_round
from .l2norm import l2norm_bf16
from .recurrent import recurrent
from .chunked import chunked
from .decode import decode_step
from .handoff import state_to_pool
from .packed_decode import packed_decode_step
from .backward import recurrent_backward

__all__ = [
    "bf16_round",
    "bf16_bits",
    "bits_to_f32",
    "f64_to_bf16_round",
    "l2norm_bf16",
    "recurrent",
    "chunked",
    "decode_step",
    "state_to_pool",
    "packed_decode_step",
    "recurrent_backward",
]
