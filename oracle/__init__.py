"""CPU oracle of the batch-1 decode step.

TEST INFRASTRUCTURE.  This package is the slow, plain reference the GPU path
is checked against.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run it; the product path never does, and it
shares no code with the GPU library (the seeded input generators in ``synth``
are the one common dependency).

Every function is written from the plain definition of the operation; see
each docstring for the passage it follows and the reading taken where the
pages are silent.  Pins (tests that fix the oracle to something other than
itself) live in ``tests/test_oracle_*.py``.

Parity unpinned: no page prints reference logits for any model, so
end-to-end logits of a whole decode step are fixed only by the pinned parts,
a naive loop re-implementation on tiny shapes and the float32/float64
agreement check.
"""
from . import codecs  # noqa: F401
from .decode import (OracleCache, OracleModel, argmax_lower_index, attention,  # noqa: F401
                     quantize_fp8_rows, dequant_fp8_rows, rmsnorm, rope, route,
                     softmax, swiglu, topk_lower_index)
