"""fp64 CPU oracle for the Gated DeltaNet layer core.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
anything in this package; only the tests, the smoke check and the benchmark's
CPU-baseline leg do. It shares no code with the HIP library.

Contents (``oracle.gdn``):
  causal_conv            depthwise causal conv1d with a per-sequence conv state
  l2norm                 per-head L2 normalisation
  gated_delta_recurrent  the token-by-token gated delta rule (the definition)
  gated_delta_chunked    the chunked (WY / UT) rewrite, used only to show that
                         chunked == recurrent and to debug chunk intermediates
  prefill_layer / decode_layer   the whole path for packed ragged sequences and
                         for one decode token per slot

Every function is pinned by CPU tests (tests/test_oracle_*.py) to closed forms,
library routines, invariants, exact rational arithmetic or brute force.
No function here is "parity unpinned".
"""

from .gdn import (  # noqa: F401
    bf16_bits_to_f64,
    causal_conv,
    decode_layer,
    gated_delta_chunked,
    gated_delta_recurrent,
    l2norm,
    prefill_layer,
    split_qkv,
    storage_to_f64,
)
