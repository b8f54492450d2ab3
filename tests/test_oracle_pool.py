"""The sharded oracle run (one job per k-head group, in worker processes) gives what one
oracle call over the whole layer gives: the slicing of channels, heads and states into
groups and back is pure bookkeeping."""

import numpy as np

from gen import RAGGED_T15717, make_prefill
from gen.inputs import LayerShape
from oracle import prefill_layer
from tests.oracle_pool import prefill_all_heads


def test_sharded_oracle_equals_whole_layer_call():
    shape = LayerShape(3, 6, 8, conv_width=4, chunk=16, in_dtype="bf16")
    inp = make_prefill(RAGGED_T15717, lens=(5, 21, 1, 9), shape=shape, s0_std=0.1, conv_state_std=1.0,
                       with_bias=True)
    kw = dict(activation="silu", scale=0.5)
    whole = prefill_layer(inp["x"], inp["conv_w"], inp["cu_seqlens"], inp["conv_state"], inp["S0"], inp["g"],
                          inp["beta"], 3, 6, 8, conv_b=inp["conv_b"], in_dtype="bf16", **kw)
    for procs in (1, 2):
        part = prefill_all_heads(inp, procs=procs, **kw)
        for key in ("o", "S", "conv_state"):
            np.testing.assert_allclose(part[key], whole[key], rtol=1e-14, atol=1e-15, err_msg=key)
        assert np.abs(part["o"]).max() > 0.05
