"""Writes tests/golden/tiny_fp32_oracle.json: the oracle's outputs on the tiny fp32
workload (1 sequence, L = 64, 2 heads, d = 32, zero states), sampled.

Calls only oracle/ and gen/. Rerun only when a reading of the method changes, and
name that reading in the commit that changes the fixture."""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from gen import TINY_FP32, make_prefill  # noqa: E402
from oracle import prefill_layer  # noqa: E402

TOKENS = [0, 1, 15, 16, 17, 40, 63]


def compute():
    inp = make_prefill(TINY_FP32)
    sh = inp["shape"]
    out = prefill_layer(inp["x"], inp["conv_w"], inp["cu_seqlens"], inp["conv_state"], inp["S0"], inp["g"],
                        inp["beta"], sh.num_k_heads, sh.num_v_heads, sh.head_dim, in_dtype="f32")
    return {
        "workload": "tiny fp32: L=64, Hk=Hv=2, d=32, conv width 4, zero initial states, identity activation",
        "tokens": TOKENS,
        "o": [[[float(x) for x in out["o"][t, h]] for h in range(2)] for t in TOKENS],
        "S_row0": [[float(x) for x in out["S"][0, h, 0]] for h in range(2)],
        "S_sum": [float(out["S"][0, h].sum()) for h in range(2)],
        "o_abs_sum": float(np.abs(out["o"]).sum()),
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_fp32_oracle.json"), "w") as f:
        json.dump(compute(), f, indent=1)
