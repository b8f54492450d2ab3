"""Prefill captured in a HIP graph: each replay continues the recurrence from the state
the previous one left (like back-to-back eager calls), so replay i must give the bits of
the (i+1)-th eager call, with the program's own eager work and synchronisations between
replays. Both entry points (conv_update + prefill_chunked, and prefill_fused), on a
ragged pack of sequences with nonzero initial and conv states."""

import numpy as np
import pytest

from gen import RAGGED_T15717, make_prefill
from gen.inputs import LayerShape
from tests.gpu_helpers import announce, bits_of, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _rig(inp, fused):
    import torch

    import gated_delta_rule_conv_amd as gdn

    sh = inp["shape"]
    dims = gdn.make_dims(sh.num_k_heads, sh.num_v_heads, sh.head_dim, conv_width=sh.conv_width,
                         chunk_size=sh.chunk, activation=gdn.GDN_ACT_SILU, in_dtype=gdn.GDN_BF16)
    N, T = len(inp["lens"]), int(inp["cu_seqlens"][-1])
    r = dict(dims=dims, fused=fused)
    r["cu"] = torch.tensor(inp["cu_seqlens"], dtype=torch.int32, device="cuda")
    r["x"] = to_dev(inp["x"], "bf16")
    r["w"] = to_dev(inp["conv_w"], "bf16")
    r["g"], r["beta"] = to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32")
    r["pool"] = gdn.SlotPool(dims, N, state=to_dev(inp["S0"], "f32"), conv_state=to_dev(inp["conv_state"], "bf16"))
    r["sp"], r["cp"] = r["pool"].pointers(torch.arange(N, dtype=torch.int32, device="cuda"))
    r["o"] = torch.empty((T, sh.num_v_heads, sh.head_dim), dtype=torch.float32, device="cuda")
    if fused:
        r["ws"] = gdn.prefill_fused_workspace(dims, N, T)
    else:
        r["y"] = torch.empty((T, sh.channels), dtype=torch.float32, device="cuda")
        r["ws"] = gdn.prefill_workspace(dims, N, T)
    return r


def _call(r):
    import gated_delta_rule_conv_amd as gdn

    if r["fused"]:
        gdn.prefill_fused(r["dims"], r["x"], r["w"], None, r["g"], r["beta"], r["o"], r["cu"], r["sp"], r["cp"],
                          r["ws"])
    else:
        gdn.conv_update(r["dims"], r["x"], r["y"], r["w"], None, r["cp"], r["cu"])
        gdn.prefill(r["dims"], r["y"], r["g"], r["beta"], r["o"], r["cu"], r["sp"], r["ws"])


def _snap(r):
    return bits_of(r["o"]), bits_of(r["pool"].state), bits_of(r["pool"].conv_state)


@pytest.mark.parametrize("fused", [False, True])
def test_prefill_graph_replays_match_eager_calls(fused):
    import torch

    announce(f"prefill graph replay x{REPLAYS} vs eager ({'fused' if fused else 'two calls'})")
    shape = LayerShape(2, 4, 128, conv_width=4, chunk=64, in_dtype="bf16")
    inp = make_prefill(RAGGED_T15717, lens=(1, 70, 300, 129, 5), shape=shape, s0_std=0.05, conv_state_std=1.0)
    eager = _rig(inp, fused)
    want = []
    for _ in range(REPLAYS):
        _call(eager)
        torch.cuda.synchronize()
        want.append(_snap(eager))

    rep = _rig(inp, fused)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()  # (capturing does not run the kernels)
    with torch.cuda.graph(graph):
        _call(rep)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        graph.replay()
        torch.cuda.synchronize()
        # eager work of the program's own between replays
        scratch = torch.empty(1 << 20, dtype=torch.float32, device="cuda").fill_(float(i))
        assert float(scratch[-1].item()) == float(i)
        got = _snap(rep)
        for a, b in zip(got, want[i]):
            np.testing.assert_array_equal(a, b)
