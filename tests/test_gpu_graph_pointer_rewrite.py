"""The 30-layer decode step captured once in a HIP graph and replayed with its device
pointer arrays rewritten in place between replays.

The graph holds the addresses of the per-layer slot-pointer arrays, not their contents, so
a serving loop can move the step to another set of slots by rewriting those arrays
(gdn_slot_pointers, outside the graph) and replaying, without capturing again (aprender
#5279, "Phase plan", phase P8: graph replay keyed by the slot-pointer arrays, equal to the
eager result; the "qLLM" page's "Results": graph decode matching eager decode). Every
replay here runs on a different slot set, some entries inactive (address 0), with fresh
inputs copied into the captured input buffers; each replay is checked against the oracle
for every (slot, v-head) of every layer, inactive entries must leave their o rows alone,
and slots outside the set must keep their bits. Every step form is captured: 30 x
(gdn_conv_update + gdn_decode_batched), 30 x gdn_decode_fused in place, and 30 x
gdn_decode_fused streaming the conv states between two pools (one graph per direction,
replayed in turn).
"""

import numpy as np
import pytest

from gen import bf16_bits_from_f32
from gen.inputs import DECODE_30_LAYERS, WORKLOADS, make_decode_pool_torch
from oracle import decode_layer
from tests.gpu_helpers import TOL_BF16, announce, bits_of, max_block_err_S, normwise_err, storage_of

pytestmark = pytest.mark.gpu

LAYERS, POOL, M = 30, 12, 6
# slot index per pointer-array entry, one set per replay; -1 gives address 0 (inactive)
SLOT_SETS = [
    [3, 7, 0, 11, 5, 9],
    [2, -1, 8, 3, -1, 10],
    [11, 10, 9, 1, 4, 6],
    [-1, 0, -1, -1, 7, -1],
]
SENTINEL = -7.0


@pytest.mark.parametrize("form", ["two_calls", "fused", "fused_stream"])
def test_graph_replay_with_rewritten_pointer_arrays_matches_oracle(form):
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce(f"graph replay, pointer arrays rewritten between replays, {LAYERS} layers, {form}")
    fused, stream = form != "two_calls", form == "fused_stream"
    sh = WORKLOADS[DECODE_30_LAYERS].shape
    Hk, Hv, d, C = sh.num_k_heads, sh.num_v_heads, sh.head_dim, sh.channels
    dims = gdn.make_dims(Hk, Hv, d, conv_width=sh.conv_width, chunk_size=sh.chunk, in_dtype=gdn.GDN_BF16)
    states, conv_states, conv_w = make_decode_pool_torch(DECODE_30_LAYERS, POOL, LAYERS, "cuda")
    conv_b = conv_states.clone()  # the streaming form's second conv pool
    s_bytes = states[0, 0].numel() * 4
    c_bytes = conv_states[0, 0].numel() * conv_states.element_size()

    # buffers the graph captures by address
    idx = torch.empty((M,), dtype=torch.int32, device="cuda")
    sptr = torch.empty((LAYERS, M), dtype=torch.int64, device="cuda")
    cptr = torch.empty((LAYERS, M), dtype=torch.int64, device="cuda")
    cptr_b = torch.empty((LAYERS, M), dtype=torch.int64, device="cuda")
    x = torch.empty((LAYERS, M, C), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((LAYERS, M, Hv), dtype=torch.float32, device="cuda")
    beta = torch.empty((LAYERS, M, Hv), dtype=torch.float32, device="cuda")
    y = torch.empty((M, C), dtype=torch.float32, device="cuda")
    o = torch.empty((LAYERS, M, Hv, d), dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5100 + int(fused))

    def point_at(slots):
        """Rewrite the captured pointer arrays in place for this slot set."""
        idx.copy_(torch.tensor(slots, dtype=torch.int32))
        for layer in range(LAYERS):
            gdn.gdn_slot_pointers(states[layer].data_ptr(), s_bytes, POOL, idx, M, sptr[layer])
            gdn.gdn_slot_pointers(conv_states[layer].data_ptr(), c_bytes, POOL, idx, M, cptr[layer])
            gdn.gdn_slot_pointers(conv_b[layer].data_ptr(), c_bytes, POOL, idx, M, cptr_b[layer])

    def fresh_inputs():
        x.copy_(torch.randn((LAYERS, M, C), generator=gen, device="cuda").to(torch.bfloat16))
        g.copy_(-torch.nn.functional.softplus(torch.randn((LAYERS, M, Hv), generator=gen, device="cuda")))
        beta.copy_(torch.sigmoid(torch.randn((LAYERS, M, Hv), generator=gen, device="cuda")))

    def step(direction=0):
        for layer in range(LAYERS):
            if stream:
                cin, cout = (cptr, cptr_b) if direction == 0 else (cptr_b, cptr)
                gdn.decode_fused(dims, x[layer], conv_w[layer], None, g[layer], beta[layer], o[layer], sptr[layer],
                                 cin[layer], cout[layer])
            elif fused:
                gdn.decode_fused(dims, x[layer], conv_w[layer], None, g[layer], beta[layer], o[layer], sptr[layer],
                                 cptr[layer])
            else:
                gdn.conv_update(dims, x[layer], y, conv_w[layer], None, cptr[layer])
                gdn.decode(dims, y, g[layer], beta[layer], o[layer], sptr[layer])

    # capture once, on a slot set whose results are thrown away (a copy of the pools is
    # restored afterwards, so the captured warm-up leaves no trace)
    keep_s, keep_c, keep_b = states.clone(), conv_states.clone(), conv_b.clone()
    point_at(SLOT_SETS[0])
    fresh_inputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
        if stream:
            step(1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for direction in range(2 if stream else 1):  # (streaming: pool A -> B, then B -> A)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(direction)
        graphs.append(graph)
    torch.cuda.synchronize()
    states.copy_(keep_s)
    conv_states.copy_(keep_c)
    conv_b.copy_(keep_b)
    del keep_s, keep_c, keep_b
    torch.cuda.synchronize()

    worst_o = worst_S = 0.0
    for rep, slots in enumerate(SLOT_SETS):
        point_at(slots)  # eager work between replays: the arrays change, the graph does not
        fresh_inputs()
        o.fill_(SENTINEL)
        act = [r for r, s in enumerate(slots) if 0 <= s < POOL]
        live = [slots[r] for r in act]
        rest = [s for s in range(POOL) if s not in live]
        torch.cuda.synchronize()
        # where this replay reads the conv states from and writes them to
        cs_in, cs_out = conv_states, conv_states
        if stream:
            cs_in, cs_out = (conv_states, conv_b) if rep % 2 == 0 else (conv_b, conv_states)
        S_before = states[:, live].cpu().numpy()
        cs_before = storage_of(cs_in[:, live], "bf16")
        in_bits = bits_of(cs_in) if stream else None
        rest_bits = (bits_of(states[:, rest]), bits_of(cs_out[:, rest]))
        graphs[rep % len(graphs)].replay()
        torch.cuda.synchronize()
        og = o.cpu().numpy()
        S_after = states[:, live].cpu().numpy()
        cs_after = storage_of(cs_out[:, live], "bf16")
        if stream:
            np.testing.assert_array_equal(bits_of(cs_in), in_bits, err_msg=f"replay {rep}: input conv pool written")
        for layer in range(LAYERS):
            ref = decode_layer(storage_of(x[layer, act], "bf16"), storage_of(conv_w[layer], "bf16"), cs_before[layer],
                               S_before[layer].astype(np.float64), g[layer, act].cpu().numpy(),
                               beta[layer, act].cpu().numpy(), Hk, Hv, d, in_dtype="bf16")
            for i, r in enumerate(act):
                for j in range(Hv):
                    worst_o = max(worst_o, normwise_err(og[layer, r, j], ref["o"][i, j]))
            worst_S = max(worst_S, max_block_err_S(S_after[layer], ref["S"]))
            np.testing.assert_array_equal(cs_after[layer], bf16_bits_from_f32(ref["conv_state"].astype(np.float32)),
                                          err_msg=f"replay {rep} layer {layer}: conv state")
        inactive = [r for r in range(M) if r not in act]
        assert np.all(og[:, inactive] == SENTINEL), f"replay {rep}: an inactive entry wrote o"
        np.testing.assert_array_equal(bits_of(states[:, rest]), rest_bits[0], err_msg=f"replay {rep}: idle state")
        np.testing.assert_array_equal(bits_of(cs_out[:, rest]), rest_bits[1],
                                      err_msg=f"replay {rep}: idle conv state")
        print(f"replay {rep} slots {slots}: max normwise err so far o={worst_o:.3e} S={worst_S:.3e}")
        assert worst_o <= TOL_BF16 and worst_S <= TOL_BF16, (rep, worst_o, worst_S)
