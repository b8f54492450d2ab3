"""GPU parity of gdn_decode_fused: the conv of gdn_conv_update (decode mode), its conv
state commit and gdn_decode_batched in one launch must give the same bits as those two
calls in sequence, and match the oracle.

("System Design", "GDN Kernel Dispatch Detail", decode branch: conv state update, decay
and delta write, query against the state; aprender #5279, "Phase plan", P5: slot-batched
decode over a device u64[m] pointer array.)
"""

import numpy as np
import pytest

from gen import DECODE_30_LAYERS, make_decode_pool, make_decode_step
from gen.inputs import LayerShape
from oracle import decode_layer
from tests.gpu_helpers import TOL_BF16, TOL_F32, announce, bits_of, max_block_err_S, normwise_err, to_dev

pytestmark = pytest.mark.gpu


def _dims(shape, act=0):
    import gated_delta_rule_conv_amd as gdn

    return gdn.make_dims(shape.num_k_heads, shape.num_v_heads, shape.head_dim, conv_width=shape.conv_width,
                         chunk_size=shape.chunk, activation=act,
                         in_dtype=gdn.GDN_BF16 if shape.in_dtype == "bf16" else gdn.GDN_F32)


def _pool(gdn, dims, base, shape):
    return gdn.SlotPool(dims, base["pool"], state=to_dev(base["S"], "f32"),
                        conv_state=to_dev(base["conv_state"], shape.in_dtype))


# (Hk, Hv, d, in_dtype, K, activation, bias, m): both unit sizes (m * Hv >= 1024 takes
# one-pass units) and both load orders of the two-pass units (conv inputs first below
# m * Hv = 256), all head dims, both input dtypes, every conv width, SiLU and bias
CASES = [
    (16, 32, 128, "bf16", 4, 0, False, 40),
    (16, 32, 128, "bf16", 4, 1, True, 16),
    (2, 4, 64, "bf16", 3, 0, False, 100),
    (16, 32, 128, "bf16", 4, 0, False, 7),
    (4, 8, 128, "f32", 3, 1, True, 5),
    (2, 4, 64, "bf16", 2, 0, True, 300),
    (2, 4, 64, "f32", 4, 1, False, 6),
    (2, 2, 32, "bf16", 4, 0, False, 9),
    (1, 4, 32, "f32", 3, 0, True, 3),
]


@pytest.mark.parametrize("hk,hv,d,dt,K,act,bias,m", CASES)
def test_fused_equals_conv_then_decode_bit_for_bit(hk, hv, d, dt, K, act, bias, m):
    """Three consecutive steps on two copies of one pool: conv_update + decode on one,
    decode_fused on the other. o of every step, every slot's state and conv state (also
    the slots outside the call) must agree bit for bit, the counters must be zero after
    every call, and the fused result must match the oracle."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce(f"decode_fused vs conv+decode hk={hk} hv={hv} d={d} {dt} K={K} act={act} bias={bias} m={m}")
    shape = LayerShape(hk, hv, d, conv_width=K, in_dtype=dt)
    dims = _dims(shape, act)
    pool_slots = m + 5
    base = make_decode_pool(DECODE_30_LAYERS, pool=pool_slots, shape=shape, with_bias=bias)
    slots = [int(s) for s in base["perm"][:m]]
    idx = torch.tensor(slots, dtype=torch.int32, device="cuda")
    conv_w = to_dev(base["conv_w"], dt)
    conv_b = to_dev(base["conv_b"], dt) if bias else None
    pa, pb = _pool(gdn, dims, base, shape), _pool(gdn, dims, base, shape)
    spa, cpa = pa.pointers(idx)
    spb, cpb = pb.pointers(idx)
    counters = gdn.decode_counters(dims, m)
    ref_S = base["S"].astype(np.float64)[slots]
    ref_cs = base["conv_state"][slots]
    for step in range(3):
        inp = make_decode_step(DECODE_30_LAYERS, step, m, shape=shape)
        x, g, beta = to_dev(inp["x"], dt), to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32")
        y = torch.empty((m, shape.channels), dtype=torch.float32, device="cuda")
        oa = torch.empty((m, hv, d), dtype=torch.float32, device="cuda")
        ob = torch.full((m, hv, d), 7.0, dtype=torch.float32, device="cuda")
        gdn.conv_update(dims, x, y, conv_w, conv_b, cpa)
        gdn.decode(dims, y, g, beta, oa, spa)
        gdn.decode_fused(dims, x, conv_w, conv_b, g, beta, ob, spb, cpb, counters)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_of(oa), bits_of(ob))
        np.testing.assert_array_equal(bits_of(pa.state), bits_of(pb.state))
        np.testing.assert_array_equal(bits_of(pa.conv_state), bits_of(pb.conv_state))
        assert int(counters.abs().sum().item()) == 0, "counters must be left at zero"
        ref = decode_layer(inp["x"], base["conv_w"], ref_cs, ref_S, inp["g"], inp["beta"], hk, hv, d,
                           in_dtype=dt, conv_b=base["conv_b"], activation="silu" if act else "none")
        ref_S, ref_cs = ref["S"], ref["conv_state"]
        if dt == "bf16":
            from gen import bf16_bits_from_f32

            ref_cs = bf16_bits_from_f32(ref_cs.astype(np.float32))
        tol = TOL_BF16 if dt == "bf16" else TOL_F32
        o_host = ob.cpu().numpy()
        err_o = max(normwise_err(o_host[i, j], ref["o"][i, j]) for i in range(m) for j in range(hv))
        err_S = max_block_err_S(pb.state[slots].cpu().numpy(), ref_S)
        print(f"step {step}: max normwise err o={err_o:.3e} S={err_S:.3e} (tol {tol:g})")
        assert err_o <= tol and err_S <= tol
        cs_gpu = pb.conv_state[slots].cpu()
        cs_gpu = cs_gpu.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else cs_gpu.numpy()
        np.testing.assert_array_equal(cs_gpu, ref_cs.astype(cs_gpu.dtype))


def test_fused_inactive_slots_are_untouched():
    """A slot whose state pointer or conv-state pointer is 0 is skipped as a whole: its
    state, conv state and o rows keep their bits; the others equal conv + decode."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce("decode_fused inactive slots")
    shape = LayerShape(16, 32, 128, in_dtype="bf16")
    dims = _dims(shape)
    base = make_decode_pool(DECODE_30_LAYERS, pool=10, shape=shape)
    inp = make_decode_step(DECODE_30_LAYERS, 4, 6, shape=shape)
    slots = [3, 8, 1, 5, 0, 9]
    x, g, beta = to_dev(inp["x"], "bf16"), to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32")
    conv_w = to_dev(base["conv_w"], "bf16")
    pa, pb = _pool(gdn, dims, base, shape), _pool(gdn, dims, base, shape)
    idx = torch.tensor(slots, dtype=torch.int32, device="cuda")
    spa, cpa = pa.pointers(idx)
    spb, cpb = pb.pointers(idx)
    # entry 1: no state pointer; entry 4: no conv-state pointer
    spb[1] = 0
    cpb[4] = 0
    live = [0, 2, 3, 5]
    spa_live = spa[live].contiguous()
    cpa_live = cpa[live].contiguous()
    y = torch.empty((4, shape.channels), dtype=torch.float32, device="cuda")
    oa = torch.empty((4, 32, 128), dtype=torch.float32, device="cuda")
    gdn.conv_update(dims, x[live].contiguous(), y, conv_w, None, cpa_live)
    gdn.decode(dims, y, g[live].contiguous(), beta[live].contiguous(), oa, spa_live)
    ob = torch.full((6, 32, 128), -5.0, dtype=torch.float32, device="cuda")
    counters = gdn.decode_counters(dims, 6)
    gdn.decode_fused(dims, x, conv_w, None, g, beta, ob, spb, cpb, counters)
    torch.cuda.synchronize()
    assert torch.all(ob[1] == -5.0) and torch.all(ob[4] == -5.0)
    np.testing.assert_array_equal(bits_of(oa), bits_of(ob[live]))
    np.testing.assert_array_equal(bits_of(pa.state), bits_of(pb.state))
    np.testing.assert_array_equal(bits_of(pa.conv_state), bits_of(pb.conv_state))
    for s in (slots[1], slots[4]):
        np.testing.assert_array_equal(bits_of(pb.state[s]), bits_of(to_dev(base["S"][s], "f32")))
        np.testing.assert_array_equal(bits_of(pb.conv_state[s]), bits_of(to_dev(base["conv_state"][s], "bf16")))
    assert int(counters.abs().sum().item()) == 0


def test_fused_graph_replay_matches_eager():
    """Two layers of decode_fused sharing one counter workspace, captured in a HIP graph
    and replayed three times with eager work between replays: each replay equals the
    eager step bit for bit, and the counters stay zero."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce("decode_fused graph replay vs eager")
    shape = LayerShape(16, 32, 128, in_dtype="bf16")
    dims = _dims(shape)
    layers, pool_slots, m = 2, 40, 36
    base = [make_decode_pool(DECODE_30_LAYERS, pool=pool_slots, shape=shape) for _ in range(layers)]
    idx = torch.tensor([int(s) for s in base[0]["perm"][:m]], dtype=torch.int32, device="cuda")
    inp = make_decode_step(DECODE_30_LAYERS, 11, m, shape=shape)
    x, g, beta = to_dev(inp["x"], "bf16"), to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32")

    def rig():
        pools = [_pool(gdn, dims, b, shape) for b in base]
        ptrs = [p.pointers(idx) for p in pools]
        ws = [to_dev(b["conv_w"], "bf16") for b in base]
        o = torch.empty((layers, m, 32, 128), dtype=torch.float32, device="cuda")
        counters = gdn.decode_counters(dims, m)

        def step():
            for layer in range(layers):
                sp, cp = ptrs[layer]
                gdn.decode_fused(dims, x, ws[layer], None, g, beta, o[layer], sp, cp, counters)
        return pools, o, counters, step

    pools_g, o_g, c_g, step_g = rig()
    pools_e, o_e, c_e, step_e = rig()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step_g()
    torch.cuda.synchronize()
    for rep in range(3):
        graph.replay()
        step_e()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_of(o_g), bits_of(o_e))
        for pg, pe in zip(pools_g, pools_e):
            np.testing.assert_array_equal(bits_of(pg.state), bits_of(pe.state))
            np.testing.assert_array_equal(bits_of(pg.conv_state), bits_of(pe.conv_state))
        assert int(c_g.abs().sum().item()) == 0 and int(c_e.abs().sum().item()) == 0
