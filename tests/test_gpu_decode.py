"""GPU parity of the decode path (gdn_conv_update in decode mode + gdn_decode_batched)
against the oracle, plus the batching and routing contracts.

("System Design", "GDN Kernel Dispatch Detail", decode branch; aprender #5279, "Phase
plan", P5: slot-batched conv and delta rule over a device u64[m] pointer array, bitwise
equal to the per-slot result; "qLLM", "What this is": fixed-size slot pool.)
"""

import numpy as np
import pytest

from gen import DECODE_M16_POOL64, make_decode_pool, make_decode_step
from gen.inputs import LayerShape
from oracle import decode_layer
from tests.gpu_helpers import (TOL_BF16, TOL_F32, announce, bits_of, max_block_err_S, normwise_err,
                               storage_of, to_dev)

pytestmark = pytest.mark.gpu


def _dims(shape, act=0):
    import gated_delta_rule_conv_amd as gdn

    return gdn.make_dims(shape.num_k_heads, shape.num_v_heads, shape.head_dim, conv_width=shape.conv_width,
                         chunk_size=shape.chunk, activation=act,
                         in_dtype=gdn.GDN_BF16 if shape.in_dtype == "bf16" else gdn.GDN_F32)


class DecodeRig:
    """A slot pool on the device plus the oracle's copy of every slot."""

    def __init__(self, wid, shape, pool_slots, act=0):
        import gated_delta_rule_conv_amd as gdn

        self.wid, self.shape, self.act = wid, shape, act
        self.dims = _dims(shape, act)
        self.np = make_decode_pool(wid, pool=pool_slots, shape=shape)
        self.pool = gdn.SlotPool(self.dims, pool_slots, state=to_dev(self.np["S"], "f32"),
                                 conv_state=to_dev(self.np["conv_state"], shape.in_dtype))
        self.conv_w = to_dev(self.np["conv_w"], shape.in_dtype)
        self.ref_S = self.np["S"].astype(np.float64)
        self.ref_cs = self.np["conv_state"].copy()

    def gpu_step(self, step, slots):
        import torch

        import gated_delta_rule_conv_amd as gdn

        m = len(slots)
        inp = make_decode_step(self.wid, step, m, shape=self.shape)
        sp, cp = self.pool.pointers(torch.tensor(slots, dtype=torch.int32, device="cuda"))
        x = to_dev(inp["x"], self.shape.in_dtype)
        y = torch.empty((m, self.shape.channels), dtype=torch.float32, device="cuda")
        o = torch.zeros((m, self.shape.num_v_heads, self.shape.head_dim), dtype=torch.float32, device="cuda")
        gdn.conv_update(self.dims, x, y, self.conv_w, None, cp)
        gdn.decode(self.dims, y, to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32"), o, sp)
        return inp, o

    def oracle_step(self, inp, slots):
        sh = self.shape
        out = decode_layer(inp["x"], self.np["conv_w"], self.ref_cs[slots], self.ref_S[slots], inp["g"],
                           inp["beta"], sh.num_k_heads, sh.num_v_heads, sh.head_dim, in_dtype=sh.in_dtype,
                           activation="silu" if self.act else "none")
        self.ref_S[slots] = out["S"]
        cs = out["conv_state"]
        if sh.in_dtype == "bf16":
            from gen import bf16_bits_from_f32

            cs = bf16_bits_from_f32(cs.astype(np.float32))
        self.ref_cs[slots] = cs
        return out["o"]


def test_decode_m16_pool64_64_steps_matches_oracle():
    """16 active slots of a 64-slot pool, pointer array in shuffled slot order, 64 steps,
    bf16 inputs, fp32 state. Every step's o, the final states and conv states."""
    import torch

    announce("decode m=16 pool=64 steps=64")
    shape = LayerShape(16, 32, 128, in_dtype="bf16")
    rig = DecodeRig(DECODE_M16_POOL64, shape, 64)
    slots = [int(s) for s in rig.np["perm"][:16]]
    worst_o = 0.0
    for step in range(64):
        inp, o = rig.gpu_step(step, slots)
        o_ref = rig.oracle_step(inp, slots)
        og = o.cpu().numpy()
        for i in range(16):
            for j in range(shape.num_v_heads):
                worst_o = max(worst_o, normwise_err(og[i, j], o_ref[i, j]))
    torch.cuda.synchronize()
    S = rig.pool.state.cpu().numpy()
    err_S = max_block_err_S(S[slots], rig.ref_S[slots])
    print(f"decode m=16 x 64 steps: max normwise err o={worst_o:.3e} S={err_S:.3e}")
    assert worst_o <= TOL_BF16 and err_S <= TOL_BF16
    np.testing.assert_array_equal(storage_of(rig.pool.conv_state, "bf16")[slots], rig.ref_cs[slots])
    # inactive slots never touched
    rest = [s for s in range(64) if s not in slots]
    np.testing.assert_array_equal(S[rest], rig.np["S"][rest])


@pytest.mark.parametrize("d,in_dtype,hk,hv", [(32, "f32", 2, 2), (64, "f32", 2, 4), (128, "f32", 4, 8),
                                              (64, "bf16", 1, 3)])
def test_decode_head_dims_match_oracle(d, in_dtype, hk, hv):
    announce(f"decode d={d} {in_dtype} hk={hk} hv={hv}")
    shape = LayerShape(hk, hv, d, in_dtype=in_dtype)
    for act in (0, 1):
        rig = DecodeRig(DECODE_M16_POOL64, shape, 9, act=act)
        slots = [3, 8, 0, 5]
        for step in range(5):
            inp, o = rig.gpu_step(step, slots)
            o_ref = rig.oracle_step(inp, slots)
            og = o.cpu().numpy()
            tol = TOL_F32 if in_dtype == "f32" else TOL_BF16
            for i in range(len(slots)):
                for j in range(hv):
                    assert normwise_err(og[i, j], o_ref[i, j]) <= tol
        S = rig.pool.state.cpu().numpy()
        assert max_block_err_S(S[slots], rig.ref_S[slots]) <= tol


def test_batched_is_bit_exact_against_m1_and_routing():
    """m = 16 in one call == 16 calls at m = 1 == the same slots in another pointer order,
    bit for bit (o, state, conv state); slots outside the call keep their bits."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce("decode bit-exact m=16 vs m=1 vs shuffled routing")
    shape = LayerShape(16, 32, 128, in_dtype="bf16")
    dims = _dims(shape)
    base = make_decode_pool(DECODE_M16_POOL64, pool=40, shape=shape)
    slots = [int(s) for s in base["perm"][:16]]
    inp = make_decode_step(DECODE_M16_POOL64, 3, 16, shape=shape)
    conv_w = to_dev(base["conv_w"], "bf16")
    x = to_dev(inp["x"], "bf16")
    g = to_dev(inp["g"], "f32")
    beta = to_dev(inp["beta"], "f32")

    def fresh_pool():
        return gdn.SlotPool(dims, 40, state=to_dev(base["S"], "f32"), conv_state=to_dev(base["conv_state"], "bf16"))

    # (a) one call, m = 16
    pa = fresh_pool()
    sp, cp = pa.pointers(torch.tensor(slots, dtype=torch.int32, device="cuda"))
    ya = torch.empty((16, shape.channels), dtype=torch.float32, device="cuda")
    oa = torch.empty((16, 32, 128), dtype=torch.float32, device="cuda")
    gdn.conv_update(dims, x, ya, conv_w, None, cp)
    gdn.decode(dims, ya, g, beta, oa, sp)
    # (b) sixteen calls, m = 1
    pb = fresh_pool()
    ob = torch.empty_like(oa)
    for i, s in enumerate(slots):
        sp1, cp1 = pb.pointers(torch.tensor([s], dtype=torch.int32, device="cuda"))
        y1 = torch.empty((1, shape.channels), dtype=torch.float32, device="cuda")
        o1 = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda")
        gdn.conv_update(dims, x[i:i + 1], y1, conv_w, None, cp1)
        gdn.decode(dims, y1, g[i:i + 1], beta[i:i + 1], o1, sp1)
        ob[i] = o1[0]
    # (c) one call, the same (slot, input) pairs in reversed pointer order
    pc = fresh_pool()
    rev = list(range(15, -1, -1))
    spc, cpc = pc.pointers(torch.tensor([slots[r] for r in rev], dtype=torch.int32, device="cuda"))
    yc = torch.empty_like(ya)
    oc = torch.empty_like(oa)
    gdn.conv_update(dims, x[rev].contiguous(), yc, conv_w, None, cpc)
    gdn.decode(dims, yc, g[rev].contiguous(), beta[rev].contiguous(), oc, spc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_of(oa), bits_of(ob))
    np.testing.assert_array_equal(bits_of(oa), bits_of(oc[rev]))
    for p in (pb, pc):
        np.testing.assert_array_equal(bits_of(pa.state), bits_of(p.state))
        np.testing.assert_array_equal(bits_of(pa.conv_state), bits_of(p.conv_state))
    untouched = [s for s in range(40) if s not in slots]
    np.testing.assert_array_equal(bits_of(pa.state[untouched]), bits_of(to_dev(base["S"], "f32")[untouched]))


def test_inactive_slot_pointers_are_skipped_and_run_twice_is_deterministic():
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce("decode inactive slots + determinism")
    shape = LayerShape(16, 32, 128, in_dtype="bf16")
    dims = _dims(shape)
    base = make_decode_pool(DECODE_M16_POOL64, pool=8, shape=shape)
    inp = make_decode_step(DECODE_M16_POOL64, 9, 5, shape=shape)
    slots = [2, -1, 6, 99, 0]  # -1 and 99 fall outside the pool -> null pointers
    outs = []
    for _ in range(2):
        pool = gdn.SlotPool(dims, 8, state=to_dev(base["S"], "f32"), conv_state=to_dev(base["conv_state"], "bf16"))
        sp, cp = pool.pointers(torch.tensor(slots, dtype=torch.int32, device="cuda"))
        assert sp[1].item() == 0 and sp[3].item() == 0
        y = torch.empty((5, shape.channels), dtype=torch.float32, device="cuda")
        o = torch.full((5, 32, 128), -3.0, dtype=torch.float32, device="cuda")
        gdn.conv_update(dims, to_dev(inp["x"], "bf16"), y, to_dev(base["conv_w"], "bf16"), None, cp)
        gdn.decode(dims, y, to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32"), o, sp)
        torch.cuda.synchronize()
        assert torch.all(o[1] == -3.0) and torch.all(o[3] == -3.0)
        outs.append((bits_of(o), bits_of(pool.state), bits_of(pool.conv_state)))
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)


def test_large_batch_unit_size_is_bit_exact_against_m1():
    """At m * Hv >= 1024 the decode launch uses one-pass units (8 state rows per wave),
    below it two-pass units; a slot's bits must not depend on which one ran. m = 40 in one
    call == the same slots one at a time (m = 1)."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce("decode bit-exact m=40 (one-pass units) vs m=1 (two-pass units)")
    shape = LayerShape(16, 32, 128, in_dtype="bf16")
    dims = _dims(shape)
    base = make_decode_pool(DECODE_M16_POOL64, pool=48, shape=shape)
    slots = [int(s) for s in base["perm"][:40]]
    inp = make_decode_step(DECODE_M16_POOL64, 5, 40, shape=shape)
    conv_w = to_dev(base["conv_w"], "bf16")
    x, g, beta = to_dev(inp["x"], "bf16"), to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32")

    def fresh_pool():
        return gdn.SlotPool(dims, 48, state=to_dev(base["S"], "f32"), conv_state=to_dev(base["conv_state"], "bf16"))

    pa = fresh_pool()
    sp, cp = pa.pointers(torch.tensor(slots, dtype=torch.int32, device="cuda"))
    ya = torch.empty((40, shape.channels), dtype=torch.float32, device="cuda")
    oa = torch.empty((40, 32, 128), dtype=torch.float32, device="cuda")
    gdn.conv_update(dims, x, ya, conv_w, None, cp)
    gdn.decode(dims, ya, g, beta, oa, sp)
    pb = fresh_pool()
    ob = torch.empty_like(oa)
    for i, s in enumerate(slots):
        sp1, cp1 = pb.pointers(torch.tensor([s], dtype=torch.int32, device="cuda"))
        y1 = torch.empty((1, shape.channels), dtype=torch.float32, device="cuda")
        o1 = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda")
        gdn.conv_update(dims, x[i:i + 1], y1, conv_w, None, cp1)
        gdn.decode(dims, y1, g[i:i + 1], beta[i:i + 1], o1, sp1)
        ob[i] = o1[0]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_of(oa), bits_of(ob))
    np.testing.assert_array_equal(bits_of(pa.state), bits_of(pb.state))
    np.testing.assert_array_equal(bits_of(pa.conv_state), bits_of(pb.conv_state))
    # and the one-pass result matches the oracle
    ref = decode_layer(inp["x"], base["conv_w"], base["conv_state"][slots], base["S"][slots], inp["g"],
                       inp["beta"], 16, 32, 128, in_dtype="bf16")
    S_gpu = pa.state[slots].cpu().numpy()
    err_S = max_block_err_S(S_gpu, ref["S"])
    err_o = max(normwise_err(oa[i, j].cpu().numpy(), ref["o"][i, j]) for i in range(40) for j in range(32))
    print(f"m=40 one-pass units: max normwise err o={err_o:.3e} S={err_S:.3e}")
    assert err_S <= TOL_BF16 and err_o <= TOL_BF16


def test_graph_replay_matches_eager_every_replay():
    """A two-layer decode step captured in a HIP graph, replayed three times with eager
    work in between: every replay equals the same step run eagerly, bit for bit."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce("decode graph replay vs eager")
    shape = LayerShape(16, 32, 128, in_dtype="bf16")
    dims = _dims(shape)
    layers, pool_slots, m = 2, 24, 20
    base = [make_decode_pool(DECODE_M16_POOL64, pool=pool_slots, shape=shape) for _ in range(layers)]
    slots = [int(s) for s in base[0]["perm"][:m]]
    idx = torch.tensor(slots, dtype=torch.int32, device="cuda")
    inp = make_decode_step(DECODE_M16_POOL64, 7, m, shape=shape)
    x, g, beta = to_dev(inp["x"], "bf16"), to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32")

    def rig():
        pools = [gdn.SlotPool(dims, pool_slots, state=to_dev(b["S"], "f32"),
                              conv_state=to_dev(b["conv_state"], "bf16")) for b in base]
        ptrs = [p.pointers(idx) for p in pools]
        ws = [to_dev(b["conv_w"], "bf16") for b in base]
        y = torch.empty((m, shape.channels), dtype=torch.float32, device="cuda")
        o = torch.empty((layers, m, 32, 128), dtype=torch.float32, device="cuda")

        def step():
            for layer in range(layers):
                sp, cp = ptrs[layer]
                gdn.conv_update(dims, x, y, ws[layer], None, cp)
                gdn.decode(dims, y, g, beta, o[layer], sp)
        return pools, o, step

    pools_g, o_g, step_g = rig()
    pools_e, o_e, step_e = rig()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step_g()
    torch.cuda.synchronize()
    for rep in range(3):
        graph.replay()
        step_e()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_of(o_g), bits_of(o_e), err_msg=f"replay {rep}: o")
        for pg, pe in zip(pools_g, pools_e):
            np.testing.assert_array_equal(bits_of(pg.state), bits_of(pe.state), err_msg=f"replay {rep}: state")
            np.testing.assert_array_equal(bits_of(pg.conv_state), bits_of(pe.conv_state),
                                          err_msg=f"replay {rep}: conv state")
