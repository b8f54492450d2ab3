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


# (Hk, Hv, d, in_dtype, K, activation, bias, m): all head dims, both input dtypes, every
# conv width, SiLU and bias; 1, 2, 3, 4 and 32 v-heads per k-head (one workgroup per
# (slot, k-head): with 4 at d = 128 every wave walks two row blocks, with 32 the workgroup
# also has more conv channel groups than threads)
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
    (2, 8, 128, "bf16", 4, 1, True, 9),
    (1, 3, 64, "f32", 4, 0, False, 5),
    (1, 32, 128, "bf16", 4, 0, True, 3),
]


def _conv_ptrs(gdn, cs, idx):
    """Device pointer array of the slots idx in a conv-state pool tensor cs [slots, K-1, C]."""
    import torch

    out = torch.empty(idx.numel(), dtype=torch.int64, device="cuda")
    gdn.gdn_slot_pointers(cs.data_ptr(), cs[0].numel() * cs.element_size(), cs.shape[0], idx, idx.numel(), out)
    return out


@pytest.mark.parametrize("stream", [False, True])
@pytest.mark.parametrize("hk,hv,d,dt,K,act,bias,m", CASES)
def test_fused_equals_conv_then_decode_bit_for_bit(hk, hv, d, dt, K, act, bias, m, stream):
    """Three consecutive steps on two copies of one pool: conv_update + decode on one,
    decode_fused on the other. o of every step, every slot's state and conv state (also
    the slots outside the call) must agree bit for bit, and the fused result must match
    the oracle. stream: the fused call reads the conv states from one pool and writes the
    new ones to a second, alternating every step; the pool it reads from must keep its
    bits, and the slots outside the call keep theirs in both."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce(f"decode_fused vs conv+decode hk={hk} hv={hv} d={d} {dt} K={K} act={act} bias={bias} m={m} "
             f"stream={stream}")
    shape = LayerShape(hk, hv, d, conv_width=K, in_dtype=dt)
    dims = _dims(shape, act)
    pool_slots = m + 5
    base = make_decode_pool(DECODE_30_LAYERS, pool=pool_slots, shape=shape, with_bias=bias)
    slots = [int(s) for s in base["perm"][:m]]
    rest = [s for s in range(pool_slots) if s not in slots]
    idx = torch.tensor(slots, dtype=torch.int32, device="cuda")
    conv_w = to_dev(base["conv_w"], dt)
    conv_b = to_dev(base["conv_b"], dt) if bias else None
    pa, pb = _pool(gdn, dims, base, shape), _pool(gdn, dims, base, shape)
    spa, cpa = pa.pointers(idx)
    spb, cpb = pb.pointers(idx)
    # the second conv pool of the streaming form: other bits everywhere, so that any slot
    # the call should not write is caught
    cs2 = torch.full_like(pb.conv_state, -3.0)
    pools = [(pb.conv_state, cpb), (cs2, _conv_ptrs(gdn, cs2, idx))]
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
        if stream:
            (cs_in, p_in), (cs_out, p_out) = pools[step % 2], pools[(step + 1) % 2]
            in_bits, out_rest = bits_of(cs_in), bits_of(cs_out[rest])
            gdn.decode_fused(dims, x, conv_w, conv_b, g, beta, ob, spb, p_in, p_out)
        else:
            cs_out = pb.conv_state
            gdn.decode_fused(dims, x, conv_w, conv_b, g, beta, ob, spb, cpb)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_of(oa), bits_of(ob))
        np.testing.assert_array_equal(bits_of(pa.state), bits_of(pb.state))
        np.testing.assert_array_equal(bits_of(pa.conv_state[slots]), bits_of(cs_out[slots]))
        if stream:
            np.testing.assert_array_equal(bits_of(cs_in), in_bits)  # only read
            np.testing.assert_array_equal(bits_of(cs_out[rest]), out_rest)
        else:
            np.testing.assert_array_equal(bits_of(pa.conv_state), bits_of(pb.conv_state))
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
        cs_gpu = cs_out[slots].cpu()
        cs_gpu = cs_gpu.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else cs_gpu.numpy()
        np.testing.assert_array_equal(cs_gpu, ref_cs.astype(cs_gpu.dtype))


@pytest.mark.parametrize("stream", [False, True])
def test_fused_inactive_slots_are_untouched(stream):
    """A slot whose state pointer or conv-state pointer (or, streaming, its output
    conv-state pointer) is 0 is skipped as a whole: its state, conv states and o rows keep
    their bits; the others equal conv + decode."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce(f"decode_fused inactive slots stream={stream}")
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
    cs2 = torch.full_like(pb.conv_state, 5.0)
    cp2 = _conv_ptrs(gdn, cs2, idx)
    # entry 1: no state pointer; entry 4: no conv-state pointer; entry 2 (streaming): no output pointer
    spb[1] = 0
    cpb[4] = 0
    dead = [1, 4]
    if stream:
        cp2[2] = 0
        dead = [1, 2, 4]
    live = [r for r in range(6) if r not in dead]
    spa_live = spa[live].contiguous()
    cpa_live = cpa[live].contiguous()
    y = torch.empty((len(live), shape.channels), dtype=torch.float32, device="cuda")
    oa = torch.empty((len(live), 32, 128), dtype=torch.float32, device="cuda")
    gdn.conv_update(dims, x[live].contiguous(), y, conv_w, None, cpa_live)
    gdn.decode(dims, y, g[live].contiguous(), beta[live].contiguous(), oa, spa_live)
    ob = torch.full((6, 32, 128), -5.0, dtype=torch.float32, device="cuda")
    gdn.decode_fused(dims, x, conv_w, None, g, beta, ob, spb, cpb, cp2 if stream else None)
    torch.cuda.synchronize()
    for r in dead:
        assert torch.all(ob[r] == -5.0)
    np.testing.assert_array_equal(bits_of(oa), bits_of(ob[live]))
    np.testing.assert_array_equal(bits_of(pa.state), bits_of(pb.state))
    new_cs = cs2 if stream else pb.conv_state
    live_slots = [slots[r] for r in live]
    np.testing.assert_array_equal(bits_of(pa.conv_state[live_slots]), bits_of(new_cs[live_slots]))
    for r in dead:
        s = slots[r]
        np.testing.assert_array_equal(bits_of(pb.state[s]), bits_of(to_dev(base["S"][s], "f32")))
        np.testing.assert_array_equal(bits_of(pb.conv_state[s]), bits_of(to_dev(base["conv_state"][s], "bf16")))
        if stream:
            assert torch.all(cs2[s].float() == 5.0)
    if stream:  # the input pool is only read
        np.testing.assert_array_equal(bits_of(pb.conv_state), bits_of(to_dev(base["conv_state"], "bf16")))


@pytest.mark.parametrize("stream", [False, True])
def test_fused_graph_replay_matches_eager(stream):
    """Two layers of decode_fused captured in a HIP graph and replayed three times with
    eager work between replays: each replay equals the eager step bit for bit. stream:
    the graph holds two steps, conv states from pool A to pool B and back."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce(f"decode_fused graph replay vs eager stream={stream}")
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
        second = [torch.zeros_like(p.conv_state) for p in pools]
        ptrs2 = [_conv_ptrs(gdn, c2, idx) for c2 in second]
        ws = [to_dev(b["conv_w"], "bf16") for b in base]
        o = torch.empty((layers, m, 32, 128), dtype=torch.float32, device="cuda")

        def step():
            for half in range(2 if stream else 1):
                for layer in range(layers):
                    sp, cp = ptrs[layer]
                    if not stream:
                        gdn.decode_fused(dims, x, ws[layer], None, g, beta, o[layer], sp, cp)
                    elif half == 0:
                        gdn.decode_fused(dims, x, ws[layer], None, g, beta, o[layer], sp, cp, ptrs2[layer])
                    else:
                        gdn.decode_fused(dims, x, ws[layer], None, g, beta, o[layer], sp, ptrs2[layer], cp)
        return pools, second, o, step

    pools_g, second_g, o_g, step_g = rig()
    pools_e, second_e, o_e, step_e = rig()
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
        for pg, pe, sg, se in zip(pools_g, pools_e, second_g, second_e):
            np.testing.assert_array_equal(bits_of(pg.state), bits_of(pe.state))
            np.testing.assert_array_equal(bits_of(pg.conv_state), bits_of(pe.conv_state))
            np.testing.assert_array_equal(bits_of(sg), bits_of(se))
