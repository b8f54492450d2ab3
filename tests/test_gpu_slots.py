"""GPU tests of gdn_slot_copy: snapshot / fork of slot state and conv state.

("qLLM", "What's still open": prefix caching needs recurrent-state snapshots; aprender
#5279, "Where concurrency is lost", item 6, and "Phase plan", P7: per-slot prefix reuse
and checkpoints.) The fixed-size state is the whole history the layer keeps, so a copied
slot must continue exactly like its source: these checks are bit-exact.
"""

import numpy as np
import pytest

from gen import DECODE_M16_POOL64, PREFILL_L4096, RAGGED_T15717, make_decode_pool, make_decode_step, make_prefill
from gen.inputs import LayerShape
from tests.gpu_helpers import announce, bits_of, to_dev

pytestmark = pytest.mark.gpu


def _dims(shape):
    import gated_delta_rule_conv_amd as gdn

    return gdn.make_dims(shape.num_k_heads, shape.num_v_heads, shape.head_dim, conv_width=shape.conv_width,
                         chunk_size=shape.chunk,
                         in_dtype=gdn.GDN_BF16 if shape.in_dtype == "bf16" else gdn.GDN_F32)


def test_fork_copies_state_and_conv_state_bit_exact():
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce("slot copy: fork 3 slots, bf16, d=128")
    shape = LayerShape(16, 32, 128, in_dtype="bf16")
    dims = _dims(shape)
    base = make_decode_pool(DECODE_M16_POOL64, pool=12, shape=shape)
    pool = gdn.SlotPool(dims, 12, state=to_dev(base["S"], "f32"), conv_state=to_dev(base["conv_state"], "bf16"))
    src, dst = [2, 2, 5], [7, 9, 0]
    pool.copy_slots(torch.tensor(src, dtype=torch.int32, device="cuda"),
                    torch.tensor(dst, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    S0, C0 = to_dev(base["S"], "f32"), to_dev(base["conv_state"], "bf16")
    for s_, d_ in zip(src, dst):
        np.testing.assert_array_equal(bits_of(pool.state[d_]), bits_of(S0[s_]))
        np.testing.assert_array_equal(bits_of(pool.conv_state[d_]), bits_of(C0[s_]))
    others = [i for i in range(12) if i not in dst]
    np.testing.assert_array_equal(bits_of(pool.state[others]), bits_of(S0[others]))
    np.testing.assert_array_equal(bits_of(pool.conv_state[others]), bits_of(C0[others]))

    # state only: the conv state of the destination keeps its bits; index -1 -> null pointer, skipped
    pool2 = gdn.SlotPool(dims, 12, state=to_dev(base["S"], "f32"), conv_state=to_dev(base["conv_state"], "bf16"))
    pool2.copy_slots(torch.tensor([3, 4], dtype=torch.int32, device="cuda"),
                     torch.tensor([8, -1], dtype=torch.int32, device="cuda"), conv_state=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_of(pool2.state[8]), bits_of(S0[3]))
    np.testing.assert_array_equal(bits_of(pool2.conv_state), bits_of(C0))
    np.testing.assert_array_equal(bits_of(pool2.state[[i for i in range(12) if i != 8]]),
                                  bits_of(S0[[i for i in range(12) if i != 8]]))


def test_forked_slot_decodes_like_its_source():
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce("slot copy: fork then decode 4 steps")
    shape = LayerShape(16, 32, 128, in_dtype="bf16")
    dims = _dims(shape)
    base = make_decode_pool(DECODE_M16_POOL64, pool=6, shape=shape)
    pool = gdn.SlotPool(dims, 6, state=to_dev(base["S"], "f32"), conv_state=to_dev(base["conv_state"], "bf16"))
    pool.copy_slots(torch.tensor([1], dtype=torch.int32, device="cuda"),
                    torch.tensor([4], dtype=torch.int32, device="cuda"))
    idx = torch.tensor([1, 4], dtype=torch.int32, device="cuda")
    sp, cp = pool.pointers(idx)
    conv_w = to_dev(base["conv_w"], "bf16")
    for step in range(4):
        inp = make_decode_step(DECODE_M16_POOL64, 20 + step, 1, shape=shape)
        x = to_dev(inp["x"], "bf16").repeat(2, 1)  # the same token for both slots
        g = to_dev(inp["g"], "f32").repeat(2, 1)
        beta = to_dev(inp["beta"], "f32").repeat(2, 1)
        y = torch.empty((2, shape.channels), dtype=torch.float32, device="cuda")
        o = torch.empty((2, 32, 128), dtype=torch.float32, device="cuda")
        gdn.conv_update(dims, x, y, conv_w, None, cp)
        gdn.decode(dims, y, g, beta, o, sp)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_of(o[0]), bits_of(o[1]), err_msg=f"step {step}")
    np.testing.assert_array_equal(bits_of(pool.state[1]), bits_of(pool.state[4]))
    np.testing.assert_array_equal(bits_of(pool.conv_state[1]), bits_of(pool.conv_state[4]))


def test_prefix_reuse_equals_one_long_prefill():
    """Prefill a 128-token prefix into one slot, fork it into two slots, continue each with
    its own 100 tokens: each result equals a single prefill of prefix + continuation, bit for
    bit (the prefix is a whole number of chunks, so the chunk boundaries coincide)."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce("slot copy: prefix reuse vs one long prefill")
    shape = LayerShape(4, 8, 128, conv_width=4, chunk=64, in_dtype="bf16")
    dims = _dims(shape)
    P, Lc = 128, 100
    full = [make_prefill(PREFILL_L4096, lens=(P + Lc,), shape=shape, s0_std=0.02, conv_state_std=1.0) for _ in range(1)][0]
    other = make_prefill(RAGGED_T15717, lens=(P + Lc,), shape=shape, s0_std=0.02, conv_state_std=1.0)
    x_a = full["x"]
    x_b = np.concatenate([full["x"][:P], other["x"][P:]], axis=0)  # same prefix, another continuation
    g_a, b_a = full["g"], full["beta"]
    g_b = np.concatenate([full["g"][:P], other["g"][P:]], axis=0)
    b_b = np.concatenate([full["beta"][:P], other["beta"][P:]], axis=0)
    conv_w = to_dev(full["conv_w"], "bf16")
    C, Hv, d = shape.channels, shape.num_v_heads, shape.head_dim

    def run(pool, slot, x, g, beta):
        T = x.shape[0]
        sp, cp = pool.pointers(torch.tensor([slot], dtype=torch.int32, device="cuda"))
        cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
        y = torch.empty((T, C), dtype=torch.float32, device="cuda")
        o = torch.empty((T, Hv, d), dtype=torch.float32, device="cuda")
        ws = gdn.prefill_workspace(dims, 1, T)
        gdn.conv_update(dims, to_dev(x, "bf16"), y, conv_w, None, cp, cu)
        gdn.prefill(dims, y, to_dev(g, "f32"), to_dev(beta, "f32"), o, cu, sp, ws)
        return o

    def fresh_pool(n):
        S = np.repeat(full["S0"][:1], n, axis=0)
        cs = np.repeat(full["conv_state"][:1], n, axis=0)
        return gdn.SlotPool(dims, n, state=to_dev(S, "f32"), conv_state=to_dev(cs, "bf16"))

    # one long prefill per continuation
    ref = fresh_pool(2)
    o_ref_a = run(ref, 0, x_a, g_a, b_a)
    o_ref_b = run(ref, 1, x_b, g_b, b_b)
    # prefix once, fork, continue
    pool = fresh_pool(3)
    o_pre = run(pool, 0, x_a[:P], g_a[:P], b_a[:P])
    pool.copy_slots(torch.tensor([0, 0], dtype=torch.int32, device="cuda"),
                    torch.tensor([1, 2], dtype=torch.int32, device="cuda"))
    o_a = run(pool, 1, x_a[P:], g_a[P:], b_a[P:])
    o_b = run(pool, 2, x_b[P:], g_b[P:], b_b[P:])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_of(o_pre), bits_of(o_ref_a[:P]))
    np.testing.assert_array_equal(bits_of(o_a), bits_of(o_ref_a[P:]))
    np.testing.assert_array_equal(bits_of(o_b), bits_of(o_ref_b[P:]))
    np.testing.assert_array_equal(bits_of(pool.state[1]), bits_of(ref.state[0]))
    np.testing.assert_array_equal(bits_of(pool.state[2]), bits_of(ref.state[1]))
    np.testing.assert_array_equal(bits_of(pool.conv_state[1]), bits_of(ref.conv_state[0]))
    np.testing.assert_array_equal(bits_of(pool.conv_state[2]), bits_of(ref.conv_state[1]))


def test_reused_slot_equals_never_used_slot():
    """A slot that served one sequence, was freed and re-zeroed, then serves a new one,
    gives the same bits as a slot never used: nothing of the old sequence survives the
    reset ("qLLM", "Results": no decode-time contamination when slots are reused). The
    new sequence runs in both slots through prefill and then decode, both entry points."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce("slot reuse: freed + re-zeroed slot == never-used slot")
    shape = LayerShape(4, 8, 128, conv_width=4, chunk=64, in_dtype="bf16")
    dims = _dims(shape)
    C, Hv, d = shape.channels, shape.num_v_heads, shape.head_dim
    old = make_prefill(RAGGED_T15717, lens=(150,), shape=shape, s0_std=0.0, conv_state_std=0.0)
    new = make_prefill(PREFILL_L4096, lens=(90,), shape=shape, s0_std=0.0, conv_state_std=0.0)
    conv_w = to_dev(new["conv_w"], "bf16")
    pool = gdn.SlotPool(dims, 4)  # zero states: fresh slots

    def prefill(slots, inp):
        T = inp["x"].shape[0]
        n = len(slots)
        sp, cp = pool.pointers(torch.tensor(slots, dtype=torch.int32, device="cuda"))
        cu = torch.tensor([i * T for i in range(n + 1)], dtype=torch.int32, device="cuda")
        x = to_dev(np.concatenate([inp["x"]] * n), "bf16")
        g = to_dev(np.concatenate([inp["g"]] * n), "f32")
        beta = to_dev(np.concatenate([inp["beta"]] * n), "f32")
        y = torch.empty((n * T, C), dtype=torch.float32, device="cuda")
        o = torch.empty((n * T, Hv, d), dtype=torch.float32, device="cuda")
        gdn.conv_update(dims, x, y, conv_w, None, cp, cu)
        gdn.prefill(dims, y, g, beta, o, cu, sp, gdn.prefill_workspace(dims, n, n * T))
        return o

    def decode(slots, step, fused):
        inp = make_decode_step(DECODE_M16_POOL64, 40 + step, 1, shape=shape)
        n = len(slots)
        sp, cp = pool.pointers(torch.tensor(slots, dtype=torch.int32, device="cuda"))
        x = to_dev(inp["x"], "bf16").repeat(n, 1)
        g = to_dev(inp["g"], "f32").repeat(n, 1)
        beta = to_dev(inp["beta"], "f32").repeat(n, 1)
        o = torch.empty((n, Hv, d), dtype=torch.float32, device="cuda")
        if fused:
            gdn.decode_fused(dims, x, conv_w, None, g, beta, o, sp, cp)
        else:
            y = torch.empty((n, C), dtype=torch.float32, device="cuda")
            gdn.conv_update(dims, x, y, conv_w, None, cp)
            gdn.decode(dims, y, g, beta, o, sp)
        return o

    # slot 1 serves an old sequence (prefill and three decode steps), then is freed
    prefill([1], old)
    for step in range(3):
        decode([1], step, fused=step % 2 == 1)
    torch.cuda.synchronize()
    assert pool.state[1].abs().max().item() > 0 and pool.conv_state[1].float().abs().max().item() > 0
    pool.state[1].zero_()
    pool.conv_state[1].zero_()
    # the new sequence in the reused slot 1 and in the never-used slot 3, side by side
    o = prefill([1, 3], new)
    T = new["x"].shape[0]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_of(o[:T]), bits_of(o[T:]))
    for step in range(4):
        od = decode([1, 3], 10 + step, fused=step >= 2)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_of(od[0]), bits_of(od[1]), err_msg=f"decode step {step}")
    np.testing.assert_array_equal(bits_of(pool.state[1]), bits_of(pool.state[3]))
    np.testing.assert_array_equal(bits_of(pool.conv_state[1]), bits_of(pool.conv_state[3]))
    # slots 0 and 2 were never touched
    assert pool.state[[0, 2]].abs().max().item() == 0 and pool.conv_state[[0, 2]].float().abs().max().item() == 0
