"""GPU parity of gdn_prefill_fused: gdn_conv_update (prefill mode) and gdn_prefill_chunked
in one call, the q/k conv computed inside the intra-chunk kernel, must give the same bits
as the two calls in sequence (o, recurrent states, conv states), and match the oracle.

("System Design", "GDN Kernel Dispatch Detail": the prefill branch runs the Conv1d with
the per-sequence conv state, then the chunked gated delta rule on (q, k, v, g, beta,
state) and updates the temporal state; aprender #5279, "Phase plan", P6: ragged lengths
give the per-slot result.)
"""

import numpy as np
import pytest

from gen import PREFILL_L4096, RAGGED_T15717, make_prefill
from gen.inputs import LayerShape
from oracle import prefill_layer
from tests.gpu_helpers import TOL_BF16, TOL_F32, announce, bits_of, max_block_err_o, max_block_err_S, to_dev

pytestmark = pytest.mark.gpu


def _dims(shape, act, form):
    import gated_delta_rule_conv_amd as gdn

    return gdn.make_dims(shape.num_k_heads, shape.num_v_heads, shape.head_dim, conv_width=shape.conv_width,
                         chunk_size=shape.chunk, activation=act, prefill_form=form,
                         in_dtype=gdn.GDN_BF16 if shape.in_dtype == "bf16" else gdn.GDN_F32)


def _run_both(inp, act, form):
    """The batch through conv_update + prefill on one pool copy and prefill_fused on
    another; returns both results (o, state, conv state) as numpy."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    sh = inp["shape"]
    dims = _dims(sh, act, form)
    N, T = len(inp["lens"]), int(inp["cu_seqlens"][-1])
    cu = torch.tensor(inp["cu_seqlens"], dtype=torch.int32, device="cuda")
    x = to_dev(inp["x"], sh.in_dtype)
    w = to_dev(inp["conv_w"], sh.in_dtype)
    b = to_dev(inp["conv_b"], sh.in_dtype) if inp["conv_b"] is not None else None
    g, beta = to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32")
    idx = torch.arange(N, dtype=torch.int32, device="cuda")
    out = []
    for fused in (False, True):
        pool = gdn.SlotPool(dims, N, state=to_dev(inp["S0"], "f32"), conv_state=to_dev(inp["conv_state"], sh.in_dtype))
        sp, cp = pool.pointers(idx)
        o = torch.full((T, sh.num_v_heads, sh.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        if fused:
            ws = gdn.prefill_fused_workspace(dims, N, T)
            ws.fill_(0xA5)  # contents on entry must not matter
            gdn.prefill_fused(dims, x, w, b, g, beta, o, cu, sp, cp, ws)
        else:
            y = torch.empty((T, sh.channels), dtype=torch.float32, device="cuda")
            ws = gdn.prefill_workspace(dims, N, T)
            gdn.conv_update(dims, x, y, w, b, cp, cu)
            gdn.prefill(dims, y, g, beta, o, cu, sp, ws)
        torch.cuda.synchronize()
        out.append((o.cpu().numpy(), pool.state.cpu().numpy(), bits_of(pool.conv_state)))
    return out


# (hk, hv, d, in_dtype, K, activation, bias, chunk, lens, prefill_form): every head dim,
# chunk size, conv width and dtype, SiLU and bias, sequences shorter than the conv window
# (their conv rows come from the conv state), an empty sequence, partial last chunks,
# both prefill forms (600 tokens at 2/4 heads take the chunk-parallel form). Whole
# sequences in 64-token chunks have the inter-chunk kernel convolve v (bf16 and fp32 x,
# every conv width, bias and SiLU, one and two 16-row blocks per workgroup); the other
# cases run the v conv as a launch of its own. Groups of 4, 9 and 12 v-heads per k-head
# take the intra-chunk kernel's decay terms in one batch of up to 8 v-heads and in two.
CASES = [
    (16, 32, 128, "bf16", 4, 0, False, 64, (1, 17, 64, 0, 300, 130), 0),
    (2, 4, 64, "bf16", 3, 1, True, 32, (2, 1, 70, 33), 0),
    (2, 4, 32, "f32", 2, 0, True, 16, (5, 40, 1), 0),
    (4, 8, 128, "f32", 4, 1, False, 64, (100, 3), 0),
    (2, 4, 128, "bf16", 4, 0, True, 64, (600,), 2),
    (2, 4, 128, "bf16", 4, 1, False, 64, (600, 2), 0),
    (1, 2, 64, "bf16", 4, 1, False, 16, (129, 7), 1),
    (2, 4, 128, "bf16", 4, 1, True, 64, (300, 70, 0, 2), 1),
    (2, 4, 128, "f32", 3, 1, True, 64, (130, 1, 64), 1),
    (2, 4, 64, "bf16", 2, 0, False, 64, (65, 2, 129), 1),
    (8, 32, 32, "f32", 4, 1, True, 64, (70, 1, 200, 0, 64, 3, 130, 17), 1),
    (2, 8, 128, "bf16", 4, 1, True, 64, (200, 64), 1),
    (1, 12, 32, "bf16", 4, 1, True, 16, (50, 3, 17), 1),
    (1, 9, 64, "f32", 3, 0, False, 64, (130, 64, 1), 0),
]


@pytest.mark.parametrize("hk,hv,d,dt,K,act,bias,chunk,lens,form", CASES)
def test_fused_equals_conv_then_prefill_bit_for_bit(hk, hv, d, dt, K, act, bias, chunk, lens, form):
    announce(f"prefill_fused vs conv+prefill hk={hk} hv={hv} d={d} {dt} K={K} act={act} bias={bias} C={chunk} "
             f"lens={lens} form={form}")
    shape = LayerShape(hk, hv, d, conv_width=K, chunk=chunk, in_dtype=dt)
    inp = make_prefill(RAGGED_T15717, lens=lens, shape=shape, s0_std=0.05, conv_state_std=1.0, with_bias=bias)
    (oa, Sa, ca), (ob, Sb, cb) = _run_both(inp, act, form)
    np.testing.assert_array_equal(oa.view(np.int32), ob.view(np.int32))
    np.testing.assert_array_equal(Sa.view(np.int32), Sb.view(np.int32))
    np.testing.assert_array_equal(ca, cb)
    ref = prefill_layer(inp["x"], inp["conv_w"], inp["cu_seqlens"], inp["conv_state"], inp["S0"], inp["g"],
                        inp["beta"], hk, hv, d, in_dtype=dt, activation="silu" if act else "none",
                        conv_b=inp["conv_b"])
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    eo = max_block_err_o(ob, ref["o"], inp["cu_seqlens"])
    eS = max_block_err_S(Sb, ref["S"])
    print(f"fused: max normwise err o={eo:.3e} S={eS:.3e} (tol {tol:g})")
    assert eo <= tol and eS <= tol, (eo, eS)


def test_fused_full_size_L4096_bit_for_bit():
    """The benchmark's launch (one 4096-token sequence, 16/32 heads, d = 128, bf16, chunk
    64): fused and two-call results agree bit for bit."""
    announce("prefill_fused vs conv+prefill L=4096")
    inp = make_prefill(PREFILL_L4096)
    (oa, Sa, ca), (ob, Sb, cb) = _run_both(inp, 0, 0)
    np.testing.assert_array_equal(oa.view(np.int32), ob.view(np.int32))
    np.testing.assert_array_equal(Sa.view(np.int32), Sb.view(np.int32))
    np.testing.assert_array_equal(ca, cb)


def test_fused_full_size_ragged_T15717_bit_for_bit():
    """The benchmark's ragged launch (8 packed sequences of 1 .. 8192 tokens, T = 15717,
    nonzero initial and conv states): fused and two-call results agree bit for bit, so the
    fused path inherits the two-call path's full-size checks against the oracle."""
    announce("prefill_fused vs conv+prefill ragged T=15717")
    inp = make_prefill(RAGGED_T15717)
    (oa, Sa, ca), (ob, Sb, cb) = _run_both(inp, 0, 0)
    np.testing.assert_array_equal(oa.view(np.int32), ob.view(np.int32))
    np.testing.assert_array_equal(Sa.view(np.int32), Sb.view(np.int32))
    np.testing.assert_array_equal(ca, cb)
