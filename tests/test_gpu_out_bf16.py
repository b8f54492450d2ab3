"""bf16 output (dims.out_dtype = GDN_BF16): o is the fp32 result rounded to the nearest
bf16 (ties to even), so it must equal, bit for bit, the fp32 run's o rounded on the host;
states and conv states are untouched by the choice. Decode (both entry points, both unit
sizes) and prefill (both entry points, both prefill forms, ragged pack)."""

import numpy as np
import pytest

from gen import DECODE_30_LAYERS, RAGGED_T15717, bf16_bits_from_f32, make_decode_pool, make_decode_step, make_prefill
from gen.inputs import LayerShape
from oracle import decode_layer
from tests.gpu_helpers import announce, bits_of, normwise_err, storage_of, to_dev

pytestmark = pytest.mark.gpu


def _dims(sh, out, form=0, act=0):
    import gated_delta_rule_conv_amd as gdn

    return gdn.make_dims(sh.num_k_heads, sh.num_v_heads, sh.head_dim, conv_width=sh.conv_width, chunk_size=sh.chunk,
                         activation=act, in_dtype=gdn.GDN_BF16, prefill_form=form,
                         out_dtype=gdn.GDN_BF16 if out == "bf16" else gdn.GDN_F32)


def _rounded(o32) -> np.ndarray:
    """Host rounding of the fp32 run's o to bf16 bits."""
    return bf16_bits_from_f32(o32.detach().cpu().numpy())


@pytest.mark.parametrize("m", [5, 40])
@pytest.mark.parametrize("fused", [False, True])
def test_decode_bf16_output_is_the_rounded_fp32_output(m, fused):
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce(f"decode out bf16 m={m} {'fused' if fused else 'two calls'}")
    sh = LayerShape(16, 32, 128, in_dtype="bf16")
    base = make_decode_pool(DECODE_30_LAYERS, pool=48, shape=sh)
    slots = [int(s) for s in base["perm"][:m]]
    inp = make_decode_step(DECODE_30_LAYERS, 2, m, shape=sh)
    x, g, beta = to_dev(inp["x"], "bf16"), to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32")
    w = to_dev(base["conv_w"], "bf16")
    res = {}
    for out in ("f32", "bf16"):
        dims = _dims(sh, out)
        pool = gdn.SlotPool(dims, 48, state=to_dev(base["S"], "f32"), conv_state=to_dev(base["conv_state"], "bf16"))
        sp, cp = pool.pointers(torch.tensor(slots, dtype=torch.int32, device="cuda"))
        o = torch.empty((m, sh.num_v_heads, sh.head_dim), dtype=torch.bfloat16 if out == "bf16" else torch.float32,
                        device="cuda")
        if fused:
            gdn.decode_fused(dims, x, w, None, g, beta, o, sp, cp)
        else:
            y = torch.empty((m, sh.channels), dtype=torch.float32, device="cuda")
            gdn.conv_update(dims, x, y, w, None, cp)
            gdn.decode(dims, y, g, beta, o, sp)
        torch.cuda.synchronize()
        res[out] = (o, bits_of(pool.state), bits_of(pool.conv_state))
    o32, S32, c32 = res["f32"]
    o16, S16, c16 = res["bf16"]
    np.testing.assert_array_equal(storage_of(o16, "bf16"), _rounded(o32))
    np.testing.assert_array_equal(S16, S32)
    np.testing.assert_array_equal(c16, c32)
    # and against the oracle: the fp32 error plus the rounding, at most 2^-8 of |o| (bf16
    # keeps 8 significant bits)
    ref = decode_layer(inp["x"], base["conv_w"], base["conv_state"][slots], base["S"][slots], inp["g"], inp["beta"],
                       16, 32, 128, in_dtype="bf16")
    og = o16.float().cpu().numpy()
    err = max(normwise_err(og[i, j], ref["o"][i, j]) for i in range(m) for j in range(32))
    print(f"decode out bf16: max normwise err vs oracle {err:.3e}")
    assert err <= 2.0 ** -8 + 1e-4


@pytest.mark.parametrize("form", [1, 2])
@pytest.mark.parametrize("fused", [False, True])
def test_prefill_bf16_output_is_the_rounded_fp32_output(form, fused):
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce(f"prefill out bf16 form={form} {'fused' if fused else 'two calls'}")
    sh = LayerShape(2, 4, 128, conv_width=4, chunk=64, in_dtype="bf16")
    inp = make_prefill(RAGGED_T15717, lens=(1, 200, 64, 77), shape=sh, s0_std=0.05, conv_state_std=1.0)
    N, T = len(inp["lens"]), int(inp["cu_seqlens"][-1])
    cu = torch.tensor(inp["cu_seqlens"], dtype=torch.int32, device="cuda")
    x, w = to_dev(inp["x"], "bf16"), to_dev(inp["conv_w"], "bf16")
    g, beta = to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32")
    res = {}
    for out in ("f32", "bf16"):
        dims = _dims(sh, out, form=form)
        pool = gdn.SlotPool(dims, N, state=to_dev(inp["S0"], "f32"), conv_state=to_dev(inp["conv_state"], "bf16"))
        sp, cp = pool.pointers(torch.arange(N, dtype=torch.int32, device="cuda"))
        o = torch.empty((T, sh.num_v_heads, sh.head_dim), dtype=torch.bfloat16 if out == "bf16" else torch.float32,
                        device="cuda")
        if fused:
            gdn.prefill_fused(dims, x, w, None, g, beta, o, cu, sp, cp, gdn.prefill_fused_workspace(dims, N, T))
        else:
            y = torch.empty((T, sh.channels), dtype=torch.float32, device="cuda")
            gdn.conv_update(dims, x, y, w, None, cp, cu)
            gdn.prefill(dims, y, g, beta, o, cu, sp, gdn.prefill_workspace(dims, N, T))
        torch.cuda.synchronize()
        res[out] = (o, bits_of(pool.state), bits_of(pool.conv_state))
    o32, S32, c32 = res["f32"]
    o16, S16, c16 = res["bf16"]
    np.testing.assert_array_equal(storage_of(o16, "bf16"), _rounded(o32))
    np.testing.assert_array_equal(S16, S32)
    np.testing.assert_array_equal(c16, c32)
