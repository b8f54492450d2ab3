"""GPU parity of gdn_conv_update (both modes) against the oracle's causal conv.

y is compared elementwise (fp32 accumulation of K products vs float64); the conv state
must equal the oracle's bit for bit, since it only copies representable inputs.
("System Design", "GDN Kernel Dispatch Detail": depthwise causal Conv1d; conv state
update in the decode branch.)
"""

import numpy as np
import pytest

from gen import DECODE_M16_POOL64, PREFILL_L4096, TINY_FP32, make_decode_pool, make_decode_step, make_prefill
from gen.inputs import LayerShape
from oracle import causal_conv, storage_to_f64
from tests.gpu_helpers import announce, storage_of, to_dev

pytestmark = pytest.mark.gpu


def _dims(shape: LayerShape, act=0):
    import gated_delta_rule_conv_amd as gdn

    return gdn.make_dims(shape.num_k_heads, shape.num_v_heads, shape.head_dim, conv_width=shape.conv_width,
                         chunk_size=shape.chunk, activation=act,
                         in_dtype=gdn.GDN_BF16 if shape.in_dtype == "bf16" else gdn.GDN_F32)


def _oracle_conv(inp, act):
    sh = inp["shape"]
    x = storage_to_f64(inp["x"], sh.in_dtype)
    w = storage_to_f64(inp["conv_w"], sh.in_dtype)
    b = storage_to_f64(inp["conv_b"], sh.in_dtype)
    cs = storage_to_f64(inp["conv_state"], sh.in_dtype)
    cu = inp["cu_seqlens"]
    y = np.zeros_like(x)
    new = np.zeros_like(cs)
    for s in range(len(cu) - 1):
        y[cu[s]:cu[s + 1]], new[s] = causal_conv(x[cu[s]:cu[s + 1]], w, b, cs[s], act)
    return y, new


def _run_prefill_conv(inp, act, x_pad=0, shuffle=False):
    import torch

    import gated_delta_rule_conv_amd as gdn

    sh = inp["shape"]
    dims = _dims(sh, act=1 if act == "silu" else 0)
    C = sh.channels
    T = inp["x"].shape[0]
    N = len(inp["lens"])
    x = to_dev(inp["x"], sh.in_dtype)
    if x_pad:
        xp = torch.zeros((T, C + x_pad), dtype=x.dtype, device="cuda")
        xp[:, :C] = x
        x = xp[:, :C]
    y = torch.full((T, C), float("nan"), dtype=torch.float32, device="cuda")
    pool = gdn.SlotPool(dims, N + 3, conv_state=None)
    order = np.random.default_rng(1).permutation(N + 3)[:N] if shuffle else np.arange(N)
    cs_dev = to_dev(inp["conv_state"], sh.in_dtype)
    for s in range(N):
        pool.conv_state[int(order[s])] = cs_dev[s]
    _, cptr = pool.pointers(torch.tensor(order, dtype=torch.int32, device="cuda"))
    cu = torch.tensor(inp["cu_seqlens"], dtype=torch.int32, device="cuda")
    gdn.conv_update(dims, x, y, to_dev(inp["conv_w"], sh.in_dtype), to_dev(inp["conv_b"], sh.in_dtype), cptr, cu)
    torch.cuda.synchronize()
    new_cs = np.stack([storage_of(pool.conv_state[int(order[s])], sh.in_dtype) for s in range(N)]) if N else None
    return y.cpu().numpy(), new_cs


CASES = [
    ("f32", 4, [0, 1, 2, 3, 17, 64, 5, 0], False, "none"),
    ("bf16", 4, [1, 2, 40, 0, 16, 15, 33], True, "none"),
    ("bf16", 4, [7, 1, 30], True, "silu"),
    ("f32", 3, [2, 1, 19, 4], False, "silu"),
    ("bf16", 2, [1, 18, 3], True, "none"),
]


@pytest.mark.parametrize("in_dtype,K,lens,bias,act", CASES)
def test_conv_prefill_matches_oracle(in_dtype, K, lens, bias, act):
    announce(f"conv prefill {in_dtype} K={K} lens={lens} bias={bias} act={act}")
    shape = LayerShape(2, 4, 32, conv_width=K, chunk=16, in_dtype=in_dtype)
    inp = make_prefill(TINY_FP32, lens=lens, shape=shape, conv_state_std=1.0, with_bias=bias)
    y_ref, cs_ref = _oracle_conv(inp, act)
    y, cs = _run_prefill_conv(inp, act, x_pad=8 if in_dtype == "f32" else 64, shuffle=True)
    np.testing.assert_allclose(y, y_ref, rtol=1e-5, atol=1e-5)
    ref_bits = inp["conv_state"].copy()
    for s in range(len(lens)):
        # the oracle's new state, rounded back to storage, must be bit-identical
        if in_dtype == "bf16":
            from gen import bf16_bits_from_f32

            ref_bits[s] = bf16_bits_from_f32(cs_ref[s].astype(np.float32))
        else:
            ref_bits[s] = cs_ref[s].astype(np.float32)
    np.testing.assert_array_equal(cs, ref_bits)


def test_conv_prefill_full_size_4096():
    """The 4096-token, 8192-channel bf16 prefill shape, launched as the benchmark does."""
    announce("conv prefill L=4096 C=8192 bf16")
    inp = make_prefill(PREFILL_L4096)
    y_ref, _ = _oracle_conv(inp, "none")
    y, cs = _run_prefill_conv(inp, "none")
    np.testing.assert_allclose(y, y_ref, rtol=1e-5, atol=1e-5)
    x = inp["x"]
    np.testing.assert_array_equal(cs[0], x[-3:])


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_conv_decode_matches_oracle_and_skips_inactive(in_dtype):
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce(f"conv decode {in_dtype}")
    shape = LayerShape(16, 32, 128, in_dtype=in_dtype)
    pool_np = make_decode_pool(DECODE_M16_POOL64, pool=12, shape=shape)
    step = make_decode_step(DECODE_M16_POOL64, 0, 6, shape=shape)
    dims = _dims(shape)
    pool = gdn.SlotPool(dims, 12, conv_state=to_dev(pool_np["conv_state"], in_dtype))
    slots = [5, 0, 11, -1, 7, 3]  # -1: inactive slot (null pointer)
    _, cptr = pool.pointers(torch.tensor(slots, dtype=torch.int32, device="cuda"))
    x = to_dev(step["x"], in_dtype)
    y = torch.full((6, shape.channels), 7.0, dtype=torch.float32, device="cuda")
    before = pool.conv_state.clone()
    gdn.conv_update(dims, x, y, to_dev(pool_np["conv_w"], in_dtype), None, cptr)
    torch.cuda.synchronize()
    xf = storage_to_f64(step["x"], in_dtype)
    w = storage_to_f64(pool_np["conv_w"], in_dtype)
    for i, s in enumerate(slots):
        if s < 0:
            assert torch.all(y[i] == 7.0)
            continue
        yr, csr = causal_conv(xf[i:i + 1], w, None, storage_to_f64(pool_np["conv_state"][s], in_dtype))
        np.testing.assert_allclose(y[i].cpu().numpy(), yr[0], rtol=1e-5, atol=1e-5)
        got = pool.conv_state[s].cpu().to(torch.float64).numpy()
        np.testing.assert_array_equal(got, csr)
    untouched = [s for s in range(12) if s not in slots]
    for s in untouched:
        assert torch.equal(pool.conv_state[s], before[s])
