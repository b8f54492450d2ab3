"""The decode step at its full size: 30 layers, each a 256-slot pool of 32 v-heads x
128 x 128 fp32 states, m = 64 active slots through a shuffled pointer array, bf16
inputs -- the launches a 30-GDN-layer hybrid makes per generated token. Every layer
runs gdn_conv_update + gdn_decode_batched as the benchmark's step does; every one of the
64 slots of three layers (first, middle, last) is checked against the oracle, inactive
slots for untouched bits, and two layers rerun through gdn_decode_fused for the same
bits."""

import numpy as np
import pytest

from gen.inputs import DECODE_30_LAYERS, ST_PERM, WORKLOADS, make_decode_pool_torch, rng_for
from oracle import decode_layer
from tests.gpu_helpers import TOL_BF16, announce, bits_of, max_block_err_S, normwise_err, storage_of

pytestmark = pytest.mark.gpu

LAYERS, POOL, M = 30, 256, 64
SAMPLE_LAYERS = (0, 13, 29)
SAMPLE_ROWS = tuple(range(M))  # positions in the pointer array: all of them


def test_decode_step_full_size_30_layers_every_slot():
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce(f"decode step full size: {LAYERS} layers, pool {POOL}, m={M}")
    sh = WORKLOADS[DECODE_30_LAYERS].shape
    Hk, Hv, d, C = sh.num_k_heads, sh.num_v_heads, sh.head_dim, sh.channels
    dims = gdn.make_dims(Hk, Hv, d, conv_width=sh.conv_width, chunk_size=sh.chunk, in_dtype=gdn.GDN_BF16)
    states, conv_states, conv_w = make_decode_pool_torch(DECODE_30_LAYERS, POOL, LAYERS, "cuda")
    slots = rng_for(DECODE_30_LAYERS, ST_PERM).permutation(POOL)[:M].astype(np.int32)
    idle = [s for s in range(POOL) if s not in set(slots.tolist())][:3]
    idx = torch.tensor(slots, dtype=torch.int32, device="cuda")
    sptr = torch.empty((LAYERS, M), dtype=torch.int64, device="cuda")
    cptr = torch.empty((LAYERS, M), dtype=torch.int64, device="cuda")
    s_bytes = states[0, 0].numel() * 4
    c_bytes = conv_states[0, 0].numel() * conv_states.element_size()
    for layer in range(LAYERS):
        gdn.gdn_slot_pointers(states[layer].data_ptr(), s_bytes, POOL, idx, M, sptr[layer])
        gdn.gdn_slot_pointers(conv_states[layer].data_ptr(), c_bytes, POOL, idx, M, cptr[layer])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3900)
    x = torch.randn((LAYERS, M, C), generator=gen, device="cuda").to(torch.bfloat16)
    g = -torch.nn.functional.softplus(torch.randn((LAYERS, M, Hv), generator=gen, device="cuda"))
    beta = torch.sigmoid(torch.randn((LAYERS, M, Hv), generator=gen, device="cuda"))

    # host copies of what the checks need, taken before the step
    pick = [int(slots[r]) for r in SAMPLE_ROWS]
    before = {l: (states[l, pick].cpu().numpy(), storage_of(conv_states[l, pick], "bf16"), conv_w[l].cpu())
              for l in SAMPLE_LAYERS}
    idle_bits = {l: (bits_of(states[l, idle]), bits_of(conv_states[l, idle])) for l in SAMPLE_LAYERS}
    fused_layers = (SAMPLE_LAYERS[0], SAMPLE_LAYERS[-1])
    copies = {l: (states[l].clone(), conv_states[l].clone()) for l in fused_layers}

    y = torch.empty((M, C), dtype=torch.float32, device="cuda")
    o = torch.empty((LAYERS, M, Hv, d), dtype=torch.float32, device="cuda")
    for layer in range(LAYERS):
        gdn.conv_update(dims, x[layer], y, conv_w[layer], None, cptr[layer])
        gdn.decode(dims, y, g[layer], beta[layer], o[layer], sptr[layer])
    torch.cuda.synchronize()

    worst_o = worst_S = 0.0
    for l in SAMPLE_LAYERS:
        S0, cs0, w = before[l]
        rows = list(SAMPLE_ROWS)
        ref = decode_layer(storage_of(x[l, rows], "bf16"), storage_of(w, "bf16"), cs0, S0.astype(np.float64),
                           g[l, rows].cpu().numpy(), beta[l, rows].cpu().numpy(), Hk, Hv, d, in_dtype="bf16")
        og = o[l, rows].cpu().numpy()
        worst_o = max(worst_o, max(normwise_err(og[i, j], ref["o"][i, j]) for i in range(len(rows))
                                   for j in range(Hv)))
        worst_S = max(worst_S, max_block_err_S(states[l, pick].cpu().numpy(), ref["S"]))
        from gen import bf16_bits_from_f32

        np.testing.assert_array_equal(storage_of(conv_states[l, pick], "bf16"),
                                      bf16_bits_from_f32(ref["conv_state"].astype(np.float32)))
        np.testing.assert_array_equal(bits_of(states[l, idle]), idle_bits[l][0])
        np.testing.assert_array_equal(bits_of(conv_states[l, idle]), idle_bits[l][1])
    print(f"decode full size: max normwise err o={worst_o:.3e} S={worst_S:.3e} (tol {TOL_BF16})")
    assert worst_o <= TOL_BF16 and worst_S <= TOL_BF16

    # the one-launch step on the pre-step copies gives the same bits
    of = torch.empty((M, Hv, d), dtype=torch.float32, device="cuda")
    for l in fused_layers:
        st, cs = copies[l]
        sp1 = torch.empty((M,), dtype=torch.int64, device="cuda")
        cp1 = torch.empty((M,), dtype=torch.int64, device="cuda")
        gdn.gdn_slot_pointers(st.data_ptr(), s_bytes, POOL, idx, M, sp1)
        gdn.gdn_slot_pointers(cs.data_ptr(), c_bytes, POOL, idx, M, cp1)
        gdn.decode_fused(dims, x[l], conv_w[l], None, g[l], beta[l], of, sp1, cp1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_of(of), bits_of(o[l]))
        np.testing.assert_array_equal(bits_of(st), bits_of(states[l]))
        np.testing.assert_array_equal(bits_of(cs), bits_of(conv_states[l]))
