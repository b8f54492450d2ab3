"""gdn_prefill_fused_static: the one-call prefill for callers that cannot allocate device
memory, its workspace the library's own device array. Two calls in a row, the second
smaller, each through the C ABI against gdn_prefill_fused with a workspace the test
allocates: the same kernels run, so o, the recurrent states and the conv states must
agree bit for bit (and the first also with the oracle)."""

import numpy as np
import pytest

from gen import RAGGED_T15717, make_prefill
from gen.inputs import LayerShape
from tests.gpu_helpers import TOL_BF16, announce, bits_of, max_block_err_o, max_block_err_S, to_dev

pytestmark = pytest.mark.gpu


def _run(inp, static):
    import torch

    import gated_delta_rule_conv_amd as gdn

    sh = inp["shape"]
    dims = gdn.make_dims(sh.num_k_heads, sh.num_v_heads, sh.head_dim, conv_width=sh.conv_width, chunk_size=sh.chunk,
                         in_dtype=gdn.GDN_BF16)
    N, T = len(inp["lens"]), int(inp["cu_seqlens"][-1])
    pool = gdn.SlotPool(dims, N, state=to_dev(inp["S0"], "f32"), conv_state=to_dev(inp["conv_state"], "bf16"))
    sp, cp = pool.pointers(torch.arange(N, dtype=torch.int32, device="cuda"))
    cu = torch.tensor(inp["cu_seqlens"], dtype=torch.int32, device="cuda")
    x, w = to_dev(inp["x"], "bf16"), to_dev(inp["conv_w"], "bf16")
    g, beta = to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32")
    o = torch.full((T, sh.num_v_heads, sh.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    if static:
        gdn.gdn_prefill_fused_static(dims, x, x.stride(0), w, None, g, beta, o, cu, N, T, sp, cp)
    else:
        ws = gdn.prefill_fused_workspace(dims, N, T)
        ws.fill_(0x5A)
        gdn.gdn_prefill_fused(dims, x, x.stride(0), w, None, g, beta, o, cu, N, T, sp, cp, ws,
                              ws.numel() * ws.element_size())
    torch.cuda.synchronize()
    return o, pool.state, pool.conv_state


@pytest.mark.parametrize("lens_pair", [((600, 300, 1), (37, 5)), ((1000,), (64, 1, 2))])
def test_static_workspace_prefill_equals_allocated_workspace_prefill(lens_pair):
    import gated_delta_rule_conv_amd as gdn

    shape = LayerShape(16, 32, 128, conv_width=4, chunk=64, in_dtype="bf16")
    for n, lens in enumerate(lens_pair):
        announce(f"prefill_fused_static call {n}: lens={lens}")
        inp = make_prefill(RAGGED_T15717, lens=lens, shape=shape, s0_std=0.02, conv_state_std=1.0)
        dims = gdn.make_dims(16, 32, 128, in_dtype=gdn.GDN_BF16)
        need = gdn.gdn_prefill_fused_workspace_size(dims, len(lens), sum(lens))
        assert need <= gdn.GDN_STATIC_SCRATCH_BYTES
        oa, Sa, ca = _run(inp, static=False)
        ob, Sb, cb = _run(inp, static=True)
        np.testing.assert_array_equal(bits_of(oa), bits_of(ob))
        np.testing.assert_array_equal(bits_of(Sa), bits_of(Sb))
        np.testing.assert_array_equal(bits_of(ca), bits_of(cb))
        if n == 0:
            from tests.oracle_pool import prefill_all_heads

            ref = prefill_all_heads(inp)
            eo = max_block_err_o(ob.cpu().numpy(), ref["o"], inp["cu_seqlens"])
            eS = max_block_err_S(Sb.cpu().numpy(), ref["S"])
            print(f"static workspace prefill: max normwise err o={eo:.3e} S={eS:.3e}")
            assert eo <= TOL_BF16 and eS <= TOL_BF16
