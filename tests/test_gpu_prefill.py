"""GPU parity of the prefill path (gdn_conv_update in prefill mode + gdn_prefill_chunked)
against the oracle, plus packing, split and edge cases.

("System Design", "GDN Kernel Dispatch Detail": prefill = Conv1d, L2 norm, chunked
gated delta rule on (q, k, v, g, beta, state), temporal state updated; aprender #5279,
"Phase plan", P6: ragged lengths such as 1, 17, 300, 4095 give the per-slot result.)
"""

import numpy as np
import pytest

from gen import PREFILL_L4096, RAGGED_T15717, TINY_FP32, make_prefill
from gen.inputs import LayerShape
from tests.gpu_helpers import (TOL_BF16, TOL_F32, announce, bits_of, max_block_err_o, max_block_err_S, storage_of,
                               to_dev)

pytestmark = pytest.mark.gpu


def _dims(shape, act=0, mma=0, form=0):
    import gated_delta_rule_conv_amd as gdn

    return gdn.make_dims(shape.num_k_heads, shape.num_v_heads, shape.head_dim, conv_width=shape.conv_width,
                         chunk_size=shape.chunk, activation=act, mma=mma, prefill_form=form,
                         in_dtype=gdn.GDN_BF16 if shape.in_dtype == "bf16" else gdn.GDN_F32)


class PrefillRun:
    """Device copies of one packed batch; run() does conv + prefill through the C ABI."""

    def __init__(self, inp, act=0, mma=0, g=None, form=0):
        import torch

        import gated_delta_rule_conv_amd as gdn

        sh = inp["shape"]
        self.inp, self.sh = inp, sh
        self.dims = _dims(sh, act, mma, form)
        self.N = len(inp["lens"])
        self.T = int(inp["cu_seqlens"][-1])
        self.pool = gdn.SlotPool(self.dims, max(self.N, 1), state=to_dev(inp["S0"], "f32"),
                                 conv_state=to_dev(inp["conv_state"], sh.in_dtype))
        self.sp, self.cp = self.pool.pointers(torch.arange(self.N, dtype=torch.int32, device="cuda"))
        self.cu = torch.tensor(inp["cu_seqlens"], dtype=torch.int32, device="cuda")
        self.x = to_dev(inp["x"], sh.in_dtype)
        self.w = to_dev(inp["conv_w"], sh.in_dtype)
        self.g = to_dev(inp["g"] if g is None else g, "f32")
        self.beta = to_dev(inp["beta"], "f32")
        self.y = torch.empty((self.T, sh.channels), dtype=torch.float32, device="cuda")
        self.o = torch.full((self.T, sh.num_v_heads, sh.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        self.ws = gdn.prefill_workspace(self.dims, self.N, self.T)

    def run(self):
        import torch

        import gated_delta_rule_conv_amd as gdn

        gdn.conv_update(self.dims, self.x, self.y, self.w, None, self.cp, self.cu)
        gdn.prefill(self.dims, self.y, self.g, self.beta, self.o, self.cu, self.sp, self.ws)
        torch.cuda.synchronize()
        return self.o.cpu().numpy(), self.pool.state.cpu().numpy()


def _oracle(inp, act="none", g=None, **kw):
    """The oracle over every v-head of the batch (sharded over host processes when the
    layer has several k-heads)."""
    from tests.oracle_pool import prefill_all_heads

    return prefill_all_heads(inp if g is None else dict(inp, g=g), activation=act, **kw)


def _check(o, S, ref, cu, tol, heads=None, label=""):
    if heads is not None:
        o = o[:, heads]
        S = S[:, heads]
    eo = max_block_err_o(o, ref["o"], cu)
    eS = max_block_err_S(S, ref["S"])
    print(f"{label}: max normwise err o={eo:.3e} S={eS:.3e} (tol {tol:g})")
    assert eo <= tol and eS <= tol, (eo, eS)
    return eo, eS


@pytest.mark.parametrize("act", [0, 1])
def test_tiny_fp32_chunk16(act):
    """1 sequence, L = 64, 2 heads, d = 32, chunk 16, fp32 inputs, zero states: 1e-5."""
    announce(f"prefill tiny fp32 act={act}")
    inp = make_prefill(TINY_FP32)
    run = PrefillRun(inp, act=act)
    o, S = run.run()
    ref = _oracle(inp, "silu" if act else "none")
    _check(o, S, ref, inp["cu_seqlens"], TOL_F32, label="tiny fp32")
    np.testing.assert_array_equal(storage_of(run.pool.conv_state, "f32")[0], ref["conv_state"][0].astype(np.float32))


@pytest.mark.parametrize("d,chunk,mma,in_dtype", [
    (64, 64, 2, "bf16"), (64, 32, 2, "bf16"), (32, 16, 2, "bf16"), (128, 64, 1, "bf16"), (64, 32, 1, "f32"),
    (128, 32, 1, "f32"), (32, 64, 1, "f32"),
])
def test_ragged_small_shapes(d, chunk, mma, in_dtype):
    announce(f"prefill ragged d={d} chunk={chunk} mma={mma} {in_dtype}")
    shape = LayerShape(2, 4, d, conv_width=4, chunk=chunk, in_dtype=in_dtype)
    lens = (1, 17, 64, 0, 33, 100, 2)
    inp = make_prefill(RAGGED_T15717, lens=lens, shape=shape, s0_std=0.05, conv_state_std=1.0)
    o, S = PrefillRun(inp, mma=mma).run()
    ref = _oracle(inp)
    tol = TOL_F32 if in_dtype == "f32" else TOL_BF16
    _check(o, S, ref, inp["cu_seqlens"], tol, label=f"ragged d={d} C={chunk}")
    # the empty sequence keeps its state
    np.testing.assert_array_equal(S[3], inp["S0"][3])


def _check_full_size(run, inp, label):
    """Every v-head of every sequence against the oracle (sharded over host processes),
    and the committed conv state of every sequence bit for bit."""
    from gen import bf16_bits_from_f32

    o, S = run.run()
    ref = _oracle(inp)
    _check(o, S, ref, inp["cu_seqlens"], TOL_BF16, label=label)
    np.testing.assert_array_equal(storage_of(run.pool.conv_state, "bf16"),
                                  bf16_bits_from_f32(ref["conv_state"].astype(np.float32)))


def test_prefill_L4096_full_size_all_heads():
    """One 4096-token sequence, 16/32 heads, d = 128, bf16, chunk 64 (the benchmark's
    launch): all 32 v-heads against the oracle over the whole sequence."""
    announce("prefill L=4096 full size, all heads")
    inp = make_prefill(PREFILL_L4096)
    _check_full_size(PrefillRun(inp), inp, "L4096 all heads")


def test_ragged_T15717_full_size_all_heads():
    """8 packed sequences {1,17,64,300,1000,2048,4095,8192}, nonzero initial conv and
    recurrent states, bf16, chunk 64: every (sequence, v-head) against the oracle and
    every sequence's conv state bit for bit."""
    announce("prefill ragged T=15717 full size, all heads")
    inp = make_prefill(RAGGED_T15717)
    _check_full_size(PrefillRun(inp), inp, "T15717 all heads")


def test_packed_equals_solo_bit_exact():
    """Chunks start at each sequence's own first token, so a sequence packed with others
    gives the same bits as the sequence alone."""
    announce("prefill packed vs solo bit-exact")
    shape = LayerShape(2, 4, 128, conv_width=4, chunk=64, in_dtype="bf16")
    lens = (5, 130, 64, 1, 77)
    inp = make_prefill(RAGGED_T15717, lens=lens, shape=shape, s0_std=0.05, conv_state_std=1.0)
    o, S = PrefillRun(inp).run()
    cu = inp["cu_seqlens"]
    for s in (1, 4, 3):
        a, b = cu[s], cu[s + 1]
        solo = dict(inp, x=inp["x"][a:b], cu_seqlens=np.array([0, b - a], dtype=np.int32),
                    conv_state=inp["conv_state"][s:s + 1], S0=inp["S0"][s:s + 1], g=inp["g"][a:b],
                    beta=inp["beta"][a:b], lens=(lens[s],))
        o1, S1 = PrefillRun(solo).run()
        np.testing.assert_array_equal(o1.view(np.int32), o[a:b].view(np.int32))
        np.testing.assert_array_equal(S1[0].view(np.int32), S[s].view(np.int32))


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_one_and_two_workgroups_per_cu_variants_bit_exact(in_dtype):
    """The inter-chunk launch has two variants with the same arithmetic: below 512 16-row
    blocks one block per workgroup, from 512 on two blocks of a head per workgroup (one set
    of operand loads for both). At 16/32 heads and d = 128 a sequence alone has 256 blocks
    and packed with a second sequence 512, so the two runs take different variants; the
    sequence's o and state must agree bit for bit, with either product precision (bf16x3
    for bf16 input, fp32 MFMA for fp32 input)."""
    announce(f"prefill inter variants (one vs two 16-row blocks per workgroup) bit-exact, {in_dtype}")
    lens = (300, 130)
    shape = LayerShape(16, 32, 128, conv_width=4, chunk=64, in_dtype=in_dtype)
    inp = make_prefill(PREFILL_L4096, lens=lens, shape=shape, s0_std=0.02, conv_state_std=1.0)
    o, S = PrefillRun(inp).run()
    solo = dict(inp, x=inp["x"][:300], cu_seqlens=np.array([0, 300], dtype=np.int32),
                conv_state=inp["conv_state"][:1], S0=inp["S0"][:1], g=inp["g"][:300], beta=inp["beta"][:300],
                lens=(300,))
    o1, S1 = PrefillRun(solo).run()
    np.testing.assert_array_equal(o1.view(np.int32), o[:300].view(np.int32))
    np.testing.assert_array_equal(S1[0].view(np.int32), S[0].view(np.int32))
    ref = _oracle(inp)
    _check(o, S, ref, inp["cu_seqlens"], TOL_BF16 if in_dtype == "bf16" else TOL_F32, label="two blocks per workgroup")


def test_split_and_decode_continuation():
    """prefill(L1) then prefill(L2) and prefill(L) then decode continue the same sequence
    (chunk boundaries differ, so this is a tolerance check against the oracle's full run)."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    announce("prefill split + decode continuation")
    shape = LayerShape(2, 4, 128, conv_width=4, chunk=64, in_dtype="bf16")
    inp = make_prefill(RAGGED_T15717, lens=(150,), shape=shape, s0_std=0.05, conv_state_std=1.0)
    ref = _oracle(inp)
    L1 = 70
    first = dict(inp, x=inp["x"][:L1], cu_seqlens=np.array([0, L1], dtype=np.int32), g=inp["g"][:L1],
                 beta=inp["beta"][:L1], lens=(L1,))
    r1 = PrefillRun(first)
    o1, _ = r1.run()
    second = dict(inp, x=inp["x"][L1:149], cu_seqlens=np.array([0, 149 - L1], dtype=np.int32),
                  g=inp["g"][L1:149], beta=inp["beta"][L1:149], lens=(149 - L1,))
    r2 = PrefillRun(second)
    r2.pool.state.copy_(r1.pool.state)
    r2.pool.conv_state.copy_(r1.pool.conv_state)
    o2, _ = r2.run()
    # the last token through the decode path
    y = torch.empty((1, shape.channels), dtype=torch.float32, device="cuda")
    o3 = torch.empty((1, 4, 128), dtype=torch.float32, device="cuda")
    gdn.conv_update(r2.dims, to_dev(inp["x"][149:150], "bf16"), y, r2.w, None, r2.cp)
    gdn.decode(r2.dims, y, to_dev(inp["g"][149:150], "f32"), to_dev(inp["beta"][149:150], "f32"), o3, r2.sp)
    torch.cuda.synchronize()
    o_all = np.concatenate([o1, o2, o3.cpu().numpy()])
    S = r2.pool.state.cpu().numpy()
    _check(o_all, S, ref, inp["cu_seqlens"], TOL_BF16, label="split+decode")


def test_strong_decay_stays_finite():
    """g = -50 on every token: every decay factor is e^(gam_t - gam_s) with t >= s, so
    nothing overflows; the state forgets its past within a token."""
    announce("prefill strong decay")
    shape = LayerShape(2, 4, 64, conv_width=4, chunk=64, in_dtype="bf16")
    inp = make_prefill(RAGGED_T15717, lens=(130, 7), shape=shape, s0_std=0.05, conv_state_std=1.0)
    g = np.full_like(inp["g"], -50.0)
    o, S = PrefillRun(inp, g=g).run()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))  # (and every value checked below)
    ref = _oracle(inp, g=g)
    _check(o, S, ref, inp["cu_seqlens"], TOL_BF16, label="g=-50")


def test_run_twice_is_deterministic():
    announce("prefill determinism")
    shape = LayerShape(2, 4, 128, conv_width=4, chunk=64, in_dtype="bf16")
    inp = make_prefill(RAGGED_T15717, lens=(3, 200, 64), shape=shape, s0_std=0.05, conv_state_std=1.0)
    a = PrefillRun(inp).run()
    b = PrefillRun(inp).run()
    for x, y in zip(a, b):
        np.testing.assert_array_equal(bits_of_np(x), bits_of_np(y))


def bits_of_np(a):
    return np.ascontiguousarray(a).view(np.int32)


def test_many_short_sequences():
    """1100 packed sequences of 0..5 tokens (zero-length ones included): the chunk table
    scans more than one 1024-sequence tile and skips the longest-first ordering (more than
    256 sequences). Every sequence is checked against the oracle, and zero-length
    sequences keep their state bits."""
    announce("prefill 1100 short sequences, fp32, d=32, chunk 16")
    rng = np.random.default_rng(77)
    lens = tuple(int(v) for v in rng.integers(0, 6, size=1100))
    shape = LayerShape(2, 2, 32, conv_width=4, chunk=16, in_dtype="f32")
    inp = make_prefill(TINY_FP32, lens=lens, shape=shape, s0_std=0.05, conv_state_std=1.0)
    run = PrefillRun(inp)
    o, S = run.run()
    ref = _oracle(inp)
    _check(o, S, ref, inp["cu_seqlens"], TOL_F32, label="1100 seqs")
    empty = [i for i, n in enumerate(lens) if n == 0]
    assert empty
    np.testing.assert_array_equal(S[empty].view(np.int32), inp["S0"][empty].view(np.int32))
