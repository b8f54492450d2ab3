"""The rule's defining special cases on the GPU, through every entry point, against the
oracle at the parity gates.

The cases (the pins the oracle itself is held to, now run through the kernels):
  * g0     : g = 0 on every token (no decay inside or across chunks), beta and keys random;
  * beta0  : beta = 0 (pure decay: S_t = e^{sum g} S_0, o_t = e^{gam_t} S_0 q^_t), slow decay;
  * orth   : g = 0, beta = 1, the keys of every chunk mutually orthogonal (associative
             memory: S k_i = v_i after the writes);
  * repeat : g = 0, beta = 1, one key repeated over each whole chunk (every write
             overwrites the last: S k = v of the chunk's last token);
  * mixed  : per token a random choice among the above.
Keys are rows of a Sylvester Hadamard matrix: +-1 entries (exact in bf16) whose rows are
mutually orthogonal, made unit by the kernels' own L2 norm. The conv taps are the identity
(w = e_{K-1}), so the conv output is x exactly and the fused entry points see the same
q, k, v as the two-call ones. ("System Design", "GDN Kernel Dispatch Detail": conv, L2
norm, then the gated delta rule, in prefill and in decode.)

A further case runs q scale != 1 with the L2 norm on through prefill and then decode.
"""

import numpy as np
import pytest

from gen import bf16_bits_from_f32
from gen.inputs import LayerShape
from oracle import prefill_layer
from tests.gpu_helpers import (TOL_BF16, TOL_F32, announce, bits_of, max_block_err_o, max_block_err_S, normwise_err,
                               storage_of, to_dev)
from tests.oracle_pool import prefill_all_heads

pytestmark = pytest.mark.gpu

CASES = ("g0", "beta0", "orth", "repeat", "mixed")
SLOW = 0.01  # beta0 and mixed: g = -softplus(z) * 0.01, so the state lives across the sequence


def _hadamard(d):
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def _store(a, dtype):
    return bf16_bits_from_f32(np.asarray(a, np.float32)) if dtype == "bf16" else np.asarray(a, np.float32)


def edge_inputs(case, shape, lens, seed=0):
    """A packed batch shaped like gen.make_prefill's output, with the case's keys, g and
    beta, identity conv taps and random conv states (which the identity taps ignore)."""
    r = np.random.default_rng([4242, CASES.index(case), seed])
    Hk, Hv, d, C, K = shape.num_k_heads, shape.num_v_heads, shape.head_dim, shape.chunk, shape.conv_width
    N, T = len(lens), int(sum(lens))
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    H = _hadamard(d)
    q = r.standard_normal((T, Hk, d))
    k = np.empty((T, Hk, d))
    v = r.standard_normal((T, Hv, d))
    g = -np.logaddexp(0.0, r.standard_normal((T, Hv)))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((T, Hv))))
    kind = np.full(T, case) if case != "mixed" else r.choice(["g0", "beta0", "orth", "repeat", "rand"], size=T)
    for s in range(N):
        for t in range(cu[s], cu[s + 1]):
            p = t - cu[s]  # position in the sequence (chunks start at the sequence start)
            for h in range(Hk):
                if kind[t] in ("orth",):
                    k[t, h] = H[(p + 7 * h) % d]
                elif kind[t] == "repeat":
                    k[t, h] = H[(5 * (p // C) + 3 * h) % d]
                else:
                    k[t, h] = r.standard_normal(d)
    for t in range(T):
        if kind[t] == "g0":
            g[t] = 0.0
        elif kind[t] == "beta0":
            beta[t] = 0.0
            g[t] *= SLOW
        elif kind[t] in ("orth", "repeat"):
            g[t] = 0.0
            beta[t] = 1.0
        else:
            g[t] *= SLOW
    x = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
    w = np.zeros((shape.channels, K))
    w[:, K - 1] = 1.0
    return dict(shape=shape, lens=tuple(lens), x=_store(x, shape.in_dtype), conv_w=_store(w, shape.in_dtype),
                conv_b=None, cu_seqlens=cu,
                conv_state=_store(r.standard_normal((N, K - 1, shape.channels)), shape.in_dtype),
                g=g.astype(np.float32), beta=beta.astype(np.float32),
                S0=(r.standard_normal((N, Hv, d, d)) * 0.05).astype(np.float32))


def _dims(shape, mma=0, form=0, scale=1.0):
    import gated_delta_rule_conv_amd as gdn

    return gdn.make_dims(shape.num_k_heads, shape.num_v_heads, shape.head_dim, conv_width=shape.conv_width,
                         chunk_size=shape.chunk, mma=mma, prefill_form=form, scale=scale,
                         in_dtype=gdn.GDN_BF16 if shape.in_dtype == "bf16" else gdn.GDN_F32)


def run_prefill(inp, dims, fused):
    """The batch through conv_update + prefill_chunked, or prefill_fused; returns o, the
    states and the conv states (bits)."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    sh = inp["shape"]
    N, T = len(inp["lens"]), int(inp["cu_seqlens"][-1])
    pool = gdn.SlotPool(dims, N, state=to_dev(inp["S0"], "f32"), conv_state=to_dev(inp["conv_state"], sh.in_dtype))
    sp, cp = pool.pointers(torch.arange(N, dtype=torch.int32, device="cuda"))
    cu = torch.tensor(inp["cu_seqlens"], dtype=torch.int32, device="cuda")
    x, w = to_dev(inp["x"], sh.in_dtype), to_dev(inp["conv_w"], sh.in_dtype)
    g, beta = to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32")
    o = torch.full((T, sh.num_v_heads, sh.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    if fused:
        ws = gdn.prefill_fused_workspace(dims, N, T)
        gdn.prefill_fused(dims, x, w, None, g, beta, o, cu, sp, cp, ws)
    else:
        y = torch.empty((T, sh.channels), dtype=torch.float32, device="cuda")
        gdn.conv_update(dims, x, y, w, None, cp, cu)
        gdn.prefill(dims, y, g, beta, o, cu, sp, gdn.prefill_workspace(dims, N, T))
    torch.cuda.synchronize()
    return o.cpu().numpy(), pool.state.cpu().numpy(), storage_of(pool.conv_state, sh.in_dtype), pool


def _gate(o, S, ref, cu, tol, label):
    eo, eS = max_block_err_o(o, ref["o"], cu), max_block_err_S(S, ref["S"])
    print(f"{label}: max normwise err o={eo:.3e} S={eS:.3e} (tol {tol:g})")
    assert eo <= tol and eS <= tol, (label, eo, eS)


def _conv_state_ref(ref, dtype):
    return _store(ref["conv_state"], dtype)


# (shape, lens, mma): d = 128 chunk 64 bf16 inputs on bf16x3 and fp32 inputs on fp32 MFMA,
# and a d = 32 chunk 16 fp32 layer; the 600-token sequence has 10 chunks, so the
# chunk-parallel form cuts it into segments
SHAPES = [
    (LayerShape(2, 4, 128, conv_width=4, chunk=64, in_dtype="bf16"), (64, 600, 1, 130), 2),
    (LayerShape(2, 4, 128, conv_width=4, chunk=64, in_dtype="f32"), (64, 600, 1, 130), 1),
    (LayerShape(1, 2, 32, conv_width=3, chunk=16, in_dtype="f32"), (16, 200, 3), 1),
]


@pytest.mark.parametrize("form", [1, 2])
@pytest.mark.parametrize("si", range(len(SHAPES)))
@pytest.mark.parametrize("case", CASES)
def test_prefill_edge_case(case, si, form):
    shape, lens, mma = SHAPES[si]
    announce(f"prefill edge case {case}: d={shape.head_dim} C={shape.chunk} {shape.in_dtype} mma={mma} "
             f"form={form} lens={lens}")
    inp = edge_inputs(case, shape, lens)
    ref = prefill_all_heads(inp)
    o, S, cs, _ = run_prefill(inp, _dims(shape, mma=mma, form=form), fused=False)
    tol = TOL_F32 if mma == 1 else TOL_BF16
    _gate(o, S, ref, inp["cu_seqlens"], tol, f"{case} form={form}")
    np.testing.assert_array_equal(cs, _conv_state_ref(ref, shape.in_dtype))


@pytest.mark.parametrize("case", CASES)
def test_prefill_fused_edge_case(case):
    """The one-call prefill (q/k conv inside the intra-chunk kernel) on the same cases:
    the same bits as the two calls, and the oracle's values."""
    shape, lens, mma = SHAPES[0]
    announce(f"prefill_fused edge case {case}")
    inp = edge_inputs(case, shape, lens, seed=1)
    dims = _dims(shape)
    o2, S2, cs2, _ = run_prefill(inp, dims, fused=False)
    o1, S1, cs1, _ = run_prefill(inp, dims, fused=True)
    np.testing.assert_array_equal(o1.view(np.int32), o2.view(np.int32))
    np.testing.assert_array_equal(S1.view(np.int32), S2.view(np.int32))
    np.testing.assert_array_equal(cs1, cs2)
    ref = prefill_all_heads(inp)
    _gate(o1, S1, ref, inp["cu_seqlens"], TOL_BF16, f"fused {case}")
    np.testing.assert_array_equal(cs1, _conv_state_ref(ref, shape.in_dtype))


def run_decode(inp, dims, fused, m):
    """Sequence s of the batch fed to slot s one token per call (every sequence has the
    same length): decode_batched after conv_update, or decode_fused. Returns o [T, Hv, d]
    in packed order and the final states."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    sh = inp["shape"]
    L = inp["lens"][0]
    assert all(n == L for n in inp["lens"]) and len(inp["lens"]) == m
    pool = gdn.SlotPool(dims, m + 2, state=torch.zeros((m + 2, sh.num_v_heads, sh.head_dim, sh.head_dim),
                                                       dtype=torch.float32, device="cuda"))
    pool.state[1:m + 1].copy_(to_dev(inp["S0"], "f32"))
    pool.conv_state[1:m + 1].copy_(to_dev(inp["conv_state"], sh.in_dtype))
    sp, cp = pool.pointers(torch.arange(1, m + 1, dtype=torch.int32, device="cuda"))  # slot s + 1 <-> sequence s
    x, w = to_dev(inp["x"], sh.in_dtype), to_dev(inp["conv_w"], sh.in_dtype)
    g, beta = to_dev(inp["g"], "f32"), to_dev(inp["beta"], "f32")
    rows = torch.tensor([[s * L + t for s in range(m)] for t in range(L)], dtype=torch.int64, device="cuda")
    o = torch.empty((L, m, sh.num_v_heads, sh.head_dim), dtype=torch.float32, device="cuda")
    y = torch.empty((m, sh.channels), dtype=torch.float32, device="cuda")
    for t in range(L):
        xt, gt, bt = x[rows[t]].contiguous(), g[rows[t]].contiguous(), beta[rows[t]].contiguous()
        if fused:
            gdn.decode_fused(dims, xt, w, None, gt, bt, o[t], sp, cp)
        else:
            gdn.conv_update(dims, xt, y, w, None, cp)
            gdn.decode(dims, y, gt, bt, o[t], sp)
    torch.cuda.synchronize()
    on = o.cpu().numpy().transpose(1, 0, 2, 3).reshape(m * L, sh.num_v_heads, sh.head_dim)
    return on, pool.state[1:m + 1].cpu().numpy(), storage_of(pool.conv_state[1:m + 1], sh.in_dtype), pool


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES)
def test_decode_edge_case(case, in_dtype, fused):
    """4 slots, 70 decode steps each (more than one chunk's worth of keys: the orth keys
    wrap, the repeated key changes every 64 tokens)."""
    shape = LayerShape(2, 4, 128, conv_width=4, chunk=64, in_dtype=in_dtype)
    m, L = 4, 70
    announce(f"decode edge case {case} {in_dtype} {'fused' if fused else 'two calls'}")
    inp = edge_inputs(case, shape, (L,) * m, seed=2)
    o, S, cs, pool = run_decode(inp, _dims(shape), fused, m)
    ref = prefill_all_heads(inp)
    tol = TOL_F32 if in_dtype == "f32" else TOL_BF16
    _gate(o, S, ref, inp["cu_seqlens"], tol, f"decode {case} {in_dtype} fused={fused}")
    np.testing.assert_array_equal(cs, _conv_state_ref(ref, in_dtype))
    # the slots around the active ones were never touched
    assert not pool.state[0].any().item() and not pool.state[m + 1].any().item()


def test_scale_with_norm_on_prefill_then_decode():
    """q scale 0.37 with the L2 norm on, through prefill (two calls and fused) and then 5
    decode steps (both entry points): q^ = 0.37 q / |q|, the states never see the scale."""
    import torch

    import gated_delta_rule_conv_amd as gdn
    from gen import RAGGED_T15717, make_prefill

    c = 0.37
    shape = LayerShape(2, 4, 128, conv_width=4, chunk=64, in_dtype="bf16")
    announce(f"scale {c} with the L2 norm on: prefill then decode")
    L1, L2 = 200, 5
    full = make_prefill(RAGGED_T15717, lens=(L1 + L2,) * 2, shape=shape, s0_std=0.05, conv_state_std=1.0)
    ref = prefill_layer(full["x"], full["conv_w"], full["cu_seqlens"], full["conv_state"], full["S0"], full["g"],
                        full["beta"], 2, 4, 128, in_dtype="bf16", scale=c)
    ref1 = prefill_layer(full["x"], full["conv_w"], full["cu_seqlens"], full["conv_state"], full["S0"], full["g"],
                         full["beta"], 2, 4, 128, in_dtype="bf16")
    assert normwise_err(ref["o"], c * ref1["o"]) < 1e-12  # (the oracle's own pin, restated at this size)
    cu = full["cu_seqlens"]
    first = np.concatenate([np.arange(cu[s], cu[s] + L1) for s in range(2)])
    part = dict(full, x=full["x"][first], g=full["g"][first], beta=full["beta"][first], lens=(L1, L1),
                cu_seqlens=np.array([0, L1, 2 * L1], dtype=np.int32))
    dims = _dims(shape, scale=c)
    for fused in (False, True):
        o1, _, _, pool = run_prefill(part, dims, fused=fused)
        sp, cp = pool.pointers(torch.arange(2, dtype=torch.int32, device="cuda"))
        w = to_dev(full["conv_w"], "bf16")
        outs = []
        for t in range(L2):
            rows = [cu[s] + L1 + t for s in range(2)]
            x = to_dev(full["x"][rows], "bf16")
            g, beta = to_dev(full["g"][rows], "f32"), to_dev(full["beta"][rows], "f32")
            o = torch.empty((2, 4, 128), dtype=torch.float32, device="cuda")
            if fused:
                gdn.decode_fused(dims, x, w, None, g, beta, o, sp, cp)
            else:
                y = torch.empty((2, shape.channels), dtype=torch.float32, device="cuda")
                gdn.conv_update(dims, x, y, w, None, cp)
                gdn.decode(dims, y, g, beta, o, sp)
            outs.append(o.cpu().numpy())
        torch.cuda.synchronize()
        o_all = np.zeros_like(ref["o"])
        for s in range(2):
            o_all[cu[s]:cu[s] + L1] = o1[s * L1:(s + 1) * L1]
            for t in range(L2):
                o_all[cu[s] + L1 + t] = outs[t][s]
        _gate(o_all, pool.state.cpu().numpy(), ref, cu, TOL_BF16, f"scale {c} fused={fused}")
        np.testing.assert_array_equal(storage_of(pool.conv_state, "bf16"), _store(ref["conv_state"], "bf16"))
        # (bits of the state do not depend on the scale: compared with a scale-1 run)
        if not fused:
            _, S_unscaled, _, _ = run_prefill(part, _dims(shape), fused=False)
            _, S_scaled, _, _ = run_prefill(part, dims, fused=False)
            np.testing.assert_array_equal(bits_of(torch.from_numpy(S_scaled)), bits_of(torch.from_numpy(S_unscaled)))
