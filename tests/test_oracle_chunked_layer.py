"""Chunked form == recurrent form, and layer-level invariants of the oracle.

("System Design", "GDN Kernel Dispatch Detail": prefill runs a chunked kernel over
(q, k, v, g, beta, state) and updates the temporal state; decode is the
single-token update. "aprender #5279", "Phase plan": ragged lengths must give the
per-slot result.)
"""

import numpy as np
import pytest

from gen import TINY_FP32, make_prefill
from gen.inputs import LayerShape
from oracle import decode_layer, gated_delta_chunked, gated_delta_recurrent, l2norm, prefill_layer

rng = np.random.default_rng(5)


def _problem(L, Hk, Hv, d, g_scale=1.0):
    q = l2norm(rng.standard_normal((L, Hk, d)), 1e-6)
    k = l2norm(rng.standard_normal((L, Hk, d)), 1e-6)
    v = rng.standard_normal((L, Hv, d))
    g = -np.logaddexp(0, rng.standard_normal((L, Hv))) * g_scale
    beta = 1 / (1 + np.exp(-rng.standard_normal((L, Hv))))
    S0 = rng.standard_normal((Hv, d, d)) * 0.05
    return q, k, v, g, beta, S0


@pytest.mark.parametrize("chunk", [16, 64])
@pytest.mark.parametrize("L", [1, 15, 16, 17, 64, 100, 130])
def test_chunked_equals_recurrent(chunk, L):
    q, k, v, g, beta, S0 = _problem(L, 2, 4, 16)
    o1, S1 = gated_delta_recurrent(q, k, v, g, beta, S0)
    o2, S2 = gated_delta_chunked(q, k, v, g, beta, S0, chunk)
    scale_o = np.abs(o1).max()
    assert np.abs(o1 - o2).max() <= 1e-12 * max(scale_o, 1)
    assert np.abs(S1 - S2).max() <= 1e-12 * max(np.abs(S1).max(), 1)


def test_chunked_equals_recurrent_d128_slow_decay():
    """Long memory: g = -softplus(z) * 0.01 keeps the state alive across chunks."""
    q, k, v, g, beta, S0 = _problem(300, 1, 1, 128, g_scale=0.01)
    o1, S1 = gated_delta_recurrent(q, k, v, g, beta, S0)
    o2, S2 = gated_delta_chunked(q, k, v, g, beta, S0, 64)
    assert np.abs(o1 - o2).max() <= 1e-11 * np.abs(o1).max()
    assert np.abs(S1 - S2).max() <= 1e-11 * np.abs(S1).max()


def test_strong_decay_stays_finite_and_forgets():
    """g = -50 per token: every factor exp(gam_t - gam_s), t >= s, stays finite and
    the chunked form still agrees; with beta = 0 the state decays to 0."""
    L = 70
    q, k, v, g, beta, S0 = _problem(L, 1, 1, 8)
    g[:] = -50.0
    o1, S1 = gated_delta_recurrent(q, k, v, g, beta, S0)
    o2, S2 = gated_delta_chunked(q, k, v, g, beta, S0, 64)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(S2))
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S2, S1, rtol=1e-10, atol=1e-12)
    _, S3 = gated_delta_chunked(q, k, v, g, np.zeros_like(beta), S0, 64)
    assert np.abs(S3).max() == 0.0


def _layer_inputs(lens, Hk=1, Hv=2, d=8, in_dtype="f32"):
    shape = LayerShape(Hk, Hv, d, conv_width=4, chunk=16, in_dtype=in_dtype)
    return make_prefill(TINY_FP32, lens=lens, shape=shape, s0_std=0.1, conv_state_std=1.0)


def _run(inp, cu=None, **kw):
    sh = inp["shape"]
    return prefill_layer(inp["x"], inp["conv_w"], inp["cu_seqlens"] if cu is None else cu, inp["conv_state"],
                         inp["S0"], inp["g"], inp["beta"], sh.num_k_heads, sh.num_v_heads, sh.head_dim,
                         in_dtype=sh.in_dtype, **kw)


def test_split_invariance_prefill_then_prefill():
    """prefill(L1) then prefill(L2) from the carried conv state and state == prefill(L1 + L2)."""
    inp = _layer_inputs([23])
    sh = inp["shape"]
    full = _run(inp)
    L1 = 9
    a = prefill_layer(inp["x"][:L1], inp["conv_w"], [0, L1], inp["conv_state"], inp["S0"], inp["g"][:L1],
                      inp["beta"][:L1], sh.num_k_heads, sh.num_v_heads, sh.head_dim)
    b = prefill_layer(inp["x"][L1:], inp["conv_w"], [0, 23 - L1], a["conv_state"], a["S"], inp["g"][L1:],
                      inp["beta"][L1:], sh.num_k_heads, sh.num_v_heads, sh.head_dim)
    np.testing.assert_allclose(np.concatenate([a["o"], b["o"]]), full["o"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b["S"], full["S"], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(b["conv_state"], full["conv_state"])


def test_prefill_then_decode_equals_longer_prefill():
    inp = _layer_inputs([12])
    sh = inp["shape"]
    full = _run(inp)
    L = 11
    a = prefill_layer(inp["x"][:L], inp["conv_w"], [0, L], inp["conv_state"], inp["S0"], inp["g"][:L],
                      inp["beta"][:L], sh.num_k_heads, sh.num_v_heads, sh.head_dim)
    b = decode_layer(inp["x"][L:], inp["conv_w"], a["conv_state"], a["S"], inp["g"][L:], inp["beta"][L:],
                     sh.num_k_heads, sh.num_v_heads, sh.head_dim)
    np.testing.assert_allclose(b["o"][0], full["o"][L], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b["S"], full["S"], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(b["conv_state"], full["conv_state"])


def test_packed_equals_solo_and_chunked_layer_equals_recurrent():
    lens = [1, 5, 16, 3, 0, 40]
    inp = _layer_inputs(lens, Hk=2, Hv=4)
    sh = inp["shape"]
    packed = _run(inp)
    chunked = _run(inp, chunk=16)
    np.testing.assert_allclose(chunked["o"], packed["o"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(chunked["S"], packed["S"], rtol=1e-11, atol=1e-12)
    cu = inp["cu_seqlens"]
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        solo = prefill_layer(inp["x"][a:b], inp["conv_w"], [0, b - a], inp["conv_state"][s:s + 1],
                             inp["S0"][s:s + 1], inp["g"][a:b], inp["beta"][a:b], sh.num_k_heads,
                             sh.num_v_heads, sh.head_dim)
        np.testing.assert_array_equal(solo["o"], packed["o"][a:b])
        np.testing.assert_array_equal(solo["S"][0], packed["S"][s])
    # an empty sequence leaves both of its states untouched
    np.testing.assert_array_equal(packed["S"][4], inp["S0"][4])
    np.testing.assert_array_equal(packed["conv_state"][4], inp["conv_state"][4])


def test_output_is_homogeneous_in_the_input_from_zero_state():
    """eps = 0, zero states: conv is linear, q^ and k^ are scale-free and o is linear in
    v, so o(c x) = c o(x) for c > 0 (and S scales the same way)."""
    inp = _layer_inputs([20])
    sh = inp["shape"]
    args = (inp["conv_w"], inp["cu_seqlens"], np.zeros_like(inp["conv_state"]), np.zeros_like(inp["S0"]),
            inp["g"], inp["beta"], sh.num_k_heads, sh.num_v_heads, sh.head_dim)
    a = prefill_layer(inp["x"], *args, eps=0.0)
    b = prefill_layer(inp["x"] * 4.0, *args, eps=0.0)  # power of two: exact in fp32
    np.testing.assert_allclose(b["o"], 4.0 * a["o"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b["S"], 4.0 * a["S"], rtol=1e-12, atol=1e-13)


def test_head_subset_matches_full():
    inp = _layer_inputs([10], Hk=2, Hv=4)
    full = _run(inp)
    sub = _run(inp, v_heads=[1, 3])
    np.testing.assert_array_equal(sub["o"], full["o"][:, [1, 3]])
    np.testing.assert_array_equal(sub["S"], full["S"][:, [1, 3]])


def test_bf16_inputs_decode_exactly():
    inp = _layer_inputs([4], in_dtype="bf16")
    assert inp["x"].dtype == np.uint16
    out = _run(inp)
    assert np.all(np.isfinite(out["o"]))


def test_qk_l2norm_off_skips_only_the_norm():
    """With identity conv taps (w = e_{K-1}, so y = x) and q, k head vectors of x that are
    unit vectors already, the layer without the L2 norm equals the layer with it at eps = 0
    (to fp32 rounding of the inputs); and without the norm o is linear in q (the norm would
    cancel a scale of q's channels), while the state does not depend on q at all."""
    inp = _layer_inputs([19, 5])
    sh = inp["shape"]
    d, Hk = sh.head_dim, sh.num_k_heads
    C = sh.channels
    w = np.zeros((C, sh.conv_width), dtype=np.float32)
    w[:, -1] = 1.0
    x = np.array(inp["x"], dtype=np.float64)
    qk = x[:, :2 * Hk * d].reshape(len(x), 2 * Hk, d)
    x[:, :2 * Hk * d] = (qk / np.linalg.norm(qk, axis=-1, keepdims=True)).reshape(len(x), -1)
    x = x.astype(np.float32)
    base = dict(inp, x=x, conv_w=w)
    on = _run(base, eps=0.0)
    off = _run(base, eps=0.0, qk_l2norm=False)
    np.testing.assert_allclose(off["o"], on["o"], rtol=0, atol=1e-5 * np.abs(on["o"]).max())
    np.testing.assert_allclose(off["S"], on["S"], rtol=0, atol=1e-5 * np.abs(on["S"]).max())
    x2 = x.copy()
    x2[:, :Hk * d] *= 2.0  # q channels only (exact in fp32)
    off2 = _run(dict(base, x=x2), eps=0.0, qk_l2norm=False)
    on2 = _run(dict(base, x=x2), eps=0.0)
    np.testing.assert_allclose(off2["o"], 2.0 * off["o"], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(off2["S"], off["S"])
    np.testing.assert_allclose(on2["o"], on["o"], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("c", [0.25, 3.0])
def test_scale_multiplies_output_only_with_norm_on(c):
    """q^ = scale * q / sqrt(|q|^2 + eps): with the norm on, o is linear in q^ and the
    state never sees q, so scale = c gives o(c) = c * o(1) and the same final states.
    A reading that scales q before the norm (where the factor cancels) gives o(c) = o(1)
    and fails the first check; one that scales k changes the states and fails the second."""
    inp = _layer_inputs([5, 37, 1], Hk=2, Hv=4, d=8)
    base = _run(inp)
    scaled = _run(inp, scale=c)
    if c == 0.25:  # a power of two: every product is exact, so the bits agree
        np.testing.assert_array_equal(scaled["o"], c * base["o"])
    else:
        np.testing.assert_allclose(scaled["o"], c * base["o"], rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(scaled["S"], base["S"])
    np.testing.assert_array_equal(scaled["conv_state"], base["conv_state"])
    assert np.abs(base["o"]).max() > 0.1  # (the check is not vacuous)
