"""Pins for the oracle's causal conv, conv-state update and L2 norm.

Each check compares the oracle with something other than itself: numpy.convolve,
shift kernels whose output is known in closed form, scipy's logistic function, or
the norm identity. ("System Design", "GDN Kernel Dispatch Detail": depthwise
causal Conv1d, conv state update in decode, L2 normalisation of q and k.)
"""

import numpy as np
import pytest
from scipy.special import expit

from oracle import causal_conv, l2norm, prefill_layer
from oracle.gdn import bf16_bits_to_f64

rng = np.random.default_rng(7)


@pytest.mark.parametrize("L", [1, 2, 3, 5, 17])
@pytest.mark.parametrize("K", [2, 3, 4])
def test_conv_matches_numpy_convolve_zero_state(L, K):
    C = 6
    x = rng.standard_normal((L, C))
    w = rng.standard_normal((C, K))
    y, _ = causal_conv(x, w)
    for c in range(C):
        # cross-correlation with K-1 zeros on the left == convolution with the
        # reversed taps, first L outputs
        ref = np.convolve(x[:, c], w[c, ::-1])[:L]
        np.testing.assert_allclose(y[:, c], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("L", [1, 2, 4, 9])
def test_conv_matches_numpy_convolve_with_state(L):
    C, K = 5, 4
    x = rng.standard_normal((L, C))
    st = rng.standard_normal((K - 1, C))
    w = rng.standard_normal((C, K))
    b = rng.standard_normal(C)
    y, _ = causal_conv(x, w, b, st)
    for c in range(C):
        z = np.concatenate([st[:, c], x[:, c]])
        ref = np.convolve(z, w[c, ::-1], mode="valid") + b[c]
        np.testing.assert_allclose(y[:, c], ref, rtol=1e-13, atol=1e-13)


def test_shift_kernels_pin_tap_and_state_order():
    C, K, L = 4, 4, 7
    x = rng.standard_normal((L, C))
    st = rng.standard_normal((K - 1, C))
    # w = e_{K-1}: the last tap multiplies the current token -> identity
    w = np.zeros((C, K))
    w[:, K - 1] = 1.0
    y, _ = causal_conv(x, w, None, st)
    np.testing.assert_array_equal(y, x)
    # w = e_0: y_t = z_t, so the first K-1 outputs replay the conv state oldest first
    w = np.zeros((C, K))
    w[:, 0] = 1.0
    y, _ = causal_conv(x, w, None, st)
    np.testing.assert_array_equal(y[: K - 1], st)
    np.testing.assert_array_equal(y[K - 1:], x[: L - (K - 1)])


@pytest.mark.parametrize("L", [0, 1, 2, 3, 8])
def test_conv_state_is_last_k_minus_1_inputs(L):
    C, K = 3, 4
    x = rng.standard_normal((L, C))
    st = rng.standard_normal((K - 1, C))
    _, new = causal_conv(x, rng.standard_normal((C, K)), None, st)
    z = np.concatenate([st, x])
    np.testing.assert_array_equal(new, z[-(K - 1):])
    if L == 1:  # one decode step: state shifts by one row
        np.testing.assert_array_equal(new[:2], st[1:])
        np.testing.assert_array_equal(new[2], x[0])
    if L == 2:  # shorter than K-1: keeps the newest old row
        np.testing.assert_array_equal(new[0], st[2])
        np.testing.assert_array_equal(new[1:], x)


def test_conv_silu_is_y_times_logistic():
    C, K, L = 4, 4, 6
    x = rng.standard_normal((L, C))
    w = rng.standard_normal((C, K))
    y_lin, _ = causal_conv(x, w)
    y_act, _ = causal_conv(x, w, activation="silu")
    np.testing.assert_allclose(y_act, y_lin * expit(y_lin), rtol=1e-14, atol=1e-15)


def test_l2norm_closed_form():
    x = rng.standard_normal((10, 3, 32)) * 3.0
    for eps in (0.0, 1e-6, 0.5):
        xn = l2norm(x, eps)
        n = np.linalg.norm(x, axis=-1)
        np.testing.assert_allclose(np.linalg.norm(xn, axis=-1), n / np.sqrt(n * n + eps), rtol=1e-14)
        # direction preserved: xn is a positive multiple of x
        ratio = xn / x
        np.testing.assert_allclose(ratio, ratio[..., :1] * np.ones_like(ratio), rtol=1e-13)
        assert np.all(ratio > 0)


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    ref = [1.0, -1.0, 3.140625, 0.0, -0.0, 3.3895313892515355e38, 9.183549615799121e-41]
    np.testing.assert_array_equal(bf16_bits_to_f64(bits), np.array(ref))


def test_packed_sequences_do_not_see_each_other():
    """Packing is per-sequence: shift kernel e_0 replays each sequence's own conv state."""
    Hk, Hv, d, K = 1, 1, 4, 4
    C = 2 * Hk * d + Hv * d
    lens = [1, 2, 5]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((T, C))
    cs = rng.standard_normal((3, K - 1, C))
    w = np.zeros((C, K))
    w[:, 0] = 1.0
    out = prefill_layer(x, w, cu, cs, np.zeros((3, Hv, d, d)), np.zeros((T, Hv)), np.zeros((T, Hv)),
                        Hk, Hv, d)
    for s, L in enumerate(lens):
        z = np.concatenate([cs[s], x[cu[s]:cu[s + 1]]])
        np.testing.assert_array_equal(out["y"][cu[s]:cu[s + 1]], z[:L])
        np.testing.assert_array_equal(out["conv_state"][s], z[-(K - 1):])


def test_conv_bias_is_added_before_silu():
    """With identity taps (w = e_{K-1}) and a bias b the conv output is silu(x + b): the
    bias sits inside the activation (y = act(b + sum_j w_j z_j)). The reverse order,
    silu(x) + b, differs for every nonzero b, so it fails this pin."""
    C, K, L = 6, 4, 9
    x = rng.standard_normal((L, C))
    st = rng.standard_normal((K - 1, C))
    b = rng.uniform(-1.0, 1.0, C)
    w = np.zeros((C, K))
    w[:, K - 1] = 1.0
    y, _ = causal_conv(x, w, b, st, activation="silu")
    pre = x + b[None, :]
    np.testing.assert_allclose(y, pre * expit(pre), rtol=1e-14, atol=1e-15)
    swapped = x * expit(x) + b[None, :]
    assert np.abs(y - swapped).min() > 1e-6
