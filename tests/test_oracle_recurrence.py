"""Pins for the oracle's gated delta rule.

The rule: S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t.
("System Design", "GDN Kernel Dispatch Detail": decode decays the temporal state,
writes the delta, then multiplies the query by the state.)

Every test here fixes the result by something other than the oracle's own formula:
a closed form, a library routine, an invariant of the rule, exact rational
arithmetic worked by hand, or an independent (Kronecker) formulation.
"""

import numpy as np
import pytest
from scipy.signal import lfilter

from oracle import gated_delta_recurrent, l2norm

rng = np.random.default_rng(11)


def _unit(n, d):
    return l2norm(rng.standard_normal((n, d)), 0.0)


def _rand_problem(L, Hk, Hv, d, s0=0.3):
    q = _unit(L * Hk, d).reshape(L, Hk, d)
    k = _unit(L * Hk, d).reshape(L, Hk, d)
    v = rng.standard_normal((L, Hv, d))
    g = -np.logaddexp(0, rng.standard_normal((L, Hv)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((L, Hv))))
    S0 = rng.standard_normal((Hv, d, d)) * s0
    return q, k, v, g, beta, S0


def test_pure_decay_when_beta_zero():
    L, H, d = 9, 3, 5
    q, k, v, g, beta, S0 = _rand_problem(L, H, H, d)
    o, S = gated_delta_recurrent(q, k, v, g, np.zeros_like(beta), S0)
    cum = np.cumsum(g, axis=0)  # [L, H]
    np.testing.assert_allclose(S, np.exp(cum[-1])[:, None, None] * S0, rtol=1e-13, atol=1e-15)
    for t in range(L):
        ref = np.exp(cum[t])[:, None] * np.einsum("jvk,jk->jv", S0, q[t])
        np.testing.assert_allclose(o[t], ref, rtol=1e-12, atol=1e-15)


def test_delta_write_stores_v_under_unit_key():
    """g = 0, beta = 1, |k| = 1: after the write, S_t k_t = v_t whatever S_{t-1} was."""
    L, H, d = 6, 2, 7
    q, k, v, _, _, S0 = _rand_problem(L, H, H, d, s0=1.0)
    for t in range(1, L + 1):
        _, S = gated_delta_recurrent(q[:t], k[:t], v[:t], np.zeros((t, H)), np.ones((t, H)), S0)
        np.testing.assert_allclose(np.einsum("jvk,jk->jv", S, k[t - 1]), v[t - 1], rtol=1e-12, atol=1e-12)


def test_same_key_twice_overwrites():
    H, d = 1, 4
    kk = _unit(1, d)[0]
    k = np.stack([kk, kk])[:, None, :]
    v = rng.standard_normal((2, H, d))
    _, S = gated_delta_recurrent(k, k, v, np.zeros((2, H)), np.ones((2, H)), np.zeros((H, d, d)))
    np.testing.assert_allclose(S[0] @ kk, v[1, 0], rtol=1e-13, atol=1e-14)


def test_orthonormal_keys_form_an_associative_memory():
    """Writing all d orthonormal keys with g = 0, beta = 1 replaces the whole state:
    S e_i = v_i for every i, independent of S0."""
    d, H = 6, 1
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Q.T[:, None, :]  # d tokens, rows orthonormal
    v = rng.standard_normal((d, H, d))
    _, S = gated_delta_recurrent(keys, keys, v, np.zeros((d, H)), np.ones((d, H)),
                                 rng.standard_normal((H, d, d)))
    np.testing.assert_allclose(S[0] @ Q, v[:, 0, :].T, rtol=1e-12, atol=1e-12)


def test_scalar_case_is_a_first_order_filter():
    """d_k = d_v = 1 and k = +-1: S_t = alpha (1 - beta) S_{t-1} + beta v_t k_t, an LTI
    first-order filter for constant alpha, beta (scipy.signal.lfilter)."""
    L = 40
    alpha, b = 0.83, 0.37
    ks = np.sign(rng.standard_normal(L))
    ks[ks == 0] = 1
    v = rng.standard_normal(L)
    k = ks[:, None, None]
    o, S = gated_delta_recurrent(k, k, v[:, None, None], np.full((L, 1), np.log(alpha)),
                                 np.full((L, 1), b), np.zeros((1, 1, 1)))
    ref = lfilter([b], [1.0, -alpha * (1 - b)], v * ks)
    np.testing.assert_allclose(o[:, 0, 0], ref * ks, rtol=1e-12, atol=1e-14)  # o = S q with q = k
    np.testing.assert_allclose(S[0, 0, 0], ref[-1], rtol=1e-12)


def test_linear_in_initial_state_and_values():
    L, Hk, Hv, d = 7, 2, 4, 5
    q, k, v1, g, beta, S1 = _rand_problem(L, Hk, Hv, d)
    v2 = rng.standard_normal(v1.shape)
    S2 = rng.standard_normal(S1.shape)
    a, b = 1.7, -0.6
    o1, F1 = gated_delta_recurrent(q, k, v1, g, beta, S1)
    o2, F2 = gated_delta_recurrent(q, k, v2, g, beta, S2)
    o3, F3 = gated_delta_recurrent(q, k, a * v1 + b * v2, g, beta, a * S1 + b * S2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(F3, a * F1 + b * F2, rtol=1e-11, atol=1e-12)


def test_frobenius_bound_each_step():
    """|S_t|_F <= alpha_t |S_{t-1}|_F + beta_t |v_t| because |I - beta k k^T|_2 <= 1."""
    L, H, d = 20, 2, 6
    q, k, v, g, beta, S = _rand_problem(L, H, H, d, s0=2.0)
    for t in range(L):
        prev = np.linalg.norm(S, axis=(1, 2))
        _, S = gated_delta_recurrent(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], S)
        bound = np.exp(g[t]) * prev + beta[t] * np.linalg.norm(v[t], axis=-1)
        assert np.all(np.linalg.norm(S, axis=(1, 2)) <= bound * (1 + 1e-12))


@pytest.mark.parametrize("dk,dv,L", [(1, 1, 5), (2, 3, 6), (3, 2, 8), (4, 4, 8)])
def test_brute_force_kronecker_form(dk, dv, L):
    """Column-major vec: vec(S_t) = (alpha (I - beta k k^T) kron I_dv) vec(S_{t-1}) + beta (k kron v).
    The whole sequence is a product of materialised (dk*dv)^2 matrices."""
    Hk = Hv = 1
    q = _unit(L, dk)[:, None, :]
    k = _unit(L, dk)[:, None, :]
    v = rng.standard_normal((L, Hv, dv))
    g = -np.logaddexp(0, rng.standard_normal((L, 1)))
    beta = rng.uniform(0, 1, (L, 1))
    S0 = rng.standard_normal((1, dv, dk))
    o, S = gated_delta_recurrent(q, k, v, g, beta, S0)
    vec = S0[0].flatten(order="F")
    for t in range(L):
        kt, vt = k[t, 0], v[t, 0]
        M = np.exp(g[t, 0]) * np.kron(np.eye(dk) - beta[t, 0] * np.outer(kt, kt), np.eye(dv))
        vec = M @ vec + beta[t, 0] * np.kron(kt, vt)
        St = vec.reshape((dv, dk), order="F")
        np.testing.assert_allclose(o[t, 0], St @ q[t, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S[0], vec.reshape((dv, dk), order="F"), rtol=1e-12, atol=1e-13)


def test_hand_worked_exact_example():
    """d = 2, S0 = 0, q = (0, 1), worked by hand in exact arithmetic.

    Step 1: k = (1, 0), v = (1, 2), alpha = beta = 1:
        S = v k^T = [[1, 0], [2, 0]],   o = S q = (0, 0).
    Step 2: k = (3/5, 4/5), v = (0, 1), alpha = beta = 1/2:
        S k = (3/5, 6/5);  S - beta (S k) k^T = [[41/50, -6/25], [82/50, -12/25]];
        times alpha: [[41/100, -3/25], [41/50, -6/25]];  plus beta v k^T = [[0, 0], [3/10, 2/5]]
        S = [[41/100, -3/25], [28/25, 4/25]],   o = (-3/25, 4/25).
    """
    q = np.array([[[0.0, 1.0]], [[0.0, 1.0]]])
    k = np.array([[[1.0, 0.0]], [[0.6, 0.8]]])
    v = np.array([[[1.0, 2.0]], [[0.0, 1.0]]])
    g = np.log(np.array([[1.0], [0.5]]))
    beta = np.array([[1.0], [0.5]])
    o, S = gated_delta_recurrent(q, k, v, g, beta, np.zeros((1, 2, 2)))
    np.testing.assert_allclose(o[0, 0], [0.0, 0.0], atol=1e-16)
    np.testing.assert_allclose(o[1, 0], [-3 / 25, 4 / 25], rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(S[0], [[41 / 100, -3 / 25], [28 / 25, 4 / 25]], rtol=1e-15, atol=1e-16)


def test_output_reads_post_update_state_and_write_is_not_decayed():
    """One token from S0 = 0: S_1 = beta v k^T (the write carries no exp(g)), and
    o_1 = S_1 q = beta (k . q) v (the query reads the state after the write)."""
    d, H = 5, 2
    q = _unit(H, d)[None]
    k = _unit(H, d)[None]
    v = rng.standard_normal((1, H, d))
    g = np.array([[-0.7, -2.0]])
    beta = np.array([[0.3, 0.9]])
    o, S = gated_delta_recurrent(q, k, v, g, beta, np.zeros((H, d, d)))
    for j in range(H):
        np.testing.assert_allclose(S[j], beta[0, j] * np.outer(v[0, j], k[0, j]), rtol=1e-14)
        np.testing.assert_allclose(o[0, j], beta[0, j] * (k[0, j] @ q[0, j]) * v[0, j], rtol=1e-13)


def test_gqa_head_map_is_consecutive_grouping():
    """Hv = 4, Hk = 2: v-heads 0, 1 read k-head 0 and v-heads 2, 3 read k-head 1.
    With k-head 0 = e0 and k-head 1 = e1, one write from S0 = 0 (g = 0, beta = 1) gives
    S_j = v_j e_{j//2}^T."""
    d = 3
    k = np.zeros((1, 2, d))
    k[0, 0, 0] = 1.0
    k[0, 1, 1] = 1.0
    v = rng.standard_normal((1, 4, d))
    _, S = gated_delta_recurrent(k, k, v, np.zeros((1, 4)), np.ones((1, 4)), np.zeros((4, d, d)))
    for j in range(4):
        ref = np.zeros((d, d))
        ref[:, j // 2] = v[0, j]
        np.testing.assert_array_equal(S[j], ref)


# Unit keys with rational coordinates (Pythagorean triples and quadruples), so that
# k k^T, and with it every step of the rule, is exact in rational arithmetic.
_RATIONAL_UNIT_KEYS = {
    2: [(3, 4, 5), (5, 12, 13), (8, 15, 17), (1, 0, 1), (0, 1, 1), (-12, 5, 13)],
    3: [(1, 2, 2, 3), (2, 3, 6, 7), (2, -6, 9, 11), (0, 0, 1, 1), (4, 4, 7, 9)],
    4: [(1, 1, 1, 1, 2), (1, 2, 2, 4, 5), (2, 4, 5, 6, 9), (-1, 1, -1, 1, 2), (0, 3, 0, 4, 5)],
}


def _exact_kronecker_run(keys, vals, qs, alphas, betas, S0):
    """The whole sequence in exact rational arithmetic (fractions.Fraction), through the
    Kronecker form with column-major vec: vec(S_t) = (alpha (I - beta k k^T) kron I_dv)
    vec(S_{t-1}) + beta (k kron v), each (dk dv) x (dk dv) matrix materialised. Returns the
    outputs S_t q_t and the final state, as Fractions."""
    from fractions import Fraction as Fr

    dv, dk = len(S0), len(S0[0])
    n = dk * dv
    vec = [S0[r][c] for c in range(dk) for r in range(dv)]  # column-major
    outs = []
    for k, v, q, a, b in zip(keys, vals, qs, alphas, betas):
        proj = [[(Fr(1) if i == j else Fr(0)) - b * k[i] * k[j] for j in range(dk)] for i in range(dk)]
        # (A kron I_dv)[(i, r), (j, s)] = A[i][j] * [r == s], index (i, r) -> i * dv + r
        big = [[a * proj[i // dv][j // dv] * (1 if i % dv == j % dv else 0) for j in range(n)] for i in range(n)]
        kv = [b * k[i // dv] * v[i % dv] for i in range(n)]
        vec = [sum(big[i][j] * vec[j] for j in range(n)) + kv[i] for i in range(n)]
        S = [[vec[c * dv + r] for c in range(dk)] for r in range(dv)]
        outs.append([sum(S[r][c] * q[c] for c in range(dk)) for r in range(dv)])
    return outs, [[vec[c * dv + r] for c in range(dk)] for r in range(dv)]


@pytest.mark.parametrize("dk,dv,L", [(2, 2, 6), (2, 3, 8), (3, 2, 5), (4, 3, 5), (4, 4, 4)])
def test_brute_force_kronecker_form_exact_rational(dk, dv, L):
    """The oracle (float64) against the exact rational result of the Kronecker form:
    rational decays alpha = exp(g) and strengths beta, Pythagorean unit keys, rational v,
    q and S0. The only rounding on the oracle's side is float64 (and g = log alpha), so the
    two agree to a few ulp of the largest value."""
    from fractions import Fraction as Fr

    r = np.random.default_rng(100 + 10 * dk + dv)
    table = _RATIONAL_UNIT_KEYS[dk]
    keys = []
    for t in range(L):
        *num, den = table[int(r.integers(len(table)))]
        keys.append([Fr(c, den) for c in num])
    vals = [[Fr(int(r.integers(-9, 10)), int(r.integers(1, 5))) for _ in range(dv)] for _ in range(L)]
    qs = [[Fr(int(r.integers(-6, 7)), 4) for _ in range(dk)] for _ in range(L)]
    alphas = [Fr(int(r.integers(1, 9)), 8) for _ in range(L)]
    betas = [Fr(int(r.integers(0, 5)), 4) for _ in range(L)]  # includes beta = 0 and beta = 1
    S0 = [[Fr(int(r.integers(-5, 6)), 8) for _ in range(dk)] for _ in range(dv)]
    outs, S_exact = _exact_kronecker_run(keys, vals, qs, alphas, betas, S0)

    def f(a):
        return np.array([[float(x) for x in row] for row in a])

    q = f(qs)[:, None, :]
    k = f(keys)[:, None, :]
    v = f(vals)[:, None, :]
    g = np.log(np.array([float(a) for a in alphas]))[:, None]
    beta = np.array([float(b) for b in betas])[:, None]
    o, S = gated_delta_recurrent(q, k, v, g, beta, f(S0)[None])
    o_ref, S_ref = f(outs), f(S_exact)
    scale = max(np.abs(o_ref).max(), np.abs(S_ref).max(), 1.0)
    np.testing.assert_allclose(o[:, 0], o_ref, rtol=0, atol=1e-13 * scale)
    np.testing.assert_allclose(S[0], S_ref, rtol=0, atol=1e-13 * scale)
