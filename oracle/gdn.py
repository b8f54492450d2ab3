"""fp64 reference implementation of the Gated DeltaNet layer core (test infrastructure).

Sources for what is computed:
  * "System Design" (project_6 SYSTEM_DESIGN.md), sections "Runtime Data Flow" and
    "GDN Kernel Dispatch Detail": inside a GatedDeltaNet layer the projected q/k/v go
    through a depthwise causal Conv1d, then q and k are L2-normalised, then the
    gated delta rule runs; prefill uses a chunked kernel taking (q, k, v, g, beta,
    state) and updates the temporal state; decode updates the conv state, decays the
    temporal state and writes the delta, then multiplies the query by the state.
    Conv state and temporal state are separate per-sequence inputs.
  * "serve: Qwen3.5 on CUDA never batches concurrent requests" (aprender #5279),
    comments "Where concurrency is lost" and "Phase plan": the conv and delta-rule
    kernels take a sequence dimension with per-sequence conv and SSM state.
  * The gated delta rule itself:
        S_t = exp(g_t) * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
        o_t = S_t q_t,
    with S in R^{d_v x d_k}.

Readings where the pages are silent (each one is listed in the design notes):
  conv is PyTorch-style cross-correlation over [conv state (K-1 rows, oldest first) ||
  tokens], so w[c, K-1] multiplies the current token; activation is the identity unless
  SiLU is asked for; the L2 norm is x / sqrt(|x|^2 + eps); v-head j reads k-head
  j // (Hv / Hk); g and beta are one scalar per (token, v-head).

Everything is float64. Nothing here is blocked, fused or reordered beyond the
definition; the chunked form is a separate function whose only job is to be
compared with the recurrent one.
"""

from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------- inputs

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact decode of bfloat16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def storage_to_f64(a, dtype: str) -> np.ndarray:
    if a is None:
        return None
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------- steps

def causal_conv(x, w, b=None, state=None, activation: str = "none"):
    """Depthwise causal conv1d over one sequence.

    x [L, C] tokens, w [C, K] taps, b [C] or None, state [K-1, C] (oldest row first,
    None means zeros). With z = [state ; x] (K-1+L rows):
        y_t[c] = b[c] + sum_{j<K} w[c, j] * z_{t+j}[c],    t = 0 .. L-1
    then y <- act(y). The new conv state is the last K-1 rows of z.
    ("System Design", "Runtime Data Flow": depthwise causal Conv1d before the L2 norm.)
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    L, C = x.shape
    K = w.shape[1]
    if state is None:
        state = np.zeros((K - 1, C))
    z = np.concatenate([np.asarray(state, dtype=np.float64), x], axis=0)
    y = np.zeros((L, C))
    for j in range(K):
        y += w[:, j][None, :] * z[j:j + L]
    if b is not None:
        y += np.asarray(b, dtype=np.float64)[None, :]
    if activation == "silu":
        y = y / (1.0 + np.exp(-y))
    elif activation != "none":
        raise ValueError(activation)
    new_state = z[L:L + K - 1].copy()
    return y, new_state


def l2norm(x, eps: float):
    """x / sqrt(sum(x^2) + eps) over the last axis (one head vector)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def split_qkv(y, Hk: int, Hv: int, dk: int, dv: int):
    """Conv output channels are laid out [q (Hk*dk) | k (Hk*dk) | v (Hv*dv)]."""
    L = y.shape[0]
    q = y[:, : Hk * dk].reshape(L, Hk, dk)
    k = y[:, Hk * dk: 2 * Hk * dk].reshape(L, Hk, dk)
    v = y[:, 2 * Hk * dk: 2 * Hk * dk + Hv * dv].reshape(L, Hv, dv)
    return q, k, v


def _kmap(Hk: int, Hv: int) -> np.ndarray:
    """v-head j reads k-head j // (Hv / Hk) (consecutive grouping)."""
    return np.arange(Hv) // (Hv // Hk)


def gated_delta_recurrent(q, k, v, g, beta, S0, kmap=None):
    """The gated delta rule, one token at a time.

    q, k [L, Hk, dk] (already normalised / scaled), v [L, Hv, dv], g and beta [L, Hv],
    S0 [Hv, dv, dk]; kmap[j] is the k-head of v-head j. For every token t and v-head j:
        S <- exp(g) * S (I - beta k k^T) + beta v k^T ;  o_t = S q
    Returns o [L, Hv, dv] and the final S [Hv, dv, dk].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    S = np.array(S0, dtype=np.float64, copy=True)
    L, Hv, dv = v.shape
    if kmap is None:
        kmap = _kmap(q.shape[1], Hv)
    o = np.empty((L, Hv, dv))
    for t in range(L):
        kt = k[t][kmap]  # [Hv, dk]
        qt = q[t][kmap]
        alpha = np.exp(g[t])[:, None, None]
        b = beta[t][:, None, None]
        Sk = np.einsum("jvk,jk->jv", S, kt)
        # S (I - beta k k^T) = S - beta (S k) k^T
        S = alpha * (S - b * Sk[:, :, None] * kt[:, None, :]) + b * v[t][:, :, None] * kt[:, None, :]
        o[t] = np.einsum("jvk,jk->jv", S, qt)
    return o, S


def gated_delta_chunked(q, k, v, g, beta, S0, chunk: int, kmap=None):
    """Chunked (WY / UT-transform) form of the same recurrence, chunks aligned to the
    sequence start. Per chunk of n tokens with state S0 on entry (per v-head):
        gam = cumsum(g)                      (inclusive)
        A[t, s] = beta_t exp(gam_t - gam_s) (k_t . k_s)   for s < t, else 0
        T = (I + A)^-1
        W = T diag(beta exp(gam)) K,   U~ = T diag(beta) V
        U = U~ - W S0^T
        O = diag(exp(gam)) Q S0^T + (M o Q K^T) U,   M[t, s] = exp(gam_t - gam_s) for s <= t
        S = exp(gam_n) S0 + U^T diag(exp(gam_n - gam)) K
    Every decay factor is exp of a difference gam_t - gam_s with t >= s, so none overflows.
    This function is only compared with ``gated_delta_recurrent``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    L, Hv, dv = v.shape
    if kmap is None:
        kmap = _kmap(q.shape[1], Hv)
    S_all = np.array(S0, dtype=np.float64, copy=True)
    o = np.empty((L, Hv, dv))
    for j in range(Hv):
        h = kmap[j]
        S = S_all[j]
        for c0 in range(0, L, chunk):
            c1 = min(L, c0 + chunk)
            n = c1 - c0
            Q, Kc, V = q[c0:c1, h], k[c0:c1, h], v[c0:c1, j]
            bt = beta[c0:c1, j]
            gam = np.cumsum(g[c0:c1, j])
            diff = gam[:, None] - gam[None, :]
            lower_strict = np.tril(np.ones((n, n)), -1)
            lower = np.tril(np.ones((n, n)))
            decay = np.exp(np.where(lower > 0, diff, -np.inf))
            A = bt[:, None] * decay * (Kc @ Kc.T) * lower_strict
            T = np.linalg.inv(np.eye(n) + A)
            W = T @ ((bt * np.exp(gam))[:, None] * Kc)
            Ut = T @ (bt[:, None] * V)
            U = Ut - W @ S.T
            P = decay * (Q @ Kc.T)
            o[c0:c1, j] = np.exp(gam)[:, None] * (Q @ S.T) + P @ U
            S = np.exp(gam[-1]) * S + U.T @ (np.exp(gam[-1] - gam)[:, None] * Kc)
        S_all[j] = S
    return o, S_all


# ----------------------------------------------------------------------------- layer

def prefill_layer(x, conv_w, cu_seqlens, conv_state, S0, g, beta, Hk: int, Hv: int, d: int,
                  conv_b=None, in_dtype: str = "f32", activation: str = "none",
                  eps: float = 1e-6, scale: float = 1.0, v_heads=None, chunk: int | None = None,
                  qk_l2norm: bool = True):
    """The whole layer core over packed ragged sequences.

    x [T, C] (storage dtype), conv_w [C, K], conv_b [C] or None, cu_seqlens [N+1],
    conv_state [N, K-1, C] (storage dtype), S0 [N, Hv, d, d], g and beta [T, Hv].
    Per sequence: conv (from its own conv state) -> split -> L2 norm (q also scaled)
    -> gated delta rule from its own recurrent state. Sequences never see each other.
    ``v_heads`` restricts the recurrence to a subset of v-heads (o and S come back for
    those heads only); ``chunk`` switches the recurrence to the chunked form;
    ``qk_l2norm=False`` skips the L2 norm (q and k used as the conv gives them, q still
    times ``scale``).

    Returns dict y [T, C], o [T, H, d], S [N, H, d, d], conv_state [N, K-1, C].
    """
    xf = storage_to_f64(x, in_dtype)
    wf = storage_to_f64(conv_w, in_dtype)
    bf = storage_to_f64(conv_b, in_dtype)
    csf = storage_to_f64(conv_state, in_dtype)
    S0 = np.asarray(S0, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    T, C = xf.shape
    heads = np.arange(Hv) if v_heads is None else np.asarray(v_heads)
    kmap = _kmap(Hk, Hv)[heads]
    y = np.zeros((T, C))
    o = np.zeros((T, len(heads), d))
    S_out = np.zeros((N, len(heads), d, d))
    cs_out = np.zeros_like(csf)
    for s in range(N):
        a, b = int(cu[s]), int(cu[s + 1])
        ys, cs_out[s] = causal_conv(xf[a:b], wf, bf, csf[s], activation)
        y[a:b] = ys
        q, k, v = split_qkv(ys, Hk, Hv, d, d)
        qn = (l2norm(q, eps) if qk_l2norm else q) * scale
        kn = l2norm(k, eps) if qk_l2norm else k
        args = (qn, kn, v[:, heads], g[a:b][:, heads], beta[a:b][:, heads], S0[s][heads])
        if chunk is None:
            o[a:b], S_out[s] = gated_delta_recurrent(*args, kmap=kmap)
        else:
            o[a:b], S_out[s] = gated_delta_chunked(*args, chunk=chunk, kmap=kmap)
    return dict(y=y, o=o, S=S_out, conv_state=cs_out)


def decode_layer(x, conv_w, conv_state, S, g, beta, Hk: int, Hv: int, d: int, **kw):
    """One decode token per slot: slot i owns token i, its conv state and its
    recurrent state ("aprender #5279", "Phase plan": the GDN conv and delta rule
    gain a slot dimension and read per-slot state through a pointer array).
    This is the prefill path with every sequence of length 1.
    Shapes: x [m, C], conv_state [m, K-1, C], S [m, Hv, d, d], g and beta [m, Hv]."""
    m = np.asarray(x).shape[0]
    cu = np.arange(m + 1, dtype=np.int64)
    return prefill_layer(x, conv_w, cu, conv_state, S, g, beta, Hk, Hv, d, **kw)
