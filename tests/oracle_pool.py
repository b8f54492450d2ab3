"""The fp64 oracle over every v-head of a full-size prefill, sharded over host processes.

Test infrastructure. A layer's k-heads are independent: k-head h, its q and k channels
and the Hv/Hk v-heads that read it form a layer of their own (one k-head, Hv/Hk v-heads)
whose conv and recurrence see nothing else. Each job hands the oracle one such group --
the input channels sliced out of x, the conv taps and the conv states, with the group's
g, beta and initial states -- and the results are put back in place. Slicing only selects
inputs; every value still comes from ``oracle.prefill_layer``.

Jobs run in fresh interpreter processes (multiprocessing "spawn": nothing of a GPU-using
parent is inherited), one single-threaded process per usable host core, at most 16.
"""

from __future__ import annotations

import os

import numpy as np


def _group_channels(h: int, Hk: int, Hv: int, d: int) -> np.ndarray:
    """Conv channels of k-head h's group in [q | k | v] order: q_h, k_h, then the v
    channels of v-heads h*G .. h*G + G - 1 (G = Hv / Hk)."""
    G = Hv // Hk
    q = np.arange(h * d, (h + 1) * d)
    k = Hk * d + q
    v = 2 * Hk * d + np.arange(h * G * d, (h + 1) * G * d)
    return np.concatenate([q, k, v])


def _job(args):
    from oracle import prefill_layer

    x, w, b, cu, cs, S0, g, beta, G, d, kw = args
    return prefill_layer(x, w, cu, cs, S0, g, beta, 1, G, d, conv_b=b, **kw)


def _init_worker():
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass


def usable_cpus() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def prefill_all_heads(inp: dict, procs: int | None = None, **kw) -> dict:
    """oracle.prefill_layer over every v-head of the packed batch ``inp`` (as made by
    gen.make_prefill), one job per k-head group. Returns o [T, Hv, d], S [N, Hv, d, d] and
    conv_state [N, K-1, C] (float64), as one prefill_layer call over the whole layer would;
    ``kw`` goes to prefill_layer (in_dtype defaults to the shape's)."""
    import multiprocessing as mp

    sh = inp["shape"]
    Hk, Hv, d = sh.num_k_heads, sh.num_v_heads, sh.head_dim
    G = Hv // Hk
    kw = dict(kw)
    kw.setdefault("in_dtype", sh.in_dtype)
    jobs, chans = [], []
    for h in range(Hk):
        ch = _group_channels(h, Hk, Hv, d)
        heads = np.arange(h * G, (h + 1) * G)
        b = None if inp.get("conv_b") is None else inp["conv_b"][ch]
        jobs.append((np.ascontiguousarray(inp["x"][:, ch]), np.ascontiguousarray(inp["conv_w"][ch]), b,
                     inp["cu_seqlens"], np.ascontiguousarray(inp["conv_state"][:, :, ch]),
                     np.ascontiguousarray(inp["S0"][:, heads]), np.ascontiguousarray(inp["g"][:, heads]),
                     np.ascontiguousarray(inp["beta"][:, heads]), G, d, kw))
        chans.append((ch, heads))
    T, C = inp["x"].shape
    # (about 0.2 ms of host time per token and v-head: a small batch runs inline, where
    # starting the worker processes would cost more than the work)
    n = procs or (1 if T * Hv < 10000 else usable_cpus())
    if n <= 1 or len(jobs) == 1:
        res = [_job(j) for j in jobs]
    else:
        with mp.get_context("spawn").Pool(min(n, len(jobs)), initializer=_init_worker) as pool:
            res = pool.map(_job, jobs)
    N = len(inp["cu_seqlens"]) - 1
    o = np.zeros((T, Hv, d))
    S = np.zeros((N, Hv, d, d))
    cs = np.zeros((N, sh.conv_width - 1, C))
    for (ch, heads), r in zip(chans, res):
        o[:, heads] = r["o"]
        S[:, heads] = r["S"]
        cs[:, :, ch] = r["conv_state"]
    return dict(o=o, S=S, conv_state=cs)
