#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet layer core on one MI355X.

One step = one pass of the whole hot path:
  * decode: a 30-layer decode step at m slots (default 64) of a 256-slot pool, over 32
    v-heads x 128x128 fp32 states addressed through per-layer device u64 pointer arrays.
    Three forms of a layer are timed, each captured in a HIP graph and replayed (the
    serving-loop form), and eagerly (one ctypes call per launch):
      - fused_stream (the headline): one gdn_decode_fused call per layer (conv, conv-state
        commit, q/k L2 norm, delta rule), the conv states read from one pool and written to
        a second, the two pools alternating from step to step (one replay = two steps);
      - fused: the same call with the conv states updated in place;
      - two_calls: gdn_conv_update (decode mode) + gdn_decode_batched;
  * prefill: one 4096-token sequence (16 q/k heads, 32 v-heads, d = 128, bf16 input,
    chunk 64) = gdn_conv_update (prefill mode) + gdn_prefill_chunked, and the same as one
    gdn_prefill_fused call. The 8-sequence ragged pack (T = 15717) and one GPU's share
    of an 8-way head split (2 q/k, 4 v heads) are timed as well.
Inputs are seeded synthetic data already resident in HBM when timing starts.

`value` is the decode state bandwidth: 30 * m * 4 MiB (each slot-layer reads and writes
its 2 MiB state once) over the graph-replayed fused_stream step. Prefill is reported as
tokens/s (eager calls, and the same calls replayed from a HIP graph) and as algorithmic
TFLOP/s against the bf16 MFMA peak. `roofline` is for the dominant kernel (the fused
decode kernel of the headline step), whose average launch time is measured with HIP
events around back-to-back launches on the stream it runs on. `ceilings` are this GPU's
measured practical rates: the library's in-place streaming pass (gdn_hbm_probe) over
4 GiB, in one launch and as 32 launches of 128 MiB (the decode step's shape; the better
of the two is the practical HBM ceiling), a torch device copy of 4 GiB and a bf16
8192^3 matmul. `cpu_baseline` times the
fp64 oracle on a bounded sample of the same decode workload on one host thread
(`cpu_baseline_all_cores`: one single-threaded process per usable core, at most 16).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
STATE_BYTES_PER_SLOT_LAYER = 2 * 32 * 128 * 128 * 4  # read + write of one 2 MiB state
# Everything one slot-layer of the fused decode must move: the state (read + write), the
# conv state (3 rows x 8192 channels bf16, read + write), x (8192 bf16), o (32 x 128 fp32)
# and g, beta (32 fp32 each); plus the conv taps (8192 x 4 bf16) once per launch.
FUSED_BYTES_PER_SLOT_LAYER = STATE_BYTES_PER_SLOT_LAYER + 2 * 3 * 8192 * 2 + 8192 * 2 + 32 * 128 * 4 + 2 * 32 * 4
CONV_TAP_BYTES = 8192 * 4 * 2


def source_key(path: str) -> str:
    """sha256 of a source file with its comments and whitespace removed: the key under
    which counter figures are filed, unchanged by an edit to comments or layout."""
    import hashlib
    import re

    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()


def measured_traffic():
    """HBM bytes per launch of the headline step's fused decode kernel (m = 64) from the
    committed counter summary, or None when csrc/decode.hip's code has changed since those
    counters were taken (its comment-free key differs from the one recorded there)."""
    prof = os.path.join(ROOT, "profiles", "hbm_counters_decode_kernels_m64.md")
    src = os.path.join(ROOT, "gated_delta_rule_conv_amd", "csrc", "decode.hip")
    try:
        fields = {}
        with open(prof) as f:
            for line in f:
                if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_launch", "decode_source_key"):
                    k, v = line.split(":", 1)
                    fields[k] = v.strip()
        if fields.get("decode_source_key") != source_key(src):
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def ev():
    import torch

    return torch.cuda.Event(enable_timing=True)


SETTLE_S = 0.1


def set_settle(seconds: float) -> None:
    global SETTLE_S
    SETTLE_S = seconds


def settle(call, seconds: float | None = None) -> None:
    """Untimed calls, back to back, for at least `seconds` before a timed section: after the
    host has been setting up (inputs, graph capture) the GPU sits at its idle clocks and
    takes tens of milliseconds of work to leave them (measured: the fused L = 4096 prefill
    takes about 205 us a call over its first 20 calls after such a gap and 177-183 us once
    the GPU has been busy for ~25 ms), and a timed section should see the clocks a busy
    server runs at. The timed calls that follow are unchanged."""
    import torch

    if seconds is None:
        seconds = SETTLE_S
    if seconds <= 0:
        return
    t0 = time.perf_counter()
    n = 0
    while True:
        call()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return


FORMS = ("fused_stream", "fused", "two_calls")


class DecodeRig:
    """30 layers of slot pools (256 slots each) and m active slots per layer, stepped in
    one of the FORMS."""

    def __init__(self, m: int, form: str, layers: int = 30, pool: int = 256, n_inputs: int = 8, device="cuda"):
        import numpy as np
        import torch

        import gated_delta_rule_conv_amd as gdn
        from gen.inputs import DECODE_30_LAYERS, ST_PERM, WORKLOADS, make_decode_pool_torch, rng_for

        assert form in FORMS
        sh = WORKLOADS[DECODE_30_LAYERS].shape
        self.m, self.layers, self.sh, self.form = m, layers, sh, form
        self.dims = gdn.make_dims(sh.num_k_heads, sh.num_v_heads, sh.head_dim, conv_width=sh.conv_width,
                                  chunk_size=sh.chunk, in_dtype=gdn.GDN_BF16)
        self.states, self.conv_states, self.conv_w = make_decode_pool_torch(DECODE_30_LAYERS, pool, layers, device)
        slots = rng_for(DECODE_30_LAYERS, ST_PERM).permutation(pool)[:m].astype(np.int32)
        idx = torch.tensor(slots, dtype=torch.int32, device=device)
        self.sptr = torch.empty((layers, m), dtype=torch.int64, device=device)
        self.cptr = torch.empty((layers, m), dtype=torch.int64, device=device)
        s_bytes = self.states[0, 0].numel() * 4
        c_bytes = self.conv_states[0, 0].numel() * self.conv_states.element_size()
        for layer in range(layers):
            gdn.gdn_slot_pointers(self.states[layer].data_ptr(), s_bytes, pool, idx, m, self.sptr[layer])
            gdn.gdn_slot_pointers(self.conv_states[layer].data_ptr(), c_bytes, pool, idx, m, self.cptr[layer])
        if form == "fused_stream":
            # the second conv pool: step n reads pool n % 2 and writes the other
            self.conv_states2 = self.conv_states.clone()
            self.cptr2 = torch.empty((layers, m), dtype=torch.int64, device=device)
            for layer in range(layers):
                gdn.gdn_slot_pointers(self.conv_states2[layer].data_ptr(), c_bytes, pool, idx, m, self.cptr2[layer])
        self.direction = 0
        gen = torch.Generator(device=device)
        gen.manual_seed(3100 + m)
        C, Hv = sh.channels, sh.num_v_heads
        self.n_inputs = n_inputs
        self.x = torch.randn((n_inputs, m, C), generator=gen, device=device).to(torch.bfloat16)
        self.g = -torch.nn.functional.softplus(torch.randn((n_inputs, m, Hv), generator=gen, device=device))
        self.beta = torch.sigmoid(torch.randn((n_inputs, m, Hv), generator=gen, device=device))
        self.y = torch.empty((m, C), dtype=torch.float32, device=device)
        self.o = torch.empty((m, Hv, sh.head_dim), dtype=torch.float32, device=device)
        self.q, self.k, self.v = gdn.qkv_views(self.dims, self.y)
        self.graph = None
        self.steps_per_replay = 2 if form == "fused_stream" else 1

    def kernel(self, layer: int, s: int) -> None:
        """The launch whose time is the roofline's: the fused kernel, or the decode kernel
        of the two-call form."""
        import gated_delta_rule_conv_amd as gdn

        if self.form == "two_calls":
            q, k, v = self.q, self.k, self.v
            gdn.gdn_decode_batched(self.dims, q, q.stride(0), k, k.stride(0), v, v.stride(0), self.g[s],
                                   self.beta[s], self.o, self.sptr[layer], self.m)
            return
        cin, cout = self.cptr[layer], None
        if self.form == "fused_stream":
            cin, cout = (self.cptr[layer], self.cptr2[layer]) if self.direction == 0 else \
                (self.cptr2[layer], self.cptr[layer])
        gdn.decode_fused(self.dims, self.x[s], self.conv_w[layer], None, self.g[s], self.beta[s], self.o,
                         self.sptr[layer], cin, cout)

    def layer(self, layer: int, s: int) -> None:
        import gated_delta_rule_conv_amd as gdn

        if self.form == "two_calls":
            gdn.conv_update(self.dims, self.x[s], self.y, self.conv_w[layer], None, self.cptr[layer])
        self.kernel(layer, s)

    def step(self) -> None:
        for layer in range(self.layers):
            self.layer(layer, layer % self.n_inputs)
        self.direction ^= 1

    def capture(self) -> None:
        """Capture steps_per_replay whole steps (30 layers each) in one HIP graph."""
        import torch

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(self.steps_per_replay):
                self.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for _ in range(self.steps_per_replay):
                self.step()
        torch.cuda.synchronize()

    def replay(self) -> None:
        self.graph.replay()


class PrefillRig:
    def __init__(self, wid: int, device="cuda", shape=None, form: int = 0, fused: bool = False):
        import numpy as np
        import torch

        import gated_delta_rule_conv_amd as gdn
        from gen import make_prefill

        inp = make_prefill(wid, shape=shape)
        sh = inp["shape"]
        self.sh = sh
        self.lens = list(inp["lens"])
        self.dims = gdn.make_dims(sh.num_k_heads, sh.num_v_heads, sh.head_dim, conv_width=sh.conv_width,
                                  chunk_size=sh.chunk, in_dtype=gdn.GDN_BF16, prefill_form=form)
        T = inp["x"].shape[0]
        N = len(inp["lens"])
        self.T, self.N = T, N

        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

        self.x = bf(inp["x"])
        self.conv_w = bf(inp["conv_w"])
        self.pool = gdn.SlotPool(self.dims, N, device=device, state=torch.from_numpy(inp["S0"]).to(device),
                                 conv_state=bf(inp["conv_state"]))
        self.sptr, self.cptr = self.pool.pointers(torch.arange(N, dtype=torch.int32, device=device))
        self.cu = torch.tensor(inp["cu_seqlens"], dtype=torch.int32, device=device)
        self.g = torch.from_numpy(inp["g"]).to(device)
        self.beta = torch.from_numpy(inp["beta"]).to(device)
        self.o = torch.empty((T, sh.num_v_heads, sh.head_dim), dtype=torch.float32, device=device)
        self.fused = fused
        if fused:
            self.y = None
            self.ws = gdn.prefill_fused_workspace(self.dims, N, T, device=device)
        else:
            self.y = torch.empty((T, sh.channels), dtype=torch.float32, device=device)
            self.ws = gdn.prefill_workspace(self.dims, N, T, device=device)

    def flops(self) -> float:
        """Algorithmic flops of the chunked form per v-head, summed over chunks of n
        tokens: K K^T, Q K^T, W, U~, U = U~ - W S0^T, Q S0^T, P U, U^T K at 2 n^2 d or
        2 n d^2 each, plus the triangular inverse at (2/3) n^3."""
        d, C, Hv = self.sh.head_dim, self.sh.chunk, self.sh.num_v_heads
        tot = 0.0
        for L in self.lens:
            for c0 in range(0, L, C):
                n = min(C, L - c0)
                tot += 5 * 2 * n * n * d + 3 * 2 * n * d * d + (2.0 / 3.0) * n ** 3
        return tot * Hv

    def capture(self):
        """One prefill call (or the two calls) captured in a HIP graph."""
        import torch

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step()
        torch.cuda.synchronize()
        return graph

    def step(self) -> None:
        import gated_delta_rule_conv_amd as gdn

        if self.fused:
            gdn.prefill_fused(self.dims, self.x, self.conv_w, None, self.g, self.beta, self.o, self.cu, self.sptr,
                              self.cptr, self.ws)
        else:
            gdn.conv_update(self.dims, self.x, self.y, self.conv_w, None, self.cptr, self.cu)
            gdn.prefill(self.dims, self.y, self.g, self.beta, self.o, self.cu, self.sptr, self.ws)


def cpu_baseline(seconds: float) -> dict:
    """The fp64 oracle's decode layer, single-threaded, on host cores: slot-layers of the
    30-layer decode workload (32 v-heads x 128x128 state each), until `seconds` pass."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    from gen import DECODE_30_LAYERS, make_decode_pool, make_decode_step
    from oracle import decode_layer

    pool = make_decode_pool(DECODE_30_LAYERS, pool=4)
    sh = pool["shape"]
    done = 0
    t0 = time.perf_counter()
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        step = 0
        while time.perf_counter() - t0 < seconds:
            inp = make_decode_step(DECODE_30_LAYERS, step, 4)
            decode_layer(inp["x"], pool["conv_w"], pool["conv_state"], pool["S"], inp["g"], inp["beta"],
                         sh.num_k_heads, sh.num_v_heads, sh.head_dim, in_dtype="bf16")
            done += 4
            step += 1
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    dt = time.perf_counter() - t0
    return {"value": round(done * STATE_BYTES_PER_SLOT_LAYER / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{done} slot-layers of the 30-layer m=64 decode workload (conv + L2 norm + one delta-rule "
                      f"step, 32 v-heads x 128x128 state, bf16 input), 4 slots per call, {dt:.1f} s of float64 "
                      f"NumPy on 1 thread; host has {os.cpu_count()} logical CPUs"}


def _oracle_worker(args):
    """One host process: the oracle's decode layer on its own slot-layers for `seconds`."""
    seconds, seed = args
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        ctx = None
    from gen import DECODE_30_LAYERS, make_decode_pool, make_decode_step
    from oracle import decode_layer

    pool = make_decode_pool(DECODE_30_LAYERS, pool=4)
    sh = pool["shape"]
    done, step = 0, seed * 1000
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        inp = make_decode_step(DECODE_30_LAYERS, step, 4)
        decode_layer(inp["x"], pool["conv_w"], pool["conv_state"], pool["S"], inp["g"], inp["beta"],
                     sh.num_k_heads, sh.num_v_heads, sh.head_dim, in_dtype="bf16")
        done += 4
        step += 1
    return done, time.perf_counter() - t0


def host_cpu() -> dict:
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    return {"model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline_pool(seconds: float) -> dict:
    """The same oracle sharded over every usable host core: one process per core, each on
    its own slot-layers (independent units), single-threaded, for `seconds`."""
    import multiprocessing as mp

    n = min(host_cpu()["usable_cpus"], 16)  # (at most 16: the GPU machine's CPU share)
    ctx = mp.get_context("spawn")  # (a fresh interpreter: nothing of this process's GPU state)
    with ctx.Pool(n) as pool:
        res = pool.map(_oracle_worker, [(seconds, i) for i in range(n)])
    done = sum(r[0] for r in res)
    dt = max(r[1] for r in res)
    return {"value": round(done * STATE_BYTES_PER_SLOT_LAYER / dt / 1e9, 4), "unit": "GB/s", "cores": n,
            "kind": "oracle", "sample": f"{done} slot-layers over {n} single-threaded processes, {dt:.1f} s"}


def ceilings() -> dict:
    """Measured practical ceilings of this GPU, medians of 5: the library's in-place
    streaming pass (gdn_hbm_probe: the decode kernel's state access pattern without its
    arithmetic) over 4 GiB, a torch device-to-device copy of 4 GiB (read + write bytes over
    time) and a bf16 8192 x 8192 x 8192 matmul."""
    import statistics

    import torch

    import gated_delta_rule_conv_amd as gdn

    out = {}
    buf = torch.empty(1 << 30, dtype=torch.float32, device="cuda").fill_(1.0)  # 4 GiB
    nbytes = buf.numel() * 4
    gdn.gdn_hbm_probe(buf, nbytes)
    ts = []
    for _ in range(5):
        a, b = ev(), ev()
        a.record()
        gdn.gdn_hbm_probe(buf, nbytes)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    out["inplace_stream_4GiB_GBps"] = round(2 * nbytes / (statistics.median(ts) * 1e-3) / 1e9, 1)
    # the same 4 GiB as 32 back-to-back launches of 128 MiB each: the decode step's shape
    # (30 launches, each streaming 64 slots x 2 MiB = 128 MiB in place) without its
    # arithmetic, over a footprint the 256 MB Infinity Cache cannot hold
    chunk = 128 << 20
    base = buf.data_ptr()
    ts = []
    for _ in range(5):
        a, b = ev(), ev()
        a.record()
        for c in range(nbytes // chunk):
            gdn.gdn_hbm_probe(base + c * chunk, chunk, 0, torch.cuda.current_stream().cuda_stream)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    out["inplace_stream_32x128MiB_GBps"] = round(2 * nbytes / (statistics.median(ts) * 1e-3) / 1e9, 1)
    # the practical HBM ceiling: the better of the two streaming rates
    out["practical_hbm_GBps"] = max(out["inplace_stream_4GiB_GBps"], out["inplace_stream_32x128MiB_GBps"])
    dst = torch.empty_like(buf)
    dst.copy_(buf)
    ts = []
    for _ in range(5):
        a, b = ev(), ev()
        a.record()
        dst.copy_(buf)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    out["d2d_copy_4GiB_GBps"] = round(2 * nbytes / (statistics.median(ts) * 1e-3) / 1e9, 1)
    del buf, dst
    torch.cuda.empty_cache()
    n = 8192
    x = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    y = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    z = torch.matmul(x, y)
    ts = []
    for _ in range(5):
        a, b = ev(), ev()
        a.record()
        z = torch.matmul(x, y)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    out["bf16_matmul_8192_TFLOPs"] = round(2 * n ** 3 / (statistics.median(ts) * 1e-3) / 1e12, 1)
    del x, y, z
    torch.cuda.empty_cache()
    return out


def time_graph_scrubbed(rig: DecodeRig, steps: int, scrub) -> float:
    """Median ms per decode step of single graph replays, each after a 1 GiB write that
    evicts the states from the GPU's caches (the write is outside the timed region)."""
    import statistics

    import torch

    ts = []
    for _ in range(steps):
        scrub.fill_(0.0)
        a, b = ev(), ev()
        a.record()
        rig.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / rig.steps_per_replay)
    return statistics.median(ts)


def time_graph(rig: DecodeRig, steps: int, warmup: int) -> float:
    """Mean ms per decode step over `steps` graph replays (a replay holds
    rig.steps_per_replay steps)."""
    import torch

    for _ in range(warmup):
        rig.replay()
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record()
    for _ in range(steps):
        rig.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (steps * rig.steps_per_replay)


def time_decode_kernel(rig: DecodeRig, rounds: int) -> float:
    """Mean us per launch of the rig's roofline kernel (rig.kernel: the fused kernel, or
    the decode kernel of the two-call form): the 30 layers' launches back to back (no conv
    launches in between), `rounds` times, events on the launching stream."""
    import torch

    a, b = ev(), ev()
    torch.cuda.synchronize()
    a.record()
    for _ in range(rounds):
        for layer in range(rig.layers):
            rig.kernel(layer, layer % rig.n_inputs)
        rig.direction ^= 1
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (rounds * rig.layers)


def copy_probe(mib: int = 256, reps: int = 4) -> None:
    """Kernels of known traffic, for scaling hardware byte counters: torch's device copy
    (reads mib MiB, writes mib MiB) and the library's in-place streaming pass
    (gdn_hbm_probe: reads and writes the same mib MiB), reps launches each."""
    import torch

    import gated_delta_rule_conv_amd as gdn

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    for i in range(reps):
        gdn.gdn_hbm_probe(src, src.numel() * 4, i + 1)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} device copies and {reps} in-place streaming passes of {mib} MiB")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed calls before each timed section (0: none, e.g. for a profiler, "
                         "whose traces then hold a fixed number of launches per section)")
    ap.add_argument("--m", type=int, default=64)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-ragged", action="store_true", help="skip the 8-sequence ragged prefill")
    ap.add_argument("--no-sweep", action="store_true", help="skip the m = 1, 4, 16 decode steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true", help="also run a 256 MiB device copy (counter scale)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured copy / matmul ceilings")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the GDN layer core here has no multi-GPU path (no collectives, "
              "no sharding code); run it with --gpus 1", file=sys.stderr)
        return 2

    # the oracle over every host core first, in processes started before this one touches
    # the GPU
    cpu_pool = None
    if not args.no_cpu_baseline:
        log("timing the oracle on all host cores")
        cpu_pool = cpu_baseline_pool(args.cpu_seconds / 2)

    import torch

    torch.cuda.set_device(0)
    log(f"device {torch.cuda.get_device_name(0)}")
    if args.copy_probe:
        copy_probe()
    K, W = args.steps, args.warmup
    set_settle(args.settle)

    # ---------------------------------------------------------------- decode, m = 64
    def run_decode(form: str):
        rig = DecodeRig(args.m, form)
        settle(rig.step)
        for _ in range(W):
            rig.step()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(K):
            rig.step()
        b.record()
        torch.cuda.synchronize()
        eager_ms = a.elapsed_time(b) / K
        rig.capture()
        settle(rig.replay)
        t_start = time.perf_counter()
        graph_ms = time_graph(rig, K, W)
        wall = time.perf_counter() - t_start
        kern_us = time_decode_kernel(rig, max(2, K // 4))
        log(f"decode {form}: eager {eager_ms:.3f} ms/step, graph {graph_ms:.3f} ms/step, kernel {kern_us:.2f} us")
        del rig
        torch.cuda.empty_cache()
        return {"eager_ms": eager_ms, "graph_ms": graph_ms, "wall": wall, "kernel_us": kern_us}

    runs = {form: run_decode(form) for form in FORMS}
    state_bytes_step = 30 * args.m * STATE_BYTES_PER_SLOT_LAYER
    head = runs["fused_stream"]
    graph_ms = head["graph_ms"]
    value = state_bytes_step / (graph_ms * 1e-3) / 1e9
    # algorithmic bytes of one fused launch: the state, the conv state (read from one pool,
    # written to another), x, o, g and beta of every slot-layer, and the taps once
    bytes_per_launch = args.m * FUSED_BYTES_PER_SLOT_LAYER + CONV_TAP_BYTES
    kern_us = head["kernel_us"]
    achieved = bytes_per_launch / (kern_us * 1e-6) / 1e9
    plain_bytes = args.m * STATE_BYTES_PER_SLOT_LAYER

    def form_row(form, note):
        r = runs[form]
        row = {"note": note, "graph_ms_per_step": round(r["graph_ms"], 4), "eager_ms_per_step": round(r["eager_ms"], 4),
               "state_GBps_graph": round(state_bytes_step / (r["graph_ms"] * 1e-3) / 1e9, 2),
               "state_GBps_eager": round(state_bytes_step / (r["eager_ms"] * 1e-3) / 1e9, 2),
               "frac_of_hbm_peak": round(state_bytes_step / (r["graph_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if form == "two_calls":
            row["decode_kernel_us"] = round(r["kernel_us"], 2)
            row["decode_kernel_GBps"] = round(plain_bytes / (r["kernel_us"] * 1e-6) / 1e9, 2)
        else:
            row["fused_kernel_us"] = round(r["kernel_us"], 2)
            row["fused_kernel_GBps"] = round(bytes_per_launch / (r["kernel_us"] * 1e-6) / 1e9, 2)
        return row

    decode_forms = {
        "fused_stream": form_row("fused_stream", "one gdn_decode_fused call per layer, conv states read from one "
                                                 "pool and written to another (alternating every step)"),
        "fused": form_row("fused", "one gdn_decode_fused call per layer, conv states updated in place"),
        "two_calls": form_row("two_calls", "gdn_conv_update (decode mode) + gdn_decode_batched per layer"),
    }

    sweep = None
    if not args.no_sweep:
        sweep = {}
        scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        for mm in (1, 4, 16):
            row = {}
            for form in FORMS:
                r = DecodeRig(mm, form)
                for _ in range(2):
                    r.step()
                r.capture()
                settle(r.replay)
                ms = time_graph(r, K, W)
                row[form + "_ms_per_step"] = round(ms, 4)
                row[form + "_state_GBps"] = round(r.layers * mm * STATE_BYTES_PER_SLOT_LAYER / ms / 1e6, 1)
                if mm * 60 < 256:  # state footprint fits the Infinity Cache: also from cold caches
                    sms = time_graph_scrubbed(r, max(5, K // 2), scrub)
                    row[form + "_scrubbed_ms_per_step"] = round(sms, 4)
                    row[form + "_scrubbed_state_GBps"] = round(
                        r.layers * mm * STATE_BYTES_PER_SLOT_LAYER / sms / 1e6, 1)
                del r
                torch.cuda.empty_cache()
            row["note"] = (("state footprint (%d MiB over 30 layers) fits the 256 MB Infinity Cache" % (mm * 60))
                           if mm * 60 < 256 else "")
            sweep[str(mm)] = row
        log("sweep done")

    # ---------------------------------------------------------------- prefill
    prefill = None
    if not args.no_prefill:
        prefill = {}
        from gen.inputs import PREFILL_L4096, RAGGED_T15717, LayerShape

        # the last two: one GPU's share of an 8-way head split of the same layer (2 q/k
        # heads, 4 v-heads), as the library runs it (chunk-parallel form) and forced to
        # walk whole sequences
        share = LayerShape(2, 4, 128, conv_width=4, chunk=64, in_dtype="bf16")
        # "_fused": the same prefill as one gdn_prefill_fused call (q/k conv inside the
        # intra-chunk kernel; bit-identical results)
        L4096, RAGGED = PREFILL_L4096, RAGGED_T15717
        runs = [(L4096, "L4096", None, 0, False), (L4096, "L4096_fused", None, 0, True),
                (RAGGED, "ragged8_T15717", None, 0, False), (RAGGED, "ragged8_T15717_fused", None, 0, True),
                (L4096, "L4096_hk2_hv4", share, 0, False), (L4096, "L4096_hk2_hv4_fused", share, 0, True),
                (L4096, "L4096_hk2_hv4_whole_sequence", share, 1, False)]
        for wid, name, shape, form, fused in runs:
            if wid == RAGGED and args.no_ragged:
                continue
            pre = PrefillRig(wid, shape=shape, form=form, fused=fused)
            settle(pre.step)
            for _ in range(W):
                pre.step()
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record()
            for _ in range(K):
                pre.step()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / K
            # the same call(s) replayed from a HIP graph (the launches without host overhead)
            graph = pre.capture()
            settle(graph.replay)
            for _ in range(W):
                graph.replay()
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record()
            for _ in range(K):
                graph.replay()
            b.record()
            torch.cuda.synchronize()
            gms = a.elapsed_time(b) / K
            del graph
            fl = pre.flops()
            prefill[name] = {
                "ms": round(ms, 4), "tokens": pre.T, "tokens_per_s": round(pre.T / (ms * 1e-3), 1),
                "graph_ms": round(gms, 4), "graph_tokens_per_s": round(pre.T / (gms * 1e-3), 1),
                "algorithmic_TFLOPs": round(fl / (ms * 1e-3) / 1e12, 2),
                "frac_of_bf16_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
                "gflop": round(fl / 1e9, 3),
                "note": ("prefill_fused" if fused else "conv_update (prefill mode) + prefill_chunked") +
                        " (bf16x3 MFMA: 3 bf16 products per "
                        "algorithmic product)" + (f"; {shape.num_k_heads} q/k heads, {shape.num_v_heads} v-heads, "
                                                 f"{'chunk-parallel' if form == 0 else 'whole-sequence'} form"
                                                 if shape is not None else "")}
            del pre
            torch.cuda.empty_cache()
            log(f"prefill {name}: {ms:.3f} ms (graph {gms:.3f} ms)")

    ceil = None
    if not args.no_ceilings:
        log("measuring the copy and matmul ceilings")
        ceil = ceilings()

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on host cores")
        cpu = cpu_baseline(args.cpu_seconds)

    if ceil and prefill:
        for row in prefill.values():
            row["frac_of_measured_bf16_matmul"] = round(row["algorithmic_TFLOPs"] / ceil["bf16_matmul_8192_TFLOPs"],
                                                        5)
    stream_ceiling = ceil["practical_hbm_GBps"] if ceil else None
    out = {
        "metric": "GDN decode state GB/s (m=64) + prefill tokens/s; % of HBM / MFMA peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(graph_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"decode step of a 30-GDN-layer hybrid: m={args.m} active slots of a 256-slot pool per "
                        f"layer, 32 v-heads / 16 k-heads, d=128, fp32 128x128 state per head, bf16 conv input "
                        f"(8192 channels, conv width 4), random per-slot state pointers; step = 30 x "
                        f"gdn_decode_fused (conv + conv-state commit + q/k L2 norm + delta rule), the conv states "
                        f"alternating between two pools, replayed as a HIP graph",
            "m": args.m, "layers": 30, "pool_slots": 256, "num_v_heads": 32, "num_k_heads": 16,
            "head_dim": 128, "parallelism": "none (1 GPU)",
        },
        "decode": {"graph_ms_per_step": round(graph_ms, 4), "eager_ms_per_step": round(head["eager_ms"], 4),
                   "state_GBps_graph": round(value, 2), "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
                   "frac_of_measured_stream_ceiling": round(value / stream_ceiling, 4) if ceil else None},
        "decode_forms": decode_forms,
        "decode_sweep": sweep,
        "prefill": prefill,
        "roofline": {"bound": "hbm", "kernel": "fused_stream_kernel<bf16, K=4, d=128, P=1> (gdn_decode_fused, "
                                               "m=64)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if args.m == 64 else None,
                     "bytes_per_launch": bytes_per_launch,
                     "avg_launch_us": round(kern_us, 2),
                     "measured_ceiling_GBps": stream_ceiling,
                     "frac_of_measured_ceiling": round(achieved / stream_ceiling, 4) if ceil else None},
        "ceilings": ceil,
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_pool,
        "host_cpu": host_cpu(),
        "wall_s": round(head["wall"], 3),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
