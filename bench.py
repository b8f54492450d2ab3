#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet layer core on one MI355X.

One step = one pass of the whole hot path:
  * decode: a 30-layer decode step at m slots (default 64) of a 256-slot pool, each
    layer = gdn_conv_update (decode mode) + gdn_decode_batched over 32 v-heads x
    128x128 fp32 states addressed through per-layer device u64 pointer arrays;
  * prefill: one 4096-token sequence (16 q/k heads, 32 v-heads, d = 128, bf16 input,
    chunk 64) = gdn_conv_update (prefill mode) + gdn_prefill_chunked.
Inputs are seeded synthetic data already resident in HBM when timing starts.

`value` is the decode state bandwidth: 30 * m * 4 MiB (each slot-layer reads and writes
its 2 MiB state once) over the decode half of the step. The prefill half is reported as
tokens/s. `roofline` is for the dominant kernel (the decode kernel), timed with HIP
events around each of its launches on the stream it runs on. `cpu_baseline` times the
fp64 oracle on a bounded sample of the same decode workload on the host.
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

HBM_PEAK_GBS = 8000.0
STATE_BYTES_PER_SLOT_LAYER = 2 * 32 * 128 * 128 * 4  # read + write of one 2 MiB state


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class DecodeRig:
    def __init__(self, m: int, layers: int = 30, pool: int = 256, n_inputs: int = 8, device="cuda"):
        import numpy as np
        import torch

        import gated_delta_rule_conv_amd as gdn
        from gen.inputs import CONFIGS, ST_PERM, make_decode_pool_torch, rng_for

        wl = CONFIGS[3]
        sh = wl.shape
        self.m, self.layers, self.sh = m, layers, sh
        self.dims = gdn.make_dims(sh.num_k_heads, sh.num_v_heads, sh.head_dim, conv_width=sh.conv_width,
                                  chunk_size=sh.chunk, in_dtype=gdn.GDN_BF16)
        self.states, self.conv_states, self.conv_w = make_decode_pool_torch(3, pool, layers, device)
        slots = rng_for(3, ST_PERM).permutation(pool)[:m].astype(np.int32)
        idx = torch.tensor(slots, dtype=torch.int32, device=device)
        self.sptr = torch.empty((layers, m), dtype=torch.int64, device=device)
        self.cptr = torch.empty((layers, m), dtype=torch.int64, device=device)
        s_bytes = self.states[0, 0].numel() * 4
        c_bytes = self.conv_states[0, 0].numel() * self.conv_states.element_size()
        for layer in range(layers):
            gdn.gdn_slot_pointers(self.states[layer].data_ptr(), s_bytes, pool, idx, m, self.sptr[layer])
            gdn.gdn_slot_pointers(self.conv_states[layer].data_ptr(), c_bytes, pool, idx, m, self.cptr[layer])
        gen = torch.Generator(device=device)
        gen.manual_seed(3100 + m)
        C, Hv = sh.channels, sh.num_v_heads
        self.n_inputs = n_inputs
        self.x = torch.randn((n_inputs, m, C), generator=gen, device=device).to(torch.bfloat16)
        self.g = -torch.nn.functional.softplus(torch.randn((n_inputs, m, Hv), generator=gen, device=device))
        self.beta = torch.sigmoid(torch.randn((n_inputs, m, Hv), generator=gen, device=device))
        self.y = torch.empty((m, C), dtype=torch.float32, device=device)
        self.o = torch.empty((m, Hv, sh.head_dim), dtype=torch.float32, device=device)
        self.slots = slots
        self.step_idx = 0

    def step(self, kernel_events=None) -> None:
        import gated_delta_rule_conv_amd as gdn
        q, k, v = gdn.qkv_views(self.dims, self.y)
        for layer in range(self.layers):
            s = (self.step_idx * self.layers + layer) % self.n_inputs
            gdn.conv_update(self.dims, self.x[s], self.y, self.conv_w[layer], None, self.cptr[layer])
            if kernel_events is not None:
                kernel_events[layer][0].record()
            gdn.gdn_decode_batched(self.dims, q, q.stride(0), k, k.stride(0), v, v.stride(0), self.g[s], self.beta[s],
                                   self.o, self.sptr[layer], self.m)
            if kernel_events is not None:
                kernel_events[layer][1].record()
        self.step_idx += 1


class PrefillRig:
    def __init__(self, cfg: int = 1, device="cuda"):
        import numpy as np
        import torch

        import gated_delta_rule_conv_amd as gdn
        from gen import make_prefill

        inp = make_prefill(cfg)
        sh = inp["shape"]
        self.sh = sh
        self.dims = gdn.make_dims(sh.num_k_heads, sh.num_v_heads, sh.head_dim, conv_width=sh.conv_width,
                                  chunk_size=sh.chunk, in_dtype=gdn.GDN_BF16)
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
        self.y = torch.empty((T, sh.channels), dtype=torch.float32, device=device)
        self.o = torch.empty((T, sh.num_v_heads, sh.head_dim), dtype=torch.float32, device=device)
        self.ws = gdn.prefill_workspace(self.dims, N, T, device=device)

    def step(self) -> None:
        import gated_delta_rule_conv_amd as gdn

        gdn.conv_update(self.dims, self.x, self.y, self.conv_w, None, self.cptr, self.cu)
        gdn.prefill(self.dims, self.y, self.g, self.beta, self.o, self.cu, self.sptr, self.ws)


def cpu_baseline(seconds: float) -> dict:
    """The fp64 oracle's decode layer, single-threaded, on host cores: slot-layers of the
    30-layer decode workload (32 v-heads x 128x128 state each), until `seconds` pass."""
    import numpy as np

    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    from gen import make_decode_pool, make_decode_step
    from oracle import decode_layer

    pool = make_decode_pool(3, pool=4)
    sh = pool["shape"]
    done = 0
    t0 = time.perf_counter()
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        step = 0
        while time.perf_counter() - t0 < seconds:
            inp = make_decode_step(3, step, 4)
            decode_layer(inp["x"], pool["conv_w"], pool["conv_state"], pool["S"], inp["g"], inp["beta"],
                         sh.num_k_heads, sh.num_v_heads, sh.head_dim, in_dtype="bf16")
            done += 4
            step += 1
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    dt = time.perf_counter() - t0
    return {"value": done * STATE_BYTES_PER_SLOT_LAYER / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} slot-layers (4 slots per call, 32 v-heads, d=128, bf16 input) in {dt:.1f} s, "
                      f"float64 NumPy, 1 thread; host has {os.cpu_count()} logical CPUs"}


def time_decode(rig: DecodeRig, steps: int, warmup: int):
    import torch

    for _ in range(warmup):
        rig.step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(rig.layers)]
           for _ in range(steps)]
    step_ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step_ev[i][0].record()
        rig.step(evs[i])
        step_ev[i][1].record()
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in step_ev]
    kern_ms = [a.elapsed_time(b) for st in evs for a, b in st]
    return step_ms, kern_ms


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--m", type=int, default=64)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--sweep", action="store_true", help="also time the decode step at m = 1, 4, 16")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (no collectives); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    torch.cuda.set_device(0)
    log(f"device {torch.cuda.get_device_name(0)}")
    rig = DecodeRig(args.m)
    log("decode rig ready")
    pre = None if args.no_prefill else PrefillRig(1)
    if pre is not None:
        log("prefill rig ready")

    # warmup of both halves
    for _ in range(args.warmup):
        rig.step()
        if pre is not None:
            pre.step()
    torch.cuda.synchronize()

    K = args.steps
    dec_ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(K)]
    pre_ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(K)]
    kern_ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
                for _ in range(rig.layers)] for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        dec_ev[i][0].record()
        rig.step(kern_ev[i])
        dec_ev[i][1].record()
        if pre is not None:
            pre_ev[i][0].record()
            pre.step()
            pre_ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    dec_ms = sum(a.elapsed_time(b) for a, b in dec_ev) / K
    kern_ms = [a.elapsed_time(b) for st in kern_ev for a, b in st]
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    pre_ms = sum(a.elapsed_time(b) for a, b in pre_ev) / K if pre is not None else None

    state_bytes_step = rig.layers * args.m * STATE_BYTES_PER_SLOT_LAYER
    value = state_bytes_step / (dec_ms * 1e-3) / 1e9
    achieved = args.m * STATE_BYTES_PER_SLOT_LAYER / (kern_avg_ms * 1e-3) / 1e9

    sweep = None
    if args.sweep:
        sweep = {}
        for mm in (1, 4, 16):
            r = DecodeRig(mm)
            step_ms, _ = time_decode(r, max(5, K // 2), 3)
            ms = sum(step_ms) / len(step_ms)
            sweep[str(mm)] = {"ms_per_step": ms, "state_GBps": r.layers * mm * STATE_BYTES_PER_SLOT_LAYER / ms / 1e6,
                              "note": "footprint under the 256 MB Infinity Cache" if mm * 60 < 256 else ""}
            del r
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on host cores")
        cpu = cpu_baseline(args.cpu_seconds)

    out = {
        "metric": "GDN decode state GB/s (m=64) + prefill tokens/s; % of HBM / MFMA peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(dec_ms + (pre_ms or 0.0), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"decode: 30 GDN layers x m={args.m} slots of a 256-slot pool, 32 v-heads / 16 k-heads, "
                        f"d=128, fp32 state, bf16 conv input, conv width 4; prefill: 1 sequence L=4096, chunk 64",
            "m": args.m, "layers": rig.layers, "pool_slots": 256, "num_v_heads": 32, "num_k_heads": 16,
            "head_dim": 128, "parallelism": "none (1 GPU)",
        },
        "decode": {"ms_per_step": round(dec_ms, 4), "state_GBps": round(value, 2),
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
                   "kernel_avg_us": round(kern_avg_ms * 1e3, 2)},
        "prefill": None if pre is None else {
            "ms": round(pre_ms, 4), "tokens_per_s": round(pre.T / (pre_ms * 1e-3), 1), "tokens": pre.T,
            "note": "conv_update (prefill mode) + prefill_chunked, one 4096-token sequence"},
        "roofline": {"bound": "hbm", "kernel": "decode_kernel<128>", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "bytes_per_launch": args.m * STATE_BYTES_PER_SLOT_LAYER},
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    if sweep is not None:
        out["decode_sweep"] = sweep
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
