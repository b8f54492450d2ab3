"""Helpers for the GPU parity tests: moving seeded inputs to the device, the normwise
error metric, and printing which case is about to run (flushed, so a run that dies
still names its case)."""

from __future__ import annotations

import sys

import numpy as np

TOL_BF16 = 2e-3  # bf16 inputs, fp32 state: max normwise relative error
TOL_F32 = 1e-5  # fp32 inputs


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a, dtype: str, device="cuda"):
    """numpy storage array (float32, or uint16 bf16 bits) -> torch device tensor."""
    import torch

    if a is None:
        return None
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def bits_of(t) -> np.ndarray:
    """Host copy of a tensor's raw bits (for bit-exact comparisons)."""
    import torch

    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().copy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().copy()
    return t.numpy().copy()


def storage_of(t, dtype: str) -> np.ndarray:
    """Device tensor -> numpy storage array in the generator's convention."""
    import torch

    t = t.detach().contiguous().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().astype(np.float32)


def normwise_err(gpu, ref) -> float:
    """max |gpu - ref| / max |ref| over one block (0 when both are 0)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(gpu - ref).max() if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def max_block_err_o(o_gpu, o_ref, cu) -> float:
    """o [T, H, d]; blocks are (sequence, v-head)."""
    worst = 0.0
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for j in range(o_ref.shape[1]):
            worst = max(worst, normwise_err(o_gpu[a:b, j], o_ref[a:b, j]))
    return worst


def max_block_err_S(S_gpu, S_ref) -> float:
    """S [N, H, d, d]; blocks are (sequence or slot, v-head)."""
    worst = 0.0
    for s in range(S_ref.shape[0]):
        for j in range(S_ref.shape[1]):
            worst = max(worst, normwise_err(S_gpu[s, j], S_ref[s, j]))
    return worst
