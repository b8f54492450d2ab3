"""Seeded input recipes for the Gated DeltaNet layer core.

Every tensor comes from ``numpy.random.default_rng([1000 + workload id, stream,
...])`` with one stream id per tensor, so any tensor of any workload can be
rebuilt on its own. Values are drawn in float64, cast to float32, and (for bf16 storage)
rounded to bfloat16 with round-to-nearest-even done on the integer bits.

Distributions (the workloads described for the layer):
  x (conv input over the q|k|v channels) ~ N(0, 1)
  conv weights ~ U(-0.5, 0.5)   (PyTorch's default bound 1/sqrt(fan_in), fan_in = 4)
  g = -softplus(z), beta = sigmoid(z), z ~ N(0, 1)   (float32)
  initial recurrent state ~ N(0, sigma)   (sigma is a standard deviation)
  conv state ~ N(0, 1) or zero
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

# stream ids, one per tensor kind
ST_X, ST_CONV_W, ST_CONV_STATE, ST_G, ST_BETA, ST_S0, ST_PERM, ST_CONV_B = 0, 1, 2, 3, 4, 5, 6, 7
ST_STEP_BASE = 100  # decode step s draws its x/g/beta from stream 100 + s


@dataclass(frozen=True)
class LayerShape:
    num_k_heads: int
    num_v_heads: int
    head_dim: int  # d_k = d_v
    conv_width: int = 4
    chunk: int = 64
    in_dtype: str = "bf16"  # storage dtype of x, conv weights, conv state

    @property
    def channels(self) -> int:
        """Conv channel count over [q | k | v]."""
        return 2 * self.num_k_heads * self.head_dim + self.num_v_heads * self.head_dim


@dataclass(frozen=True)
class Workload:
    wid: int  # workload id (also the seed of its generators)
    name: str
    shape: LayerShape
    s0_std: float
    conv_state_std: float  # 0 means a zero conv state
    lens: tuple = ()
    m: int = 0
    ms: tuple = ()
    pool: int = 0
    steps: int = 0
    layers: int = 1
    notes: dict = field(default_factory=dict)


_QWEN_LIKE = LayerShape(num_k_heads=16, num_v_heads=32, head_dim=128, conv_width=4, chunk=64, in_dtype="bf16")

# Workload ids; each also seeds its tensors' generators.
TINY_FP32 = 0          # 1 sequence, L = 64, 2/2 heads, d = 32, chunk 16, fp32, zero initial state
PREFILL_L4096 = 1      # 1 sequence, L = 4096, 16 q/k / 32 v heads, d = 128, bf16
DECODE_M16_POOL64 = 2  # 16 active slots of a 64-slot pool, 64 decode steps
DECODE_30_LAYERS = 3   # m in {1, 4, 16, 64} of a 256-slot pool per layer, 30 layers
RAGGED_T15717 = 4      # 8 packed sequences of lengths 1 .. 8192, T = 15717

WORKLOADS = {
    TINY_FP32: Workload(TINY_FP32, "tiny_fp32_L64_h2_d32",
                        LayerShape(2, 2, 32, conv_width=4, chunk=16, in_dtype="f32"),
                        s0_std=0.0, conv_state_std=0.0, lens=(64,)),
    PREFILL_L4096: Workload(PREFILL_L4096, "prefill_L4096_hk16_hv32_d128", _QWEN_LIKE,
                            s0_std=0.02, conv_state_std=0.0, lens=(4096,)),
    DECODE_M16_POOL64: Workload(DECODE_M16_POOL64, "decode_m16_pool64_64steps", _QWEN_LIKE,
                                s0_std=0.05, conv_state_std=1.0, m=16, pool=64, steps=64),
    DECODE_30_LAYERS: Workload(DECODE_30_LAYERS, "decode_30layers_pool256", _QWEN_LIKE,
                               s0_std=0.05, conv_state_std=1.0, ms=(1, 4, 16, 64), pool=256, layers=30),
    RAGGED_T15717: Workload(RAGGED_T15717, "ragged_prefill_8seq_T15717", _QWEN_LIKE,
                            s0_std=0.02, conv_state_std=1.0, lens=(1, 17, 64, 300, 1000, 2048, 4095, 8192)),
}


def rng_for(wid: int, stream: int, *sub: int) -> np.random.Generator:
    return np.random.default_rng([1000 + int(wid), int(stream), *[int(s) for s in sub]])


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits.

    Inputs are finite by construction (normal / uniform draws)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    # finite inputs: u + 0x8000 stays below 2**32, so uint32 arithmetic cannot wrap
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def _store(a64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 draw -> storage array: float32, or uint16 bf16 bits."""
    if dtype == "f32":
        return np.ascontiguousarray(a64, dtype=np.float32)
    if dtype != "bf16":
        raise ValueError(dtype)
    flat = np.asarray(a64).reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 20  # blocks keep the temporaries in cache
    for i in range(0, flat.size, step):
        out[i:i + step] = bf16_bits_from_f32(flat[i:i + step].astype(np.float32))
    return out.reshape(np.shape(a64))


def _gates(rng_g, rng_b, shape):
    zg = rng_g.standard_normal(shape)
    zb = rng_b.standard_normal(shape)
    g = (-np.logaddexp(0.0, zg)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    return g, beta


def make_prefill(wid: int, lens=None, shape: LayerShape | None = None, s0_std=None,
                 conv_state_std=None, with_bias: bool = False) -> dict:
    """Packed ragged prefill inputs.

    Returns x [T, C] (storage dtype), conv_w [C, K], conv_b [C] or None,
    cu_seqlens int32 [N+1], conv_state [N, K-1, C] (storage dtype),
    g, beta float32 [T, Hv], S0 float32 [N, Hv, d, d]."""
    wl = WORKLOADS[wid]
    shape = shape or wl.shape
    lens = tuple(wl.lens if lens is None else lens)
    s0_std = wl.s0_std if s0_std is None else s0_std
    conv_state_std = wl.conv_state_std if conv_state_std is None else conv_state_std
    C, K, d, Hv = shape.channels, shape.conv_width, shape.head_dim, shape.num_v_heads
    N, T = len(lens), int(sum(lens))
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    x = _store(rng_for(wid, ST_X).standard_normal((T, C)), shape.in_dtype)
    conv_w = _store(rng_for(wid, ST_CONV_W).uniform(-0.5, 0.5, (C, K)), shape.in_dtype)
    conv_b = _store(rng_for(wid, ST_CONV_B).uniform(-0.5, 0.5, (C,)), shape.in_dtype) if with_bias else None
    cs = rng_for(wid, ST_CONV_STATE).standard_normal((N, K - 1, C)) * conv_state_std
    conv_state = _store(cs, shape.in_dtype)
    g, beta = _gates(rng_for(wid, ST_G), rng_for(wid, ST_BETA), (T, Hv))
    S0 = (rng_for(wid, ST_S0).standard_normal((N, Hv, d, d)) * s0_std).astype(np.float32)
    return dict(shape=shape, lens=lens, x=x, conv_w=conv_w, conv_b=conv_b, cu_seqlens=cu,
                conv_state=conv_state, g=g, beta=beta, S0=S0)


def make_decode_pool(wid: int, pool: int | None = None, shape: LayerShape | None = None,
                     s0_std=None, conv_state_std=None, with_bias: bool = False) -> dict:
    """One layer's slot pool: conv weights, per-slot conv states and recurrent states,
    and a seeded permutation of the slot indices."""
    wl = WORKLOADS[wid]
    shape = shape or wl.shape
    pool = wl.pool if pool is None else pool
    s0_std = wl.s0_std if s0_std is None else s0_std
    conv_state_std = wl.conv_state_std if conv_state_std is None else conv_state_std
    C, K, d, Hv = shape.channels, shape.conv_width, shape.head_dim, shape.num_v_heads
    conv_w = _store(rng_for(wid, ST_CONV_W).uniform(-0.5, 0.5, (C, K)), shape.in_dtype)
    conv_b = _store(rng_for(wid, ST_CONV_B).uniform(-0.5, 0.5, (C,)), shape.in_dtype) if with_bias else None
    conv_state = _store(rng_for(wid, ST_CONV_STATE).standard_normal((pool, K - 1, C)) * conv_state_std,
                        shape.in_dtype)
    S = (rng_for(wid, ST_S0).standard_normal((pool, Hv, d, d)) * s0_std).astype(np.float32)
    perm = rng_for(wid, ST_PERM).permutation(pool).astype(np.int32)
    return dict(shape=shape, pool=pool, conv_w=conv_w, conv_b=conv_b, conv_state=conv_state, S=S, perm=perm)


def make_decode_step(wid: int, step: int, m: int, shape: LayerShape | None = None) -> dict:
    """One decode step's per-slot inputs: x [m, C], g and beta [m, Hv]."""
    wl = WORKLOADS[wid]
    shape = shape or wl.shape
    C, Hv = shape.channels, shape.num_v_heads
    s = ST_STEP_BASE + int(step)
    x = _store(rng_for(wid, s, ST_X).standard_normal((m, C)), shape.in_dtype)
    g, beta = _gates(rng_for(wid, s, ST_G), rng_for(wid, s, ST_BETA), (m, Hv))
    return dict(x=x, g=g, beta=beta)


def make_decode_pool_torch(wid: int, pool: int, layers: int, device, shape: LayerShape | None = None,
                           s0_std=None, conv_state_std=None):
    """Large slot pools drawn directly in device memory (torch's seeded generator), for
    workloads whose state does not fit a host-side draw in reasonable time.

    Returns (states [layers, pool, Hv, d, d] f32, conv_states [layers, pool, K-1, C] bf16/f32,
    conv_w [layers, C, K]). Values follow the same distributions as the host recipes; the
    bits differ from the host recipes (a different generator), so checks against the oracle
    copy the sampled slots back to the host first."""
    import torch

    wl = WORKLOADS[wid]
    shape = shape or wl.shape
    s0_std = wl.s0_std if s0_std is None else s0_std
    conv_state_std = wl.conv_state_std if conv_state_std is None else conv_state_std
    C, K, d, Hv = shape.channels, shape.conv_width, shape.head_dim, shape.num_v_heads
    tdt = torch.bfloat16 if shape.in_dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 + wid)
    states = torch.empty((layers, pool, Hv, d, d), dtype=torch.float32, device=device)
    for layer in range(layers):
        states[layer].normal_(0.0, s0_std, generator=gen)
    conv_states = (torch.randn((layers, pool, K - 1, C), generator=gen, device=device) * conv_state_std).to(tdt)
    conv_w = (torch.rand((layers, C, K), generator=gen, device=device) - 0.5).to(tdt)
    return states, conv_states, conv_w


def with_lens(wid: int, lens) -> Workload:
    return replace(WORKLOADS[wid], lens=tuple(lens))
