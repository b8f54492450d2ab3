"""The shared input generator: seeding, shapes and bf16 rounding.

bf16 rounding is checked against torch's float32 -> bfloat16 cast (round to
nearest, ties to even), a library routine independent of the generator."""

import numpy as np
import torch

from gen import DECODE_M16_POOL64, PREFILL_L4096, RAGGED_T15717, TINY_FP32, WORKLOADS, bf16_bits_from_f32, make_decode_pool, make_decode_step, make_prefill


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0, 1e-40, 3e38],
                                 dtype=np.float32)])
    ours = bf16_bits_from_f32(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_seeded_and_shaped():
    a = make_prefill(RAGGED_T15717)
    np.testing.assert_array_equal(make_prefill(PREFILL_L4096, lens=(5,))["x"], make_prefill(PREFILL_L4096, lens=(5,))["x"])
    sh = WORKLOADS[RAGGED_T15717].shape
    T = sum(WORKLOADS[RAGGED_T15717].lens)
    assert T == 15717
    assert a["x"].shape == (T, sh.channels) and a["x"].dtype == np.uint16
    assert a["cu_seqlens"][-1] == T and a["cu_seqlens"].dtype == np.int32
    assert a["S0"].shape == (8, 32, 128, 128)
    assert np.all(a["g"] < 0) and np.all((a["beta"] > 0) & (a["beta"] < 1))
    p = make_decode_pool(DECODE_M16_POOL64)
    assert sorted(p["perm"].tolist()) == list(range(64))
    s = make_decode_step(DECODE_M16_POOL64, 5, 16)
    assert s["x"].shape == (16, sh.channels)
    c0 = make_prefill(TINY_FP32)
    assert c0["x"].dtype == np.float32 and np.all(c0["S0"] == 0) and np.all(c0["conv_state"] == 0)
