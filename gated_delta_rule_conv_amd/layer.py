"""Tensor-level helpers over the C ABI (argument marshalling only).

``SlotPool`` is the caller-owned slot pool: one device allocation of equal-sized
fp32 recurrent-state blocks and one of conv-state blocks, addressed per call through
device arrays of 64-bit block addresses that gdn_slot_pointers builds on the device.
(The "qLLM" page, section "What this is", keeps the linear-attention layers' recurrent
and conv state in such a pool of slots; aprender #5279, "Phase plan", phase P5, puts
the slot index on the launch grid and hands the kernels one address per slot.)

``conv_update``, ``prefill``, ``decode`` and ``decode_fused`` derive pointers, strides and views from
torch tensors and call the library; all arithmetic happens in the HIP kernels.
"""

from __future__ import annotations

import torch

from . import _lib
from ._lib import GDN_BF16, GDN_F32, gdn_dims


def channels(dims: gdn_dims) -> int:
    return dims.head_dim * (2 * dims.num_k_heads + dims.num_v_heads)


def torch_in_dtype(dims: gdn_dims) -> torch.dtype:
    return torch.bfloat16 if dims.in_dtype == GDN_BF16 else torch.float32


class SlotPool:
    """pool_slots fixed-size slots: state [Hv, d, d] fp32 and conv state [K-1, C] in_dtype."""

    def __init__(self, dims: gdn_dims, pool_slots: int, device="cuda", state=None, conv_state=None):
        self.dims = dims
        self.pool_slots = pool_slots
        d, Hv, K, C = dims.head_dim, dims.num_v_heads, dims.conv_width, channels(dims)
        self.state = state if state is not None else torch.zeros(
            (pool_slots, Hv, d, d), dtype=torch.float32, device=device)
        self.conv_state = conv_state if conv_state is not None else torch.zeros(
            (pool_slots, K - 1, C), dtype=torch_in_dtype(dims), device=device)
        assert self.state.is_contiguous() and self.conv_state.is_contiguous()
        assert tuple(self.state.shape) == (pool_slots, Hv, d, d)
        assert tuple(self.conv_state.shape) == (pool_slots, K - 1, C)

    @property
    def state_slot_bytes(self) -> int:
        return self.state[0].numel() * 4

    @property
    def conv_slot_bytes(self) -> int:
        return self.conv_state[0].numel() * self.conv_state.element_size()

    def pointers(self, slot_idx: torch.Tensor):
        """Device u64 pointer arrays (state, conv state) for int32 slot indices on the
        device; indices outside the pool give 0 (inactive slot)."""
        assert slot_idx.dtype == torch.int32 and slot_idx.is_cuda
        m = slot_idx.numel()
        sp = torch.empty(m, dtype=torch.int64, device=slot_idx.device)
        cp = torch.empty(m, dtype=torch.int64, device=slot_idx.device)
        _lib.gdn_slot_pointers(self.state.data_ptr(), self.state_slot_bytes, self.pool_slots, slot_idx, m, sp)
        _lib.gdn_slot_pointers(self.conv_state.data_ptr(), self.conv_slot_bytes, self.pool_slots, slot_idx, m, cp)
        return sp, cp


    def copy_slots(self, src_idx: torch.Tensor, dst_idx: torch.Tensor, state: bool = True,
                   conv_state: bool = True, stream=None) -> None:
        """Snapshot / fork: slot dst_idx[i] takes the state and conv state of slot src_idx[i]
        (int32 device index tensors of equal length; destinations distinct from each other
        and from every source)."""
        assert src_idx.numel() == dst_idx.numel()
        n = src_idx.numel()
        ss, sc = self.pointers(src_idx)
        ds, dc = self.pointers(dst_idx)
        _lib.gdn_slot_copy(self.dims, ss if state else None, ds if state else None, sc if conv_state else None,
                           dc if conv_state else None, n, stream)


def qkv_views(dims: gdn_dims, y: torch.Tensor):
    """q, k, v views of the conv output y [T, C] (channels [q | k | v])."""
    hk = dims.num_k_heads * dims.head_dim
    return y[:, :hk], y[:, hk:2 * hk], y[:, 2 * hk:]


def conv_update(dims: gdn_dims, x: torch.Tensor, y: torch.Tensor, conv_w: torch.Tensor, conv_b,
                conv_state_ptrs: torch.Tensor, cu_seqlens=None, stream=None) -> None:
    n = conv_state_ptrs.numel()
    _lib.gdn_conv_update(dims, x, x.stride(0), y, y.stride(0), conv_w, conv_b, cu_seqlens, conv_state_ptrs, n,
                         x.shape[0], stream)


def prefill(dims: gdn_dims, y: torch.Tensor, g: torch.Tensor, beta: torch.Tensor, o: torch.Tensor,
            cu_seqlens: torch.Tensor, state_ptrs: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    q, k, v = qkv_views(dims, y)
    _lib.gdn_prefill_chunked(dims, q, q.stride(0), k, k.stride(0), v, v.stride(0), g, beta, o, cu_seqlens,
                             state_ptrs.numel(), y.shape[0], state_ptrs, workspace,
                             workspace.numel() * workspace.element_size(), stream)


def prefill_fused(dims: gdn_dims, x: torch.Tensor, conv_w: torch.Tensor, conv_b, g: torch.Tensor, beta: torch.Tensor,
                  o: torch.Tensor, cu_seqlens: torch.Tensor, state_ptrs: torch.Tensor, conv_state_ptrs: torch.Tensor,
                  workspace: torch.Tensor, stream=None) -> None:
    """conv_update (prefill mode) + prefill in one call; workspace from prefill_fused_workspace()."""
    _lib.gdn_prefill_fused(dims, x, x.stride(0), conv_w, conv_b, g, beta, o, cu_seqlens, state_ptrs.numel(),
                           x.shape[0], state_ptrs, conv_state_ptrs, workspace,
                           workspace.numel() * workspace.element_size(), stream)


def prefill_fused_static(dims: gdn_dims, x: torch.Tensor, conv_w: torch.Tensor, conv_b, g: torch.Tensor,
                         beta: torch.Tensor, o: torch.Tensor, cu_seqlens: torch.Tensor, state_ptrs: torch.Tensor,
                         conv_state_ptrs: torch.Tensor, stream=None) -> None:
    """prefill_fused with the library's own 64 MiB device workspace: nothing allocated."""
    _lib.gdn_prefill_fused_static(dims, x, x.stride(0), conv_w, conv_b, g, beta, o, cu_seqlens, state_ptrs.numel(),
                                  x.shape[0], state_ptrs, conv_state_ptrs, stream)


def decode(dims: gdn_dims, y: torch.Tensor, g: torch.Tensor, beta: torch.Tensor, o: torch.Tensor,
           state_ptrs: torch.Tensor, stream=None) -> None:
    q, k, v = qkv_views(dims, y)
    _lib.gdn_decode_batched(dims, q, q.stride(0), k, k.stride(0), v, v.stride(0), g, beta, o, state_ptrs,
                            state_ptrs.numel(), stream)


def decode_fused(dims: gdn_dims, x: torch.Tensor, conv_w: torch.Tensor, conv_b, g: torch.Tensor, beta: torch.Tensor,
                 o: torch.Tensor, state_ptrs: torch.Tensor, conv_state_ptrs: torch.Tensor,
                 conv_state_out_ptrs=None, stream=None) -> None:
    """conv_update (decode mode) + decode in one launch. The new conv states go to
    conv_state_out_ptrs (other buffers, the faster form) or, when None, in place."""
    _lib.gdn_decode_fused(dims, x, x.stride(0), conv_w, conv_b, g, beta, o, state_ptrs, conv_state_ptrs,
                          conv_state_out_ptrs, state_ptrs.numel(), stream)


def prefill_workspace(dims: gdn_dims, num_seqs: int, total_tokens: int, device="cuda") -> torch.Tensor:
    nbytes = _lib.gdn_prefill_workspace_size(dims, num_seqs, total_tokens)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def prefill_fused_workspace(dims: gdn_dims, num_seqs: int, total_tokens: int, device="cuda") -> torch.Tensor:
    nbytes = _lib.gdn_prefill_fused_workspace_size(dims, num_seqs, total_tokens)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


__all__ = ["SlotPool", "channels", "conv_update", "decode", "decode_fused", "prefill", "prefill_fused",
           "prefill_fused_static", "prefill_fused_workspace", "prefill_workspace", "qkv_views", "torch_in_dtype",
           "GDN_F32", "GDN_BF16"]
