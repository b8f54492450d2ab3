"""ctypes binding of libgdn.so: the C-ABI entry points under the same names.

Argument marshalling only. Tensors are passed as raw device addresses (``data_ptr``);
the stream defaults to torch's current stream on the tensors' device. Every step of
the layer runs inside the library's HIP kernels: there is no fallback of any kind,
and importing this module fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_ALIGN, GDN_ERR_WORKSPACE, GDN_ERR_UNSUPPORTED, \
    GDN_ERR_HIP = range(8)
STATUS_NAMES = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_DTYPE", 4: "GDN_ERR_ALIGN",
                5: "GDN_ERR_WORKSPACE", 6: "GDN_ERR_UNSUPPORTED", 7: "GDN_ERR_HIP"}
GDN_F32, GDN_BF16 = 0, 1
GDN_ACT_NONE, GDN_ACT_SILU = 0, 1
GDN_MMA_AUTO, GDN_MMA_FP32, GDN_MMA_BF16X3 = 0, 1, 2
GDN_PREFILL_AUTO, GDN_PREFILL_WHOLE, GDN_PREFILL_SEGMENTS = 0, 1, 2

EXPORTED = ("gdn_dims_init", "gdn_conv_update", "gdn_prefill_workspace_size", "gdn_prefill_chunked",
            "gdn_prefill_fused_workspace_size", "gdn_prefill_fused", "gdn_prefill_fused_static", "gdn_decode_batched",
            "gdn_decode_fused",
            "gdn_slot_copy", "gdn_slot_pointers", "gdn_last_error", "gdn_abi_version", "gdn_hbm_probe")


class gdn_dims(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("conv_width", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("activation", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("mma", ctypes.c_int32),
        ("l2_eps", ctypes.c_float),
        ("scale", ctypes.c_float),
        ("prefill_form", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("qk_l2norm_off", ctypes.c_int32),
    ]


def make_dims(num_k_heads: int, num_v_heads: int, head_dim: int, conv_width: int = 4, chunk_size: int = 64,
              activation: int = GDN_ACT_NONE, in_dtype: int = GDN_BF16, mma: int = GDN_MMA_AUTO,
              l2_eps: float = 1e-6, scale: float = 1.0, prefill_form: int = 0, out_dtype: int = GDN_F32,
              qk_l2norm: bool = True) -> gdn_dims:
    """gdn_dims with struct_size set; ``qk_l2norm=False`` sets the struct's qk_l2norm_off."""
    return gdn_dims(ctypes.sizeof(gdn_dims), num_k_heads, num_v_heads, head_dim, conv_width, chunk_size,
                    activation, in_dtype, mma, l2_eps, scale, prefill_form, out_dtype, 0 if qk_l2norm else 1)


class GDNError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {text}")
        self.status = status


def _hip_runtimes() -> set:
    """Distinct HIP runtime files mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            return {ln.split()[-1] for ln in f if "libamdhip64.so" in ln}
    except OSError:  # pragma: no cover
        return set()


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with gated_delta_rule_conv_amd/build_lib.py "
                          "(or __graft_entry__.build()); there is no fallback path")
    # The library takes device pointers and hipStream_t handles made by torch, so it has
    # to run on the HIP runtime torch already loaded. Both runtimes carry the soname
    # libamdhip64.so.7: importing torch first makes the loader reuse torch's copy for
    # libgdn.so instead of mapping a second, independent runtime.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are mapped into this process ({sorted(runtimes)}); libgdn.so must "
                          "share torch's runtime")
    P, I32, I64, U64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
    D = ctypes.POINTER(gdn_dims)
    lib.gdn_dims_init.argtypes = [D, I32, I32, I32]
    lib.gdn_conv_update.argtypes = [D, P, I64, P, I64, P, P, P, P, I32, I32, P]
    lib.gdn_prefill_workspace_size.argtypes = [D, I32, I32, ctypes.POINTER(SZ)]
    lib.gdn_prefill_chunked.argtypes = [D, P, I64, P, I64, P, I64, P, P, P, P, I32, I32, P, P, SZ, P]
    lib.gdn_prefill_fused_workspace_size.argtypes = [D, I32, I32, ctypes.POINTER(SZ)]
    lib.gdn_prefill_fused.argtypes = [D, P, I64, P, P, P, P, P, P, I32, I32, P, P, P, SZ, P]
    lib.gdn_prefill_fused_static.argtypes = [D, P, I64, P, P, P, P, P, P, I32, I32, P, P, P]
    lib.gdn_decode_batched.argtypes = [D, P, I64, P, I64, P, I64, P, P, P, P, I32, P]
    lib.gdn_decode_fused.argtypes = [D, P, I64, P, P, P, P, P, P, P, P, I32, P]
    lib.gdn_slot_copy.argtypes = [D, P, P, P, P, I32, P]
    lib.gdn_slot_pointers.argtypes = [U64, I64, I32, P, I32, P, P]
    for fn in ("gdn_dims_init", "gdn_conv_update", "gdn_prefill_workspace_size", "gdn_prefill_chunked",
               "gdn_prefill_fused_workspace_size", "gdn_prefill_fused", "gdn_prefill_fused_static", "gdn_decode_batched",
               "gdn_decode_fused", "gdn_slot_copy", "gdn_slot_pointers"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.gdn_hbm_probe.argtypes = [P, SZ, ctypes.c_uint32, P]
    lib.gdn_hbm_probe.restype = ctypes.c_int
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = ctypes.c_int32
    return lib


_LIB = _load()


def lib() -> ctypes.CDLL:
    return _LIB


def _ptr(t) -> int | None:
    """Device address of a tensor, an int address, or None (NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream, *tensors) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    for t in tensors:
        if t is not None and not isinstance(t, int) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(fn: str, status: int) -> None:
    if status != GDN_OK:
        raise GDNError(fn, status, (_LIB.gdn_last_error() or b"").decode())


def gdn_last_error() -> str:
    return (_LIB.gdn_last_error() or b"").decode()


def gdn_abi_version() -> int:
    return int(_LIB.gdn_abi_version())


def gdn_dims_init(num_k_heads: int, num_v_heads: int, head_dim: int) -> gdn_dims:
    """The library's default-filled gdn_dims for these sizes."""
    d = gdn_dims()
    _check("gdn_dims_init", _LIB.gdn_dims_init(ctypes.byref(d), num_k_heads, num_v_heads, head_dim))
    return d


def gdn_conv_update(dims: gdn_dims, x, x_stride: int, y, y_stride: int, conv_w, conv_b, cu_seqlens,
                    conv_state_ptrs, n: int, total_tokens: int, stream=None) -> None:
    st = _LIB.gdn_conv_update(ctypes.byref(dims), _ptr(x), x_stride, _ptr(y), y_stride, _ptr(conv_w), _ptr(conv_b),
                              _ptr(cu_seqlens), _ptr(conv_state_ptrs), n, total_tokens,
                              _stream(stream, x, y, conv_state_ptrs))
    _check("gdn_conv_update", st)


def gdn_prefill_workspace_size(dims: gdn_dims, num_seqs: int, total_tokens: int) -> int:
    out = ctypes.c_size_t(0)
    _check("gdn_prefill_workspace_size",
           _LIB.gdn_prefill_workspace_size(ctypes.byref(dims), num_seqs, total_tokens, ctypes.byref(out)))
    return int(out.value)


def gdn_prefill_chunked(dims: gdn_dims, q, q_stride: int, k, k_stride: int, v, v_stride: int, g, beta, o,
                        cu_seqlens, num_seqs: int, total_tokens: int, state_ptrs, workspace, workspace_bytes: int,
                        stream=None) -> None:
    st = _LIB.gdn_prefill_chunked(ctypes.byref(dims), _ptr(q), q_stride, _ptr(k), k_stride, _ptr(v), v_stride,
                                  _ptr(g), _ptr(beta), _ptr(o), _ptr(cu_seqlens), num_seqs, total_tokens,
                                  _ptr(state_ptrs), _ptr(workspace), workspace_bytes,
                                  _stream(stream, q, o, state_ptrs))
    _check("gdn_prefill_chunked", st)


def gdn_prefill_fused_workspace_size(dims: gdn_dims, num_seqs: int, total_tokens: int) -> int:
    out = ctypes.c_size_t(0)
    _check("gdn_prefill_fused_workspace_size",
           _LIB.gdn_prefill_fused_workspace_size(ctypes.byref(dims), num_seqs, total_tokens, ctypes.byref(out)))
    return int(out.value)


def gdn_prefill_fused(dims: gdn_dims, x, x_stride: int, conv_w, conv_b, g, beta, o, cu_seqlens, num_seqs: int,
                      total_tokens: int, state_ptrs, conv_state_ptrs, workspace, workspace_bytes: int,
                      stream=None) -> None:
    st = _LIB.gdn_prefill_fused(ctypes.byref(dims), _ptr(x), x_stride, _ptr(conv_w), _ptr(conv_b), _ptr(g),
                                _ptr(beta), _ptr(o), _ptr(cu_seqlens), num_seqs, total_tokens, _ptr(state_ptrs),
                                _ptr(conv_state_ptrs), _ptr(workspace), workspace_bytes,
                                _stream(stream, x, o, state_ptrs))
    _check("gdn_prefill_fused", st)


GDN_STATIC_SCRATCH_BYTES = 64 << 20


def gdn_prefill_fused_static(dims: gdn_dims, x, x_stride: int, conv_w, conv_b, g, beta, o, cu_seqlens,
                             num_seqs: int, total_tokens: int, state_ptrs, conv_state_ptrs, stream=None) -> None:
    st = _LIB.gdn_prefill_fused_static(ctypes.byref(dims), _ptr(x), x_stride, _ptr(conv_w), _ptr(conv_b), _ptr(g),
                                       _ptr(beta), _ptr(o), _ptr(cu_seqlens), num_seqs, total_tokens,
                                       _ptr(state_ptrs), _ptr(conv_state_ptrs), _stream(stream, x, o, state_ptrs))
    _check("gdn_prefill_fused_static", st)


def gdn_decode_batched(dims: gdn_dims, q, q_stride: int, k, k_stride: int, v, v_stride: int, g, beta, o,
                       state_ptrs, m: int, stream=None) -> None:
    st = _LIB.gdn_decode_batched(ctypes.byref(dims), _ptr(q), q_stride, _ptr(k), k_stride, _ptr(v), v_stride,
                                 _ptr(g), _ptr(beta), _ptr(o), _ptr(state_ptrs), m, _stream(stream, q, o, state_ptrs))
    _check("gdn_decode_batched", st)


def gdn_decode_fused(dims: gdn_dims, x, x_stride: int, conv_w, conv_b, g, beta, o, state_ptrs, conv_state_ptrs,
                     conv_state_out_ptrs, m: int, stream=None) -> None:
    st = _LIB.gdn_decode_fused(ctypes.byref(dims), _ptr(x), x_stride, _ptr(conv_w), _ptr(conv_b), _ptr(g),
                               _ptr(beta), _ptr(o), _ptr(state_ptrs), _ptr(conv_state_ptrs),
                               _ptr(conv_state_out_ptrs), m, _stream(stream, x, o, state_ptrs))
    _check("gdn_decode_fused", st)


def gdn_slot_copy(dims: gdn_dims, src_state_ptrs, dst_state_ptrs, src_conv_ptrs, dst_conv_ptrs, n: int,
                  stream=None) -> None:
    st = _LIB.gdn_slot_copy(ctypes.byref(dims), _ptr(src_state_ptrs), _ptr(dst_state_ptrs), _ptr(src_conv_ptrs),
                            _ptr(dst_conv_ptrs), n,
                            _stream(stream, src_state_ptrs, dst_state_ptrs, src_conv_ptrs, dst_conv_ptrs))
    _check("gdn_slot_copy", st)


def gdn_hbm_probe(buf, nbytes: int, salt: int = 0, stream=None) -> None:
    """Measurement helper (include/gdn_probe.h): an in-place streaming pass over buf."""
    st = _LIB.gdn_hbm_probe(_ptr(buf), nbytes, salt, _stream(stream, buf))
    if st != GDN_OK:
        raise GDNError("gdn_hbm_probe", st, "buffer NULL, misaligned or not a multiple of 16 KiB")


def gdn_slot_pointers(pool_base: int, slot_bytes: int, pool_slots: int, slot_idx, m: int, out_ptrs,
                      stream=None) -> None:
    st = _LIB.gdn_slot_pointers(ctypes.c_uint64(pool_base), slot_bytes, pool_slots, _ptr(slot_idx), m,
                                _ptr(out_ptrs), _stream(stream, slot_idx, out_ptrs))
    _check("gdn_slot_pointers", st)
