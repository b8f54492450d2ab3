"""Host-side tests of the C-ABI library (no GPU needed).

The library must load without a GPU, export every entry point include/gdn.h declares,
and reject every invalid call with the documented status before any HIP call. Every
call below carries at least one argument that fails a host check, so none of them
can launch a kernel (the fake addresses are never dereferenced).
"""

import ctypes
import os
import re

import pytest

import gated_delta_rule_conv_amd as gdn
from gated_delta_rule_conv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def _declared_symbols():
    """Every function declared in include/*.h."""
    syms = set()
    for name in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if name.endswith(".h"):
            with open(os.path.join(ROOT, "include", name)) as f:
                text = f.read()
            syms |= set(re.findall(r"^(?:gdn_status|const char\*|int32_t)\s+(gdn_\w+)\s*\(", text, re.M))
    return sorted(syms)


def test_header_symbols_are_exported():
    syms = _declared_symbols()
    assert set(syms) == set(_lib.EXPORTED)
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), s


def test_abi_version_and_struct_size():
    assert gdn.gdn_abi_version() == 6
    assert ctypes.sizeof(_lib.gdn_dims) == 14 * 4


def dims(**kw):
    base = dict(num_k_heads=16, num_v_heads=32, head_dim=128, conv_width=4, chunk_size=64)
    base.update(kw)
    return gdn.make_dims(**base)


def _status(fn, *args):
    with pytest.raises(gdn.GDNError) as e:
        fn(*args)
    return e.value.status, str(e.value)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), _lib.GDN_ERR_UNSUPPORTED),
    (dict(conv_width=5), _lib.GDN_ERR_UNSUPPORTED),
    (dict(conv_width=1), _lib.GDN_ERR_UNSUPPORTED),
    (dict(chunk_size=128), _lib.GDN_ERR_UNSUPPORTED),
    (dict(num_k_heads=3, num_v_heads=32), _lib.GDN_ERR_SHAPE),
    (dict(num_k_heads=0), _lib.GDN_ERR_SHAPE),
    (dict(in_dtype=7), _lib.GDN_ERR_DTYPE),
    (dict(out_dtype=2), _lib.GDN_ERR_DTYPE),
    (dict(qk_l2norm_off=2), _lib.GDN_ERR_DTYPE),
    (dict(activation=3), _lib.GDN_ERR_DTYPE),
    (dict(mma=9), _lib.GDN_ERR_DTYPE),
    (dict(l2_eps=-1.0), _lib.GDN_ERR_SHAPE),
    (dict(scale=0.0), _lib.GDN_ERR_SHAPE),
    (dict(scale=float("inf")), _lib.GDN_ERR_SHAPE),
    (dict(prefill_form=3), _lib.GDN_ERR_DTYPE),
])
def test_bad_dims_rejected_everywhere(kw, status):
    """Every enumerated field or switch with an unknown value gives GDN_ERR_DTYPE; an
    out-of-range number gives GDN_ERR_SHAPE; a size that is not built, _UNSUPPORTED."""
    raw = {k: kw.pop(k) for k in list(kw) if k == "qk_l2norm_off"}
    d = dims(**kw)
    for k, val in raw.items():
        setattr(d, k, val)
    st, _ = _status(gdn.gdn_prefill_workspace_size, d, 1, 10)
    assert st == status
    st, _ = _status(gdn.gdn_decode_batched, d, FAKE, 4096, FAKE, 4096, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, 4, 0)
    assert st == status
    st, _ = _status(gdn.gdn_conv_update, d, FAKE, 8192, FAKE, 8192, FAKE, None, FAKE, FAKE, 1, 4, 0)
    assert st == status


def test_struct_size_checked():
    d = dims()
    d.struct_size = 12
    st, msg = _status(gdn.gdn_prefill_workspace_size, d, 1, 10)
    assert st == _lib.GDN_ERR_SHAPE and "struct_size" in msg


def test_null_dims():
    lib = _lib.lib()
    size = ctypes.c_size_t()
    assert lib.gdn_prefill_workspace_size(None, 1, 1, ctypes.byref(size)) == _lib.GDN_ERR_NULL
    assert "dims" in gdn.gdn_last_error()


def test_decode_argument_checks():
    d = dims()
    ok = (FAKE, 4096, FAKE, 4096, FAKE, 4096, FAKE, FAKE, FAKE)
    # missing state pointer array
    assert _status(gdn.gdn_decode_batched, d, *ok, None, 4, 0)[0] == _lib.GDN_ERR_NULL
    # missing o
    assert _status(gdn.gdn_decode_batched, d, FAKE, 4096, FAKE, 4096, FAKE, 4096, FAKE, FAKE, None, FAKE, 4,
                   0)[0] == _lib.GDN_ERR_NULL
    # misaligned q
    assert _status(gdn.gdn_decode_batched, d, FAKE + 4, 4096, FAKE, 4096, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, 4,
                   0)[0] == _lib.GDN_ERR_ALIGN
    # stride not a multiple of 4 elements
    assert _status(gdn.gdn_decode_batched, d, FAKE, 4098, FAKE, 4096, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, 4,
                   0)[0] == _lib.GDN_ERR_ALIGN
    # stride below the row width
    assert _status(gdn.gdn_decode_batched, d, FAKE, 1024, FAKE, 4096, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, 4,
                   0)[0] == _lib.GDN_ERR_SHAPE
    assert _status(gdn.gdn_decode_batched, d, *ok, FAKE, -1, 0)[0] == _lib.GDN_ERR_SHAPE
    assert _status(gdn.gdn_decode_batched, d, *ok, FAKE, 70000, 0)[0] == _lib.GDN_ERR_SHAPE
    # m = 0 is a no-op that launches nothing
    gdn.gdn_decode_batched(d, *ok, FAKE, 0, 0)


def test_decode_fused_argument_checks():
    d = dims()
    C = 8192
    pre = (FAKE, C, FAKE, None, FAKE, FAKE, FAKE)  # x, x_stride, conv_w, conv_b, g, beta, o

    def call(*args, dm=d):
        return _status(gdn.gdn_decode_fused, dm, *args)[0]

    # the state and conv-state pointer arrays are required (the output array is optional)
    assert call(*pre, None, FAKE, None, 4, 0) == _lib.GDN_ERR_NULL
    assert call(*pre, FAKE, None, None, 4, 0) == _lib.GDN_ERR_NULL
    assert call(*pre, FAKE, None, FAKE, 4, 0) == _lib.GDN_ERR_NULL
    assert call(None, *pre[1:], FAKE, FAKE, None, 4, 0) == _lib.GDN_ERR_NULL
    # x stride below C, or not a multiple of 16 bytes; misaligned x
    assert call(FAKE, C - 8, *pre[2:], FAKE, FAKE, None, 4, 0) == _lib.GDN_ERR_SHAPE
    assert call(FAKE, C + 4, *pre[2:], FAKE, FAKE, None, 4, 0) == _lib.GDN_ERR_ALIGN
    assert call(FAKE + 8, C, *pre[2:], FAKE, FAKE, None, 4, 0) == _lib.GDN_ERR_ALIGN
    assert call(*pre, FAKE, FAKE, None, -1, 0) == _lib.GDN_ERR_SHAPE
    # in place, one workgroup per (slot, k-head) holds the conv output of the k-head's q, k
    # and its v-heads in LDS: (2 + Hv/Hk) * d * 4 bytes may not exceed 64 KiB
    wide = dims(num_k_heads=1, num_v_heads=200, head_dim=128)
    st, msg = _status(gdn.gdn_decode_fused, wide, FAKE, 202 * 128, *pre[2:], FAKE, FAKE, None, 4, 0)
    assert st == _lib.GDN_ERR_UNSUPPORTED and "LDS" in msg
    # m = 0 launches nothing
    gdn.gdn_decode_fused(d, *pre, FAKE, FAKE, None, 0, 0)


def test_conv_argument_checks():
    d = dims()
    C = 8192
    # decode mode needs total_tokens == n
    assert _status(gdn.gdn_conv_update, d, FAKE, C, FAKE, C, FAKE, None, None, FAKE, 4, 5, 0)[0] == _lib.GDN_ERR_SHAPE
    # missing conv state pointers
    assert _status(gdn.gdn_conv_update, d, FAKE, C, FAKE, C, FAKE, None, None, None, 4, 4, 0)[0] == _lib.GDN_ERR_NULL
    # x row stride below C
    assert _status(gdn.gdn_conv_update, d, FAKE, C - 8, FAKE, C, FAKE, None, FAKE, FAKE, 2, 9, 0)[0] == \
        _lib.GDN_ERR_SHAPE
    # misaligned bias
    assert _status(gdn.gdn_conv_update, d, FAKE, C, FAKE, C, FAKE, FAKE + 2, FAKE, FAKE, 2, 9, 0)[0] == \
        _lib.GDN_ERR_ALIGN
    # bf16 x row stride of 4 elements = 8 bytes breaks the 16-byte rule
    d1 = dims(num_k_heads=1, num_v_heads=1, head_dim=32)
    assert _status(gdn.gdn_conv_update, d1, FAKE, 100, FAKE, 100, FAKE, None, FAKE, FAKE, 1, 2, 0)[0] == \
        _lib.GDN_ERR_ALIGN
    # tokens without sequences
    assert _status(gdn.gdn_conv_update, d, FAKE, C, FAKE, C, FAKE, None, FAKE, FAKE, 0, 3, 0)[0] == _lib.GDN_ERR_SHAPE
    # nothing at all is a no-op
    gdn.gdn_conv_update(d, None, 0, None, 0, None, None, None, None, 0, 0, 0)


def test_prefill_workspace_and_checks():
    d = dims()
    need = gdn.gdn_prefill_workspace_size(d, 8, 15717)
    assert need > 0
    # grows with tokens and sequences
    assert gdn.gdn_prefill_workspace_size(d, 8, 30000) > need
    assert gdn.gdn_prefill_workspace_size(d, 100, 15717) > need
    qkv = (FAKE, 8192, FAKE, 8192, FAKE, 8192, FAKE, FAKE, FAKE)
    st, msg = _status(gdn.gdn_prefill_chunked, d, *qkv, FAKE, 8, 15717, FAKE, FAKE, need - 1, 0)
    assert st == _lib.GDN_ERR_WORKSPACE and str(need) in msg
    assert _status(gdn.gdn_prefill_chunked, d, *qkv, FAKE, 8, 15717, FAKE, None, need, 0)[0] == \
        _lib.GDN_ERR_WORKSPACE
    assert _status(gdn.gdn_prefill_chunked, d, *qkv, FAKE, 8, 15717, FAKE, FAKE + 16, need, 0)[0] == \
        _lib.GDN_ERR_ALIGN
    assert _status(gdn.gdn_prefill_chunked, d, *qkv, None, 8, 15717, FAKE, FAKE, need, 0)[0] == _lib.GDN_ERR_NULL
    assert _status(gdn.gdn_prefill_chunked, d, *qkv, FAKE, 0, 5, FAKE, FAKE, need, 0)[0] == _lib.GDN_ERR_SHAPE
    # no sequences: no-op
    gdn.gdn_prefill_chunked(d, *qkv, FAKE, 0, 0, FAKE, None, 0, 0)


def test_prefill_fused_workspace_and_checks():
    """The fused prefill needs the chunked prefill's workspace plus the v part of the conv
    output, and rejects what either of the two calls would."""
    d = dims()
    pre = gdn.gdn_prefill_workspace_size(d, 8, 15717)
    need = gdn.gdn_prefill_fused_workspace_size(d, 8, 15717)
    assert need >= pre + 15717 * 32 * 128 * 4
    args = (FAKE, 8192, FAKE, None, FAKE, FAKE, FAKE, FAKE, 8, 15717, FAKE, FAKE)
    st, msg = _status(gdn.gdn_prefill_fused, d, *args, FAKE, need - 1, 0)
    assert st == _lib.GDN_ERR_WORKSPACE and str(need) in msg
    assert _status(gdn.gdn_prefill_fused, d, *args, None, need, 0)[0] == _lib.GDN_ERR_WORKSPACE
    assert _status(gdn.gdn_prefill_fused, d, *args, FAKE + 16, need, 0)[0] == _lib.GDN_ERR_ALIGN
    # x, conv_w and the pointer arrays are required; x rows must hold every channel
    no_x = (None,) + args[1:]
    assert _status(gdn.gdn_prefill_fused, d, *no_x, FAKE, need, 0)[0] == _lib.GDN_ERR_NULL
    no_cs = args[:11] + (None,)
    assert _status(gdn.gdn_prefill_fused, d, *no_cs, FAKE, need, 0)[0] == _lib.GDN_ERR_NULL
    short = (FAKE, 8000) + args[2:]
    assert _status(gdn.gdn_prefill_fused, d, *short, FAKE, need, 0)[0] == _lib.GDN_ERR_SHAPE
    odd = (FAKE, 8196) + args[2:]  # 8196 bf16 = 16392 bytes: not a multiple of 16
    assert _status(gdn.gdn_prefill_fused, d, *odd, FAKE, need, 0)[0] == _lib.GDN_ERR_ALIGN
    bad_b = args[:3] + (FAKE + 8,) + args[4:]
    assert _status(gdn.gdn_prefill_fused, d, *bad_b, FAKE, need, 0)[0] == _lib.GDN_ERR_ALIGN
    assert _status(gdn.gdn_prefill_fused, d, *args[:8], 0, 5, *args[10:], FAKE, need, 0)[0] == _lib.GDN_ERR_SHAPE
    assert _status(gdn.gdn_prefill_fused, dims(conv_width=9), *args, FAKE, need, 0)[0] == _lib.GDN_ERR_UNSUPPORTED
    # no sequences: no-op
    gdn.gdn_prefill_fused(d, *args[:8], 0, 0, None, None, None, 0, 0)


def test_prefill_form_workspace():
    """The chunk-parallel form needs room for per-segment state maps; AUTO takes it below
    256 state-row workgroups ((d / 16) * Hv * num_seqs), so its size counts the maps
    whenever a single sequence would take that form."""
    few = dict(num_k_heads=2, num_v_heads=4)  # 8 * 4 = 32 workgroups per sequence
    whole = gdn.gdn_prefill_workspace_size(dims(**few, prefill_form=_lib.GDN_PREFILL_WHOLE), 1, 4096)
    segs = gdn.gdn_prefill_workspace_size(dims(**few, prefill_form=_lib.GDN_PREFILL_SEGMENTS), 1, 4096)
    auto = gdn.gdn_prefill_workspace_size(dims(**few), 1, 4096)
    assert segs > whole and auto == segs
    # 8 sequences of 32 workgroups fill 256 CUs, so such a call walks whole sequences, but
    # the size for 8 sequences must also cover a call with one: the maps are counted
    assert gdn.gdn_prefill_workspace_size(dims(**few), 8, 4096) == \
        gdn.gdn_prefill_workspace_size(dims(**few, prefill_form=_lib.GDN_PREFILL_SEGMENTS), 8, 4096)
    # the 16/32-head layer has 256 workgroups per sequence: whole sequences
    assert gdn.gdn_prefill_workspace_size(dims(), 1, 4096) == \
        gdn.gdn_prefill_workspace_size(dims(prefill_form=_lib.GDN_PREFILL_WHOLE), 1, 4096)
    # room for the largest possible number of segments: T / (2 C) + 2 N + 1 state maps of
    # 3 x d x d fp32 per v-head
    extra = segs - whole
    assert extra >= (4096 // 128 + 3) * 4 * 3 * 128 * 128 * 4


def test_slot_pointer_checks():
    assert _status(gdn.gdn_slot_pointers, FAKE + 8, 256, 4, FAKE, 4, FAKE)[0] == _lib.GDN_ERR_ALIGN
    assert _status(gdn.gdn_slot_pointers, FAKE, 1928, 4, FAKE, 4, FAKE)[0] == _lib.GDN_ERR_ALIGN
    assert _status(gdn.gdn_slot_pointers, FAKE, 0, 4, FAKE, 4, FAKE)[0] == _lib.GDN_ERR_SHAPE
    assert _status(gdn.gdn_slot_pointers, FAKE, 256, 4, None, 4, FAKE)[0] == _lib.GDN_ERR_NULL
    gdn.gdn_slot_pointers(FAKE, 256, 4, FAKE, 0, FAKE)


def test_library_shares_torchs_hip_runtime():
    """libgdn.so receives torch's device pointers and stream handles, so exactly one HIP
    runtime (torch's) may be mapped into the process, whatever was imported first."""
    runtimes = _lib._hip_runtimes()
    assert len(runtimes) == 1, runtimes
    import torch

    assert os.path.dirname(next(iter(runtimes))) == os.path.join(os.path.dirname(torch.__file__), "lib")


def test_slot_copy_checks():
    dims = gdn.make_dims(16, 32, 128)
    # pointer arrays come in (source, destination) pairs
    assert _status(gdn.gdn_slot_copy, dims, FAKE, None, None, None, 4)[0] == _lib.GDN_ERR_NULL
    assert _status(gdn.gdn_slot_copy, dims, None, None, None, FAKE, 4)[0] == _lib.GDN_ERR_NULL
    assert _status(gdn.gdn_slot_copy, dims, FAKE, FAKE, None, None, -1)[0] == _lib.GDN_ERR_SHAPE
    bad = gdn.make_dims(16, 30, 128)  # Hv % Hk != 0
    assert _status(gdn.gdn_slot_copy, bad, FAKE, FAKE, None, None, 4)[0] == _lib.GDN_ERR_SHAPE
    gdn.gdn_slot_copy(dims, FAKE, FAKE, FAKE, FAKE, 0)  # n = 0: nothing to do, nothing launched


@pytest.mark.parametrize("form", [_lib.GDN_PREFILL_AUTO, _lib.GDN_PREFILL_WHOLE, _lib.GDN_PREFILL_SEGMENTS])
@pytest.mark.parametrize("heads", [(2, 4, 128), (16, 32, 128), (1, 1, 32), (4, 8, 64), (16, 16, 64)])
def test_workspace_size_covers_every_smaller_call(form, heads):
    """A workspace sized for (N, T) is enough for every call with N' <= N sequences and
    T' <= T tokens: the size each such call needs is at most the size for (N, T)."""
    hk, hv, d = heads
    dm = dims(num_k_heads=hk, num_v_heads=hv, head_dim=d, prefill_form=form)
    for fn in (gdn.gdn_prefill_workspace_size, gdn.gdn_prefill_fused_workspace_size):
        for N, T in [(8, 15717), (3, 4096), (64, 1000), (300, 20000)]:
            big = fn(dm, N, T)
            for n2 in sorted({1, 2, N // 2, N - 1, N}):
                for t2 in sorted({n2, T // 3, T}):
                    if n2 < 1 or t2 < n2:
                        continue
                    assert fn(dm, n2, t2) <= big, (fn.__name__, N, T, n2, t2)


def test_dims_init_fills_defaults():
    d = gdn.gdn_dims_init(16, 32, 128)
    assert (d.struct_size, d.num_k_heads, d.num_v_heads, d.head_dim) == (ctypes.sizeof(_lib.gdn_dims), 16, 32, 128)
    assert (d.conv_width, d.chunk_size, d.activation, d.in_dtype, d.mma) == (4, 64, 0, _lib.GDN_F32, 0)
    assert (d.prefill_form, d.out_dtype, d.qk_l2norm_off) == (0, _lib.GDN_F32, 0)
    assert d.scale == 1.0 and abs(d.l2_eps - 1e-6) < 1e-12
    assert gdn.gdn_prefill_workspace_size(d, 1, 64) > 0  # accepted by the entry points
    assert gdn.make_dims(16, 32, 128).qk_l2norm_off == 0
    assert gdn.make_dims(16, 32, 128, qk_l2norm=False).qk_l2norm_off == 1


_C99_PROBE = r"""
#include <stdio.h>
#include <string.h>
#include "gdn.h"
#include "gdn_probe.h"

int main(void) {
  gdn_dims z = {0};  /* zero-filled: every enumerated field at its default */
  size_t bytes = 0;
  gdn_dims d;
  z.struct_size = (int32_t)sizeof z;
  z.num_k_heads = 16;
  z.num_v_heads = 32;
  z.head_dim = 128;
  z.conv_width = 4;
  z.chunk_size = 64;
  if (z.qk_l2norm_off != 0) return 10;  /* the q/k L2 norm is on */
  /* scale has no usable zero: rejected instead of silently zeroing every output */
  if (gdn_prefill_workspace_size(&z, 1, 64, &bytes) != GDN_ERR_SHAPE) return 11;
  if (strstr(gdn_last_error(), "scale") == NULL) return 12;
  z.scale = 1.0f;
  if (gdn_prefill_workspace_size(&z, 1, 64, &bytes) != GDN_OK || bytes == 0) return 13;
  if (gdn_dims_init(&d, 16, 32, 128) != GDN_OK) return 14;
  if (d.struct_size != (int32_t)sizeof d || d.qk_l2norm_off != 0 || d.scale != 1.0f || d.conv_width != 4 ||
      d.chunk_size != 64 || d.activation != GDN_ACT_NONE || d.mma != GDN_MMA_AUTO ||
      d.prefill_form != GDN_PREFILL_AUTO || d.out_dtype != GDN_F32 || d.in_dtype != GDN_F32)
    return 15;
  if (gdn_dims_init(NULL, 1, 1, 32) != GDN_ERR_NULL) return 16;
  if (gdn_abi_version() != GDN_ABI_VERSION) return 17;
  if (gdn_hbm_probe(NULL, 16384, 0, NULL) != GDN_ERR_NULL) return 18;
  printf("c99 ok\n");
  return 0;
}
"""


def test_header_compiles_as_c99_and_zero_filled_dims_normalise(tmp_path):
    """include/gdn.h is plain C99 (no C++ in the declarations); a C caller that zero-fills
    gdn_dims gets the q/k L2 norm on, and the library's host checks behave as declared."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "probe.c"
    src.write_text(_C99_PROBE)
    exe = tmp_path / "probe"
    libdir = os.path.dirname(_lib.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{os.path.join(ROOT, 'include')}",
                        str(src), "-o", str(exe), f"-L{libdir}", "-lgdn", f"-Wl,-rpath,{libdir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c99 ok" in r.stdout, (r.returncode, r.stdout, r.stderr)


def test_hbm_probe_checks():
    assert _status(gdn.gdn_hbm_probe, None, 16384)[0] == _lib.GDN_ERR_NULL
    assert _status(gdn.gdn_hbm_probe, FAKE + 8, 16384)[0] == _lib.GDN_ERR_ALIGN
    assert _status(gdn.gdn_hbm_probe, FAKE, 16384 + 16)[0] == _lib.GDN_ERR_ALIGN
    gdn.gdn_hbm_probe(FAKE, 0)  # nothing to stream: nothing launched


def test_prefill_fused_static_limit_checked_before_any_launch():
    """The no-allocation prefill takes its workspace from the library's own 64 MiB device
    array: a call needing more is refused on the host (nothing launched), as are the
    arguments gdn_prefill_fused refuses."""
    d = dims()
    args = (FAKE, 8192, FAKE, None, FAKE, FAKE, FAKE, FAKE)  # x, x_stride, conv_w, conv_b, g, beta, o, cu
    assert gdn.gdn_prefill_fused_workspace_size(d, 8, 15717) > gdn.GDN_STATIC_SCRATCH_BYTES
    st, msg = _status(gdn.gdn_prefill_fused_static, d, *args, 8, 15717, FAKE, FAKE)
    assert st == _lib.GDN_ERR_WORKSPACE and str(gdn.GDN_STATIC_SCRATCH_BYTES) in msg
    assert gdn.gdn_prefill_fused_workspace_size(d, 1, 1024) <= gdn.GDN_STATIC_SCRATCH_BYTES
    assert _status(gdn.gdn_prefill_fused_static, dims(conv_width=9), *args, 1, 64, FAKE, FAKE)[0] == \
        _lib.GDN_ERR_UNSUPPORTED
    assert _status(gdn.gdn_prefill_fused_static, d, *args[:7], None, 1, 64, FAKE, FAKE)[0] == _lib.GDN_ERR_NULL
    gdn.gdn_prefill_fused_static(d, *args, 0, 0, None, None)  # no sequences: nothing to do
