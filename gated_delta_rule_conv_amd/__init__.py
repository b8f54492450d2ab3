"""MI355X (gfx950) Gated DeltaNet layer core: depthwise causal conv with per-sequence
conv state, L2-normalised q/k, and the gated delta rule as chunked prefill over packed
ragged sequences and as batched single-token decode over slot-pool pointers.

The compute lives in libgdn.so (hand-written HIP kernels behind a C ABI, declared in
include/gdn.h); this package is the thin Python binding over it.
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    GDN_ACT_NONE,
    GDN_ACT_SILU,
    GDN_BF16,
    GDN_F32,
    GDN_MMA_AUTO,
    GDN_MMA_BF16X3,
    GDN_MMA_FP32,
    GDN_PREFILL_AUTO,
    GDN_PREFILL_SEGMENTS,
    GDN_PREFILL_WHOLE,
    GDNError,
    LIB_PATH,
    gdn_abi_version,
    gdn_conv_update,
    gdn_decode_batched,
    gdn_decode_fused,
    gdn_dims,
    gdn_dims_init,
    gdn_hbm_probe,
    gdn_last_error,
    gdn_prefill_chunked,
    gdn_prefill_fused,
    gdn_prefill_fused_static,
    GDN_STATIC_SCRATCH_BYTES,
    gdn_prefill_fused_workspace_size,
    gdn_prefill_workspace_size,
    gdn_slot_copy,
    gdn_slot_pointers,
    make_dims,
)
from .layer import (  # noqa: F401
    SlotPool,
    channels,
    conv_update,
    decode,
    decode_fused,
    prefill,
    prefill_fused,
    prefill_fused_workspace,
    prefill_workspace,
    qkv_views,
)
