"""FlashAttention-2 style exact-attention forward for AMD MI355X (gfx950).

The computation runs entirely in the HIP kernels of ``libfa2.so`` behind the
C ABI of ``include/fa2.h``; this package only marshals torch tensors (device
memory and the current stream) into those calls.  There is no CPU fallback:
if the library is missing or a GPU is absent the calls raise.
"""
from ._binding import (  # noqa: F401
    FA2_MAX_SPLITS,
    Fa2Error,
    attention,
    backward,
    bwd_workspace_bytes,
    config_name,
    default_config,
    decode_fp8,
    forward,
    forward_blocksparse,
    MASK_BLOCK_K,
    MASK_BLOCK_Q,
    forward_config,
    forward_fp8,
    forward_splitkv,
    forward_splitkv_noalloc,
    NOALLOC_SCRATCH_BYTES,
    forward_window,
    fp8_vt_stride,
    lib_path,
    library_at,
    load_library,
    open_library,
    poison_lib_path,
    num_configs,
    num_splits,
    probe_xcc,
    quantize_fp8,
    splitkv_workspace_bytes,
    status_string,
)
