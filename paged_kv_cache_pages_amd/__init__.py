"""Paged KV cache decode step for AMD Instinct MI355X (gfx950).

``kv_append`` and ``paged_decode_attention`` are thin bindings of the C ABI in
``include/pagedkv.h``; the work runs in hand-written HIP kernels (``csrc/``).  ``PageAllocator``
binds the host page allocator (C++) that fills the block tables.  PyTorch supplies
device memory and the current stream only.
"""

from ._binding import (  # noqa: F401
    LIB_PATH,
    PKV_OUT_BF16,
    PKV_OUT_F32,
    AllocStats,
    PageAllocator,
    STATIC_SCRATCH_BYTES,
    SIGNATURES,
    STATUS_NAMES,
    PagedKVError,
    Pool,
    PreparedDecodeStep,
    cu_count,
    decode_step,
    decode_step_static,
    decode_workspace_bytes,
    kv_append,
    library,
    paged_decode_attention,
    paged_prefill_attention,
    plan_partition_pages,
    prefill_kv_append,
    release_cached_workspaces,
    require_library,
    rope_kv_append,
    validate_append_host,
    validate_decode_host,
    validate_finite_rows_host,
    validate_prefill_host,
)
