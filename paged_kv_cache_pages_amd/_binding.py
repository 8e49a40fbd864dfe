"""ctypes binding of libpagedkv: argument marshalling only.

Every step of the decode path runs in the HIP kernels of ``libpagedkv.so``; this module checks
tensor dtypes, shapes, devices and contiguity, takes raw pointers and the current HIP stream from
PyTorch, and calls the C ABI declared in ``include/pagedkv.h``.  There is no fallback: without the
built library every call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libpagedkv.so")

PKV_OK = 0
PKV_OUT_BF16 = 0
PKV_OUT_F32 = 1
STATUS_NAMES = {
    0: "PKV_OK",
    1: "PKV_ERR_NULL",
    2: "PKV_ERR_SHAPE",
    3: "PKV_ERR_UNSUPPORTED",
    4: "PKV_ERR_WORKSPACE",
    5: "PKV_ERR_VALIDATION",
    6: "PKV_ERR_HIP",
    7: "PKV_ERR_ALIGNMENT",
    8: "PKV_ERR_REJECTED",
    9: "PKV_ERR_STATE",
    10: "PKV_ERR_EXHAUSTED",
    11: "PKV_ERR_SCRATCH",
}

# Every symbol the header declares, with its ctypes signature.
_c_int32 = ctypes.c_int32
_c_size = ctypes.c_size_t
_vp = ctypes.c_void_p


class Pool(ctypes.Structure):
    _fields_ = [
        ("k_pool", _vp),
        ("v_pool", _vp),
        ("num_pages", _c_int32),
        ("num_kv_heads", _c_int32),
        ("head_dim", _c_int32),
        ("block_size", _c_int32),
    ]


class AllocStats(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "pool_pages", "free_pages", "credits_reserved", "active", "waiting", "peak_active", "peak_assigned",
        "largest_batch", "admission_waits", "rejected")]


SIGNATURES = {
    "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_abi_version": (_c_int32, []),
    "pkv_kv_append": (ctypes.c_int, [ctypes.POINTER(Pool), _vp, _c_int32, _vp, _vp, _vp, _c_int32, _vp]),
    "pkv_paged_decode_attention": (
        ctypes.c_int,
        [_vp, _vp, _vp, _c_int32, _vp, _c_int32, _vp, _vp, ctypes.c_int, _c_int32, _c_int32, _c_int32, _c_int32,
         _c_int32, ctypes.c_float, _c_int32, _vp, _c_size, _vp],
    ),
    "pkv_rope_kv_append": (
        ctypes.c_int,
        [ctypes.POINTER(Pool), _vp, _c_int32, _vp, _vp, _vp, _c_int32, _vp, _vp, _vp, _vp, _c_int32, _c_int32, _vp],
    ),
    "pkv_decode_step": (
        ctypes.c_int,
        [ctypes.POINTER(Pool), _vp, _vp, _c_int32, _vp, _vp, _vp, _vp, ctypes.c_int, _c_int32, _c_int32,
         ctypes.c_float, _c_int32, _vp, _c_size, _vp],
    ),
    "pkv_decode_step_static": (
        ctypes.c_int,
        [ctypes.POINTER(Pool), _vp, _vp, _c_int32, _vp, _vp, _vp, _vp, ctypes.c_int, _c_int32, _c_int32,
         ctypes.c_float, _c_int32, _vp],
    ),
    "pkv_plan_partition_pages": (_c_int32, [_c_int32, _c_int32, _c_int32, _c_int32]),
    "pkv_plan_partition_pages_for_context": (_c_int32, [_c_int32, _c_int32, _c_int32, _c_int32, _c_int32]),
    "pkv_decode_workspace_bytes": (_c_size, [_c_int32, _c_int32, _c_int32, _c_int32]),
    "pkv_device_cu_count": (_c_int32, []),
    "pkv_validate_append_host": (ctypes.c_int, [_vp, _c_int32, _vp, _c_int32, _c_int32, _vp]),
    "pkv_validate_decode_host": (ctypes.c_int, [_vp, _c_int32, _vp, _c_int32, _c_int32, _vp]),
    "pkv_prefill_kv_append": (
        ctypes.c_int,
        [ctypes.POINTER(Pool), _vp, _c_int32, _vp, _vp, _vp, _vp, _c_int32, _c_int32, _c_int32, _vp],
    ),
    "pkv_paged_prefill_attention": (
        ctypes.c_int,
        [ctypes.POINTER(Pool), _vp, _vp, _c_int32, _vp, _vp, _vp, ctypes.c_int, _c_int32, _c_int32, _c_int32,
         _c_int32, ctypes.c_float, _vp],
    ),
    "pkv_validate_prefill_host": (
        ctypes.c_int, [_vp, _c_int32, _vp, _vp, _c_int32, _c_int32, _c_int32, _c_int32, _vp]),
    "pkv_validate_finite_rows_host": (ctypes.c_int, [_vp, _c_int32, _c_int32, _vp]),
    "pkv_alloc_create": (ctypes.c_int, [_c_int32, _c_int32, _c_int32, _vp, _c_int32, ctypes.POINTER(_vp)]),
    "pkv_alloc_destroy": (None, [_vp]),
    "pkv_alloc_submit": (ctypes.c_int, [_vp, ctypes.c_int64, _c_int32, _c_int32]),
    "pkv_alloc_admit": (ctypes.c_int, [_vp, _vp, _c_int32, ctypes.POINTER(_c_int32)]),
    "pkv_alloc_ensure": (ctypes.c_int, [_vp, ctypes.c_int64, _c_int32]),
    "pkv_alloc_prepare_step": (ctypes.c_int, [_vp, _vp, _vp, _c_int32, _vp, ctypes.POINTER(_c_int32)]),
    "pkv_alloc_table": (ctypes.c_int, [_vp, ctypes.c_int64, _vp]),
    "pkv_alloc_release": (ctypes.c_int, [_vp, ctypes.c_int64]),
    "pkv_alloc_get_stats": (ctypes.c_int, [_vp, ctypes.POINTER(AllocStats)]),
}

_lib = None
_lock = threading.Lock()


class PagedKVError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        name = STATUS_NAMES.get(status, str(status))
        detail = library().pkv_status_string(status).decode()
        super().__init__(f"{call} failed: {name} ({detail})")


def library() -> ctypes.CDLL:
    """The loaded libpagedkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_pages_amd._build` "
                    "(there is no CPU fallback)"
                )
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def require_library() -> None:
    library()


def _check(call: str, status: int) -> None:
    if status != PKV_OK:
        raise PagedKVError(call, status)


# ---------------------------------------------------------------------------------------------
# tensor helpers (torch is imported lazily so that host-only users need not load it)
# ---------------------------------------------------------------------------------------------

def _torch():
    import torch

    return torch


def _dev_tensor(name, t, dtype, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got shape {tuple(t.shape)})")
    return t


def _stream_handle(stream, device):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


_cu_counts = {}
_plans = {}
_workspaces = {}


def cu_count(device=None) -> int:
    """Compute units of a device (queried once per device through the library)."""
    torch = _torch()
    idx = torch.cuda.current_device() if device is None else torch.device(device).index
    n = _cu_counts.get(idx)
    if n is None:
        with torch.cuda.device(idx):
            n = int(library().pkv_device_cu_count())
        if n <= 0:
            raise RuntimeError("no HIP device available")
        _cu_counts[idx] = n
    return n


def plan_partition_pages(batch: int, num_kv_heads: int, max_blocks_per_seq: int, num_cus: int | None = None,
                         max_context: int | None = None) -> int:
    """Pages per partition; ``max_context`` (the longest context of the batch, when the caller
    knows it on the host) lets a batch whose sequences all fit one partition skip the split."""
    mc = -1 if max_context is None else int(max_context)
    key = (batch, num_kv_heads, max_blocks_per_seq, num_cus, mc)
    r = _plans.get(key)
    if r is None:
        cus = cu_count() if num_cus is None else int(num_cus)
        r = int(library().pkv_plan_partition_pages_for_context(batch, num_kv_heads, max_blocks_per_seq, mc, cus))
        if r <= 0:
            raise ValueError("invalid planning arguments")
        if num_cus is not None:
            _plans[key] = r
    return r


def decode_workspace_bytes(batch: int, num_q_heads: int, max_blocks_per_seq: int, partition_pages: int) -> int:
    return int(library().pkv_decode_workspace_bytes(batch, num_q_heads, max_blocks_per_seq, partition_pages))


def _cached_workspace(nbytes: int, device, stream):
    """A zero-filled workspace tensor kept per (device, stream) and grown on demand (at least
    doubling, so a stream holds at most about twice its largest request); every call leaves its
    counters at zero again.  Calls on one stream are ordered, so
    reusing its workspace is safe; other streams get their own.  A workspace that a larger one
    replaces is retired, not freed: a HIP graph captured with it may still be replayed.  Cached and
    retired workspaces live until ``release_cached_workspaces()``."""
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    key = (device.index, s.cuda_stream)
    with _lock:
        ws = _workspaces.get(key)
        if ws is None or ws.numel() < nbytes:
            size = max(nbytes, 1 << 16, 2 * ws.numel() if ws is not None else 0)
            with torch.cuda.stream(s):
                new = torch.zeros(size, dtype=torch.uint8, device=device)
            if ws is not None:
                _retired_workspaces.append(ws)
            _workspaces[key] = ws = new
    return ws


_retired_workspaces = []


def release_cached_workspaces() -> int:
    """Free the workspaces the calls without an explicit ``workspace`` cached (per device and
    stream), after waiting for the device.  The caller guarantees that no HIP graph captured with
    one of them is replayed afterwards.  Returns the bytes released."""
    torch = _torch()
    with _lock:
        held = list(_workspaces.values()) + _retired_workspaces
        freed = sum(int(t.numel()) for t in held)
        _workspaces.clear()
        _retired_workspaces.clear()
    if held and torch.cuda.is_available():
        torch.cuda.synchronize()
    del held
    return freed


# ---------------------------------------------------------------------------------------------
# the two method calls
# ---------------------------------------------------------------------------------------------

def kv_append(k_pool, v_pool, block_tables, positions, k_new, v_new, stream=None) -> None:
    """Write k_new/v_new [B][Hkv][D] into slot pos % 16 of page block_tables[b][pos // 16]."""
    torch = _torch()
    _dev_tensor("k_pool", k_pool, torch.bfloat16, 4)
    _dev_tensor("v_pool", v_pool, torch.bfloat16, 4)
    _dev_tensor("block_tables", block_tables, torch.int32, 2)
    _dev_tensor("positions", positions, torch.int32, 1)
    _dev_tensor("k_new", k_new, torch.bfloat16, 3)
    _dev_tensor("v_new", v_new, torch.bfloat16, 3)
    num_pages, hkv, block, dim = k_pool.shape
    if tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_pool and v_pool shapes differ")
    batch = positions.shape[0]
    if block_tables.shape[0] != batch or tuple(k_new.shape) != (batch, hkv, dim) or k_new.shape != v_new.shape:
        raise ValueError("inconsistent batch / head shapes")
    pool = Pool(k_pool.data_ptr(), v_pool.data_ptr(), num_pages, hkv, dim, block)
    st = library().pkv_kv_append(
        ctypes.byref(pool), block_tables.data_ptr(), block_tables.shape[1], positions.data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), batch, _stream_handle(stream, k_pool.device),
    )
    _check("pkv_kv_append", st)


def rope_kv_append(k_pool, v_pool, block_tables, positions, q, k_new, v_new, cos_table, sin_table, q_out=None,
                   stream=None):
    """Rotate q and k_new at each sequence's position (tables [rows][64] float32), write the
    rotated key and v_new into the pool; returns the rotated q (``q_out``, which may be ``q``)."""
    torch = _torch()
    _dev_tensor("k_pool", k_pool, torch.bfloat16, 4)
    _dev_tensor("v_pool", v_pool, torch.bfloat16, 4)
    _dev_tensor("block_tables", block_tables, torch.int32, 2)
    _dev_tensor("positions", positions, torch.int32, 1)
    _dev_tensor("q", q, torch.bfloat16, 3)
    _dev_tensor("k_new", k_new, torch.bfloat16, 3)
    _dev_tensor("v_new", v_new, torch.bfloat16, 3)
    _dev_tensor("cos_table", cos_table, torch.float32, 2)
    _dev_tensor("sin_table", sin_table, torch.float32, 2)
    if q_out is None:
        q_out = torch.empty_like(q)
    _dev_tensor("q_out", q_out, torch.bfloat16, 3)
    num_pages, hkv, block, dim = k_pool.shape
    batch, hq, _ = q.shape
    if tuple(v_pool.shape) != tuple(k_pool.shape) or tuple(q_out.shape) != tuple(q.shape):
        raise ValueError("inconsistent pool / q shapes")
    if positions.shape[0] != batch or block_tables.shape[0] != batch or tuple(k_new.shape) != (batch, hkv, dim) \
            or k_new.shape != v_new.shape:
        raise ValueError("inconsistent batch / head shapes")
    if tuple(cos_table.shape) != tuple(sin_table.shape) or cos_table.shape[1] != dim:
        raise ValueError("cos/sin tables must both be [rows][head_dim]")
    pool = Pool(k_pool.data_ptr(), v_pool.data_ptr(), num_pages, hkv, dim, block)
    st = library().pkv_rope_kv_append(
        ctypes.byref(pool), block_tables.data_ptr(), block_tables.shape[1], positions.data_ptr(), q.data_ptr(),
        q_out.data_ptr(), hq, k_new.data_ptr(), v_new.data_ptr(), cos_table.data_ptr(), sin_table.data_ptr(),
        cos_table.shape[0], batch, _stream_handle(stream, k_pool.device),
    )
    _check("pkv_rope_kv_append", st)
    return q_out


def paged_decode_attention(q, k_pool, v_pool, block_tables, context_lens, out=None, *, out_dtype=None, scale=None,
                           partition_pages: int = 0, max_context: int | None = None, workspace=None, stream=None):
    """Decode attention of q [B][Hq][D] over each sequence's pages; returns out [B][Hq][D].

    ``out_dtype`` is torch.bfloat16 (default) or torch.float32; ``scale`` defaults to
    1/sqrt(head_dim).  ``partition_pages`` <= 0 lets the library plan the context split (with
    ``max_context``, the longest context if the caller knows it, a batch that fits one partition
    is not split); when no workspace is passed, a torch buffer cached per (device, stream) is used
    (it stays allocated until ``release_cached_workspaces()``, so a HIP graph captured with it
    stays valid until then; passing an explicit workspace keeps its lifetime in the caller's hands).
    """
    torch = _torch()
    _dev_tensor("q", q, torch.bfloat16, 3)
    _dev_tensor("k_pool", k_pool, torch.bfloat16, 4)
    _dev_tensor("v_pool", v_pool, torch.bfloat16, 4)
    _dev_tensor("block_tables", block_tables, torch.int32, 2)
    _dev_tensor("context_lens", context_lens, torch.int32, 1)
    batch, hq, dim = q.shape
    num_pages, hkv, block, _ = k_pool.shape
    if tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_pool and v_pool shapes differ")
    if block_tables.shape[0] != batch or context_lens.shape[0] != batch:
        raise ValueError("block_tables / context_lens batch differs from q")
    max_blocks = block_tables.shape[1]
    if out is None:
        out = torch.empty((batch, hq, dim), dtype=out_dtype or torch.bfloat16, device=q.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _dev_tensor("out", out, out.dtype, 3)
    if tuple(out.shape) != (batch, hq, dim):
        raise ValueError("out shape differs from q")
    if scale is None:
        scale = 1.0 / float(dim) ** 0.5
    pp = int(partition_pages)
    if pp <= 0:
        pp = plan_partition_pages(batch, hkv, max_blocks, cu_count(q.device), max_context)
    need = decode_workspace_bytes(batch, hq, max_blocks, pp)
    sh = _stream_handle(stream, q.device)
    ws_ptr, ws_bytes = None, 0
    if need > 0:
        if workspace is None:
            workspace = _cached_workspace(need, q.device, stream)
        _dev_tensor("workspace", workspace, workspace.dtype)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = library().pkv_paged_decode_attention(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), num_pages, block_tables.data_ptr(), max_blocks,
        context_lens.data_ptr(), out.data_ptr(), PKV_OUT_BF16 if out.dtype == torch.bfloat16 else PKV_OUT_F32,
        batch, hq, hkv, dim, block, float(scale), pp, ws_ptr, ws_bytes, sh,
    )
    _check("pkv_paged_decode_attention", st)
    return out


def decode_step(q, k_pool, v_pool, block_tables, positions, k_new, v_new, out=None, *, out_dtype=None, scale=None,
                partition_pages: int = 0, max_context: int | None = None, workspace=None, stream=None):
    """kv_append then decode attention over positions + 1 tokens, in one launch; returns out.
    Partition planning and the workspace work as in ``paged_decode_attention``."""
    torch = _torch()
    _dev_tensor("q", q, torch.bfloat16, 3)
    _dev_tensor("k_pool", k_pool, torch.bfloat16, 4)
    _dev_tensor("v_pool", v_pool, torch.bfloat16, 4)
    _dev_tensor("block_tables", block_tables, torch.int32, 2)
    _dev_tensor("positions", positions, torch.int32, 1)
    _dev_tensor("k_new", k_new, torch.bfloat16, 3)
    _dev_tensor("v_new", v_new, torch.bfloat16, 3)
    batch, hq, dim = q.shape
    num_pages, hkv, block, _ = k_pool.shape
    if tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_pool and v_pool shapes differ")
    if block_tables.shape[0] != batch or positions.shape[0] != batch:
        raise ValueError("block_tables / positions batch differs from q")
    if tuple(k_new.shape) != (batch, hkv, dim) or k_new.shape != v_new.shape:
        raise ValueError("k_new / v_new must be [batch][kv_heads][head_dim]")
    max_blocks = block_tables.shape[1]
    if out is None:
        out = torch.empty((batch, hq, dim), dtype=out_dtype or torch.bfloat16, device=q.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _dev_tensor("out", out, out.dtype, 3)
    if tuple(out.shape) != (batch, hq, dim):
        raise ValueError("out shape differs from q")
    if scale is None:
        scale = 1.0 / float(dim) ** 0.5
    pp = int(partition_pages)
    if pp <= 0:
        pp = plan_partition_pages(batch, hkv, max_blocks, cu_count(q.device), max_context)
    need = decode_workspace_bytes(batch, hq, max_blocks, pp)
    sh = _stream_handle(stream, q.device)
    ws_ptr, ws_bytes = None, 0
    if need > 0:
        if workspace is None:
            workspace = _cached_workspace(need, q.device, stream)
        _dev_tensor("workspace", workspace, workspace.dtype)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    pool = Pool(k_pool.data_ptr(), v_pool.data_ptr(), num_pages, hkv, dim, block)
    st = library().pkv_decode_step(
        ctypes.byref(pool), q.data_ptr(), block_tables.data_ptr(), max_blocks, positions.data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), out.data_ptr(), PKV_OUT_BF16 if out.dtype == torch.bfloat16 else PKV_OUT_F32, batch, hq,
        float(scale), pp, ws_ptr, ws_bytes, sh,
    )
    _check("pkv_decode_step", st)
    return out


STATIC_SCRATCH_BYTES = 4 << 20  # PKV_STATIC_SCRATCH_BYTES


def decode_step_static(q, k_pool, v_pool, block_tables, positions, k_new, v_new, out, *, scale=None,
                       partition_pages: int = 0, max_context: int | None = None, stream=None):
    """pkv_decode_step_static: decode_step without a workspace; a split uses the library's static
    per-GPU scratch (PKV_STATIC_SCRATCH_BYTES), so the call allocates no device memory.  ``out``
    must be given (bfloat16 or float32 [B][Hq][D]).  Calls that may overlap on one GPU race."""
    torch = _torch()
    _dev_tensor("q", q, torch.bfloat16, 3)
    _dev_tensor("k_pool", k_pool, torch.bfloat16, 4)
    _dev_tensor("v_pool", v_pool, torch.bfloat16, 4)
    _dev_tensor("block_tables", block_tables, torch.int32, 2)
    _dev_tensor("positions", positions, torch.int32, 1)
    _dev_tensor("k_new", k_new, torch.bfloat16, 3)
    _dev_tensor("v_new", v_new, torch.bfloat16, 3)
    if not isinstance(out, torch.Tensor) or out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be a bfloat16 or float32 tensor")
    _dev_tensor("out", out, out.dtype, 3)
    batch, hq, dim = q.shape
    num_pages, hkv, block, _ = k_pool.shape
    if tuple(v_pool.shape) != tuple(k_pool.shape) or tuple(out.shape) != (batch, hq, dim):
        raise ValueError("inconsistent pool / out shapes")
    if block_tables.shape[0] != batch or positions.shape[0] != batch:
        raise ValueError("block_tables / positions batch differs from q")
    if tuple(k_new.shape) != (batch, hkv, dim) or k_new.shape != v_new.shape:
        raise ValueError("k_new / v_new must be [batch][kv_heads][head_dim]")
    max_blocks = block_tables.shape[1]
    scale = 1.0 / float(dim) ** 0.5 if scale is None else float(scale)
    pp = int(partition_pages)
    if pp <= 0:
        pp = plan_partition_pages(batch, hkv, max_blocks, cu_count(q.device), max_context)
    pool = Pool(k_pool.data_ptr(), v_pool.data_ptr(), num_pages, hkv, dim, block)
    st = library().pkv_decode_step_static(
        ctypes.byref(pool), q.data_ptr(), block_tables.data_ptr(), max_blocks, positions.data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), out.data_ptr(), PKV_OUT_BF16 if out.dtype == torch.bfloat16 else PKV_OUT_F32, batch, hq,
        scale, pp, _stream_handle(stream, q.device),
    )
    _check("pkv_decode_step_static", st)
    return out


class PreparedDecodeStep:
    """pkv_decode_step on fixed buffers, for loops that reuse the same tensors and update their
    contents in place.  Shapes, dtypes, the partition plan, the workspace and the stream are
    checked and chosen once (as decode_step does on every call); each call then passes the cached
    arguments straight to the library, on ``stream`` if one was given, else on the stream current
    at the call (so the step can be captured into a graph).  The tensors are kept alive by this
    object; their contents (q, block_tables, positions, k_new, v_new, the pools) are read at
    launch time.  A workspace it allocates itself is recorded on every stream it launches on."""

    def __init__(self, q, k_pool, v_pool, block_tables, positions, k_new, v_new, out, *, scale=None,
                 partition_pages: int = 0, max_context: int | None = None, workspace=None, stream=None):
        torch = _torch()
        _dev_tensor("q", q, torch.bfloat16, 3)
        _dev_tensor("k_pool", k_pool, torch.bfloat16, 4)
        _dev_tensor("v_pool", v_pool, torch.bfloat16, 4)
        _dev_tensor("block_tables", block_tables, torch.int32, 2)
        _dev_tensor("positions", positions, torch.int32, 1)
        _dev_tensor("k_new", k_new, torch.bfloat16, 3)
        _dev_tensor("v_new", v_new, torch.bfloat16, 3)
        if not isinstance(out, torch.Tensor) or out.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("out must be a bfloat16 or float32 tensor")
        _dev_tensor("out", out, out.dtype, 3)
        batch, hq, dim = q.shape
        num_pages, hkv, block, _ = k_pool.shape
        if tuple(v_pool.shape) != tuple(k_pool.shape) or tuple(out.shape) != (batch, hq, dim):
            raise ValueError("inconsistent pool / out shapes")
        if block_tables.shape[0] != batch or positions.shape[0] != batch:
            raise ValueError("block_tables / positions batch differs from q")
        if tuple(k_new.shape) != (batch, hkv, dim) or k_new.shape != v_new.shape:
            raise ValueError("k_new / v_new must be [batch][kv_heads][head_dim]")
        max_blocks = block_tables.shape[1]
        scale = 1.0 / float(dim) ** 0.5 if scale is None else float(scale)
        pp = int(partition_pages)
        if pp <= 0:
            pp = plan_partition_pages(batch, hkv, max_blocks, cu_count(q.device), max_context)
        need = decode_workspace_bytes(batch, hq, max_blocks, pp)
        ws_ptr, ws_bytes = None, 0
        self._own_ws = None
        if need > 0:
            if workspace is None:
                workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
                # allocated on the stream current now; launches on any other stream are recorded
                # on it, so torch does not hand the memory out again while they may still run
                self._own_ws = (workspace, {torch.cuda.current_stream(q.device).cuda_stream})
            _dev_tensor("workspace", workspace, workspace.dtype)
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
            if ws_bytes < need:
                raise ValueError(f"workspace holds {ws_bytes} bytes, {need} needed")
        self.out = out
        self.partition_pages = pp
        self._keep = (q, k_pool, v_pool, block_tables, positions, k_new, v_new, out, workspace)
        self._pool = Pool(k_pool.data_ptr(), v_pool.data_ptr(), num_pages, hkv, dim, block)
        self._fn = library().pkv_decode_step
        self._args = (
            ctypes.byref(self._pool), q.data_ptr(), block_tables.data_ptr(), max_blocks, positions.data_ptr(),
            k_new.data_ptr(), v_new.data_ptr(), out.data_ptr(),
            PKV_OUT_BF16 if out.dtype == torch.bfloat16 else PKV_OUT_F32, batch, hq, scale, pp, ws_ptr, ws_bytes,
        )
        self._stream = None if stream is None else _stream_handle(stream, q.device)
        self._device = q.device
        # torch's raw current-stream query is ~10x cheaper per call than current_stream()
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        index = q.device.index
        self._current = (lambda: raw(index)) if raw is not None else (
            lambda: torch.cuda.current_stream(self._device).cuda_stream)

    def __call__(self):
        sh = self._stream if self._stream is not None else self._current()
        if self._own_ws is not None and sh not in self._own_ws[1]:
            torch = _torch()
            self._own_ws[0].record_stream(torch.cuda.ExternalStream(sh, device=self._device))
            self._own_ws[1].add(sh)
        st = self._fn(*self._args, sh)
        if st != PKV_OK:
            raise PagedKVError("pkv_decode_step", st)
        return self.out


def _prefill_args(k_pool, v_pool, block_tables, cu_seqlens, start_pos, max_prompt_len):
    torch = _torch()
    _dev_tensor("k_pool", k_pool, torch.bfloat16, 4)
    _dev_tensor("v_pool", v_pool, torch.bfloat16, 4)
    _dev_tensor("block_tables", block_tables, torch.int32, 2)
    _dev_tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    _dev_tensor("start_pos", start_pos, torch.int32, 1)
    if tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_pool and v_pool shapes differ")
    batch = start_pos.shape[0]
    if cu_seqlens.shape[0] != batch + 1 or block_tables.shape[0] != batch:
        raise ValueError("cu_seqlens must hold batch + 1 entries and block_tables batch rows")
    if max_prompt_len is None:  # convenience only: reads the lengths back to the host
        max_prompt_len = int(torch.diff(cu_seqlens).max().item()) if batch else 0
    num_pages, hkv, block, dim = k_pool.shape
    pool = Pool(k_pool.data_ptr(), v_pool.data_ptr(), num_pages, hkv, dim, block)
    return pool, batch, int(max_prompt_len)


def prefill_kv_append(k_pool, v_pool, block_tables, cu_seqlens, start_pos, k_new, v_new, *, max_prompt_len=None,
                      stream=None) -> None:
    """Write the packed prompt rows k_new/v_new [N][Hkv][D] of every sequence at positions
    start_pos[b] + i through its block table.  ``max_prompt_len`` (a bound on every prompt
    length) is read back from ``cu_seqlens`` when omitted."""
    torch = _torch()
    pool, batch, mpl = _prefill_args(k_pool, v_pool, block_tables, cu_seqlens, start_pos, max_prompt_len)
    _dev_tensor("k_new", k_new, torch.bfloat16, 3)
    _dev_tensor("v_new", v_new, torch.bfloat16, 3)
    if k_new.shape != v_new.shape or k_new.shape[1:] != k_pool.shape[1:2] + k_pool.shape[3:]:
        raise ValueError("k_new / v_new must be [N][num_kv_heads][head_dim]")
    st = library().pkv_prefill_kv_append(
        ctypes.byref(pool), block_tables.data_ptr(), block_tables.shape[1], cu_seqlens.data_ptr(),
        start_pos.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), batch, k_new.shape[0], mpl,
        _stream_handle(stream, k_pool.device),
    )
    _check("pkv_prefill_kv_append", st)


def paged_prefill_attention(q, k_pool, v_pool, block_tables, cu_seqlens, start_pos, out=None, *, max_prompt_len=None,
                            out_dtype=None, scale=None, stream=None):
    """Causal attention of the packed prompt rows q [N][Hq][D] over their sequences' pages
    (positions 0 .. start + i for row i); returns out [N][Hq][D] (bfloat16 by default)."""
    torch = _torch()
    pool, batch, mpl = _prefill_args(k_pool, v_pool, block_tables, cu_seqlens, start_pos, max_prompt_len)
    _dev_tensor("q", q, torch.bfloat16, 3)
    tokens, hq, dim = q.shape
    if out is None:
        out = torch.empty((tokens, hq, dim), dtype=out_dtype or torch.bfloat16, device=q.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _dev_tensor("out", out, out.dtype, 3)
    if tuple(out.shape) != (tokens, hq, dim):
        raise ValueError("out shape differs from q")
    if scale is None:
        scale = 1.0 / float(dim) ** 0.5
    st = library().pkv_paged_prefill_attention(
        ctypes.byref(pool), q.data_ptr(), block_tables.data_ptr(), block_tables.shape[1], cu_seqlens.data_ptr(),
        start_pos.data_ptr(), out.data_ptr(), PKV_OUT_BF16 if out.dtype == torch.bfloat16 else PKV_OUT_F32, batch,
        tokens, mpl, hq, float(scale), _stream_handle(stream, q.device),
    )
    _check("pkv_paged_prefill_attention", st)
    return out


def validate_prefill_host(block_tables, cu_seqlens, start_pos, num_tokens: int, max_prompt_len: int, num_pages: int):
    """Host-side prefill validation on numpy int32 arrays: (status, bad_sequence)."""
    import numpy as np

    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    sp = np.ascontiguousarray(start_pos, dtype=np.int32)
    bad = ctypes.c_int32(-2)
    st = library().pkv_validate_prefill_host(
        bt.ctypes.data, bt.shape[1] if bt.ndim == 2 else 0, cu.ctypes.data, sp.ctypes.data, sp.shape[0], num_tokens,
        max_prompt_len, num_pages, ctypes.byref(bad),
    )
    return int(st), int(bad.value)


def validate_finite_rows_host(rows):
    """Host-side finiteness check of BF16 bit patterns (numpy uint16, first axis = rows):
    (status, first bad row)."""
    import numpy as np

    a = np.ascontiguousarray(rows, dtype=np.uint16)
    n = a.shape[0] if a.ndim else 0
    elems = int(np.prod(a.shape[1:])) if a.ndim > 1 else 1
    bad = ctypes.c_int32(-2)
    st = library().pkv_validate_finite_rows_host(a.ctypes.data, n, elems, ctypes.byref(bad))
    return int(st), int(bad.value)


def validate_append_host(block_tables, positions, num_pages: int):
    """Host-side append validation on numpy int32 arrays: (status, bad_row)."""
    import numpy as np

    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    bad = ctypes.c_int32(-2)
    st = library().pkv_validate_append_host(
        bt.ctypes.data, bt.shape[1] if bt.ndim == 2 else 0, pos.ctypes.data, pos.shape[0], num_pages, ctypes.byref(bad)
    )
    return int(st), int(bad.value)


def validate_decode_host(block_tables, context_lens, num_pages: int):
    """Host-side decode validation on numpy int32 arrays: (status, bad_row)."""
    import numpy as np

    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    bad = ctypes.c_int32(-2)
    st = library().pkv_validate_decode_host(
        bt.ctypes.data, bt.shape[1] if bt.ndim == 2 else 0, lens.ctypes.data, lens.shape[0], num_pages, ctypes.byref(bad)
    )
    return int(st), int(bad.value)


class PageAllocator:
    """Host page allocator with admission credits (the ``pkv_alloc_*`` calls of the C ABI).

    Methods return the C status (``submit``, ``ensure``, ``release``) or raise ``PagedKVError``
    on argument errors; tables come back as numpy int32 arrays."""

    def __init__(self, num_pages: int, layers: int, max_blocks: int, free_order=None, static: bool = False):
        import numpy as np

        self.layers, self.max_blocks = int(layers), int(max_blocks)
        self._order = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        if self._order is not None and self._order.shape != (num_pages,):
            raise ValueError("free_order must hold num_pages entries")
        handle = _vp()
        st = library().pkv_alloc_create(num_pages, layers, max_blocks,
                                        None if self._order is None else self._order.ctypes.data, int(bool(static)),
                                        ctypes.byref(handle))
        _check("pkv_alloc_create", st)
        self._h = handle

    def close(self) -> None:
        if getattr(self, "_h", None):
            library().pkv_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def submit(self, request_id: int, prompt_tokens: int, max_new_tokens: int) -> int:
        return int(library().pkv_alloc_submit(self._h, request_id, prompt_tokens, max_new_tokens))

    def admit(self, capacity: int = 1 << 20) -> list:
        import numpy as np

        ids = np.zeros(max(capacity, 1), dtype=np.int64)
        n = ctypes.c_int32(0)
        _check("pkv_alloc_admit", library().pkv_alloc_admit(self._h, ids.ctypes.data, capacity, ctypes.byref(n)))
        return [int(x) for x in ids[: n.value]]

    def ensure(self, request_id: int, pos: int) -> int:
        return int(library().pkv_alloc_ensure(self._h, request_id, pos))

    def prepare_step(self, request_ids, positions, out=None):
        """(status, bad_row, tables int32[layers][batch][max_blocks])."""
        import numpy as np

        ids = np.ascontiguousarray(request_ids, dtype=np.int64)
        pos = np.ascontiguousarray(positions, dtype=np.int32)
        if ids.shape != pos.shape or ids.ndim != 1:
            raise ValueError("request_ids and positions must be 1-D of one length")
        shape = (self.layers, ids.shape[0], self.max_blocks)
        if out is None:
            out = np.empty(shape, dtype=np.int32)
        elif out.shape != shape or out.dtype != np.int32 or not out.flags.c_contiguous:
            raise ValueError(f"out must be a contiguous int32 array of shape {shape}")
        bad = ctypes.c_int32(-2)
        st = library().pkv_alloc_prepare_step(self._h, ids.ctypes.data, pos.ctypes.data, ids.shape[0],
                                              out.ctypes.data, ctypes.byref(bad))
        return int(st), int(bad.value), out

    def table(self, request_id: int):
        import numpy as np

        out = np.empty((self.layers, self.max_blocks), dtype=np.int32)
        _check("pkv_alloc_table", library().pkv_alloc_table(self._h, request_id, out.ctypes.data))
        return out

    def release(self, request_id: int) -> int:
        return int(library().pkv_alloc_release(self._h, request_id))

    def stats(self) -> dict:
        st = AllocStats()
        _check("pkv_alloc_get_stats", library().pkv_alloc_get_stats(self._h, ctypes.byref(st)))
        return {name: int(getattr(st, name)) for name, _ in AllocStats._fields_}
