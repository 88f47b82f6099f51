"""ctypes binding of libpkv.so (include/pkv.h).

Argument marshalling only: tensors are checked for dtype, device and layout, their device
pointers and PyTorch's current HIP stream are passed through, and non-zero return codes become
``PkvError``.  Every step of the computation runs in the library's HIP kernels; there is no other
code path.  PyTorch supplies device memory and the stream.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ELAUNCH, PKV_EWORKSPACE = 0, -1, -2, -3, -4
PKV_F32, PKV_BF16, PKV_F16 = 0, 1, 2
ERROR_NAMES = {PKV_EINVAL: "PKV_EINVAL", PKV_EUNSUPPORTED: "PKV_EUNSUPPORTED",
               PKV_ELAUNCH: "PKV_ELAUNCH", PKV_EWORKSPACE: "PKV_EWORKSPACE"}

# Device-side metadata status bits (pkv_validate_metadata).
STATUS_PAGE_RANGE, STATUS_CAPACITY, STATUS_APPEND_ALIAS = 1, 2, 4


class PkvError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code


class PkvShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_SIGNATURES = {
    "pkv_paged_decode_attention": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                                  ctypes.POINTER(PkvShape), _vp]),
    "pkv_paged_decode_attention_partial": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                                                          _i32, _vp, _vp, _i32,
                                                          ctypes.POINTER(PkvShape), _vp]),
    "pkv_lse_merge": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _vp, _vp,
                                     ctypes.POINTER(PkvShape), _vp]),
    "pkv_paged_kv_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp,
                                           ctypes.POINTER(PkvShape), _vp]),
    "pkv_validate_metadata": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp,
                                             ctypes.POINTER(PkvShape), _vp]),
    "pkv_paged_decode_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                                             _vp, ctypes.c_size_t, _vp, _vp,
                                             ctypes.POINTER(PkvShape), _vp]),
    "pkv_paged_decode_step_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                     ctypes.c_float, _vp, _vp,
                                                     ctypes.POINTER(PkvShape), _vp]),
    "pkv_paged_decode_cascade": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, ctypes.c_float,
                                                _i32, _vp, _vp, _i32, _vp, _vp,
                                                ctypes.POINTER(PkvShape), _vp]),
    "pkv_rope_kv_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                                          ctypes.POINTER(PkvShape), _vp]),
    "pkv_paged_decode_step_rope": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                                  ctypes.c_float, _vp, ctypes.c_size_t, _vp, _vp,
                                                  ctypes.POINTER(PkvShape), _vp]),
    "pkv_paged_decode_multi_query": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, ctypes.c_float,
                                                    _i32, _vp, _vp, _i32, _vp, _vp,
                                                    ctypes.POINTER(PkvShape), _vp]),
    "pkv_paged_decode_multi_query_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, ctypes.c_float,
                                                         _vp, ctypes.c_size_t, _vp, _vp,
                                                         ctypes.POINTER(PkvShape), _vp]),
    "pkv_multi_query_step_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(PkvShape), _i32]),
    "pkv_copy_pages": (ctypes.c_int, [_vp, _vp, _vp, _i32, ctypes.POINTER(PkvShape), _vp]),
    "pkv_read_stream": (ctypes.c_int, [_vp, ctypes.c_size_t, _vp, _vp]),
    "pkv_pages_create": (_vp, [_i32, _i32]),
    "pkv_pages_destroy": (None, [_vp]),
    "pkv_pages_free_count": (_i32, [_vp]),
    "pkv_pages_refcount": (_i32, [_vp, _i32]),
    "pkv_pages_seq_create": (ctypes.c_int, [_vp, ctypes.POINTER(_i32)]),
    "pkv_pages_seq_fork": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_i32)]),
    "pkv_pages_seq_release": (ctypes.c_int, [_vp, _i32]),
    "pkv_pages_seq_reserve": (ctypes.c_int, [_vp, _i32, _i32, ctypes.POINTER(_i32), _i32,
                                             ctypes.POINTER(_i32)]),
    "pkv_pages_seq_length": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_i32)]),
    "pkv_pages_seq_table": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_i32), _i32,
                                           ctypes.POINTER(_i32)]),
    "pkv_pages_prefix_insert": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_i32), _i32]),
    "pkv_pages_seq_create_with_prefix": (ctypes.c_int, [_vp, ctypes.POINTER(_i32), _i32,
                                                        ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "pkv_pages_prefix_evict": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_i32)]),
    "pkv_pages_last_error": (ctypes.c_char_p, []),
    "pkv_decode_step_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(PkvShape)]),
    "pkv_partial_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(PkvShape), _i32]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python paged_kv_cache_203_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def version() -> str:
    return lib.pkv_version().decode()


def last_error() -> str:
    return lib.pkv_last_error().decode()


def _check(rc: int) -> None:
    if rc != PKV_OK:
        raise PkvError(rc, last_error())


# ----------------------------------------------------------------------------------------------
# tensor marshalling
# ----------------------------------------------------------------------------------------------

def _torch():
    import torch  # deferred: the CPU-side ABI checks do not need it
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16, torch.float16: PKV_F16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported element type {t.dtype}")
    return codes[t.dtype]


def _require(t, name, dtype=None, ndim=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")


def _stream(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def make_shape(batch, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
               max_pages_per_seq, dtype) -> PkvShape:
    return PkvShape(batch, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                    max_pages_per_seq, dtype)


def _attention_shape(q, k_pool, v_pool, page_table, context_lens) -> PkvShape:
    torch = _torch()
    _require(q, "q", ndim=3)
    dev = q.device
    _require(k_pool, "k_pool", dtype=q.dtype, ndim=4, device=dev)
    _require(v_pool, "v_pool", dtype=q.dtype, ndim=4, device=dev)
    _require(page_table, "page_table", dtype=torch.int32, ndim=2, device=dev)
    _require(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=dev)
    B, Hq, D = q.shape
    NP, PS, Hkv, D2 = k_pool.shape
    if tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_pool and v_pool shapes differ")
    if D2 != D:
        raise ValueError("head_dim of q and the pools differ")
    if page_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("page_table / context_lens batch differs from q")
    return make_shape(B, Hq, Hkv, D, PS, NP, page_table.shape[1], _dtype_code(q))


def _default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def partitions_needed(page_size: int, max_pages_per_seq: int, partition_tokens: int) -> int:
    return -(-(page_size * max_pages_per_seq) // partition_tokens)


# ----------------------------------------------------------------------------------------------
# entry points (same names as the C ABI, without the prefix)
# ----------------------------------------------------------------------------------------------

def paged_decode_attention(q, k_pool, v_pool, page_table, context_lens,
                           scale: Optional[float] = None, out=None):
    """Single-pass decode attention; returns ``out [B, Hq, D]`` (dtype of q)."""
    s = _attention_shape(q, k_pool, v_pool, page_table, context_lens)
    if out is None:
        out = _torch().empty_like(q)
    _require(out, "out", dtype=q.dtype, ndim=3, device=q.device)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    scale = _default_scale(s.head_dim) if scale is None else float(scale)
    _check(lib.pkv_paged_decode_attention(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                          page_table.data_ptr(), context_lens.data_ptr(),
                                          scale, out.data_ptr(), ctypes.byref(s),
                                          _stream(q.device)))
    return out


def paged_decode_attention_partial(q, k_pool, v_pool, page_table, context_lens,
                                   partition_tokens: int, scale: Optional[float] = None,
                                   partial_out=None, partial_lse=None,
                                   max_partitions: Optional[int] = None) -> Tuple:
    """Split-KV partials; returns ``(partial_out [B,Hq,P,D], partial_lse [B,Hq,P])`` float32."""
    torch = _torch()
    s = _attention_shape(q, k_pool, v_pool, page_table, context_lens)
    if max_partitions is None:
        max_partitions = (partial_lse.shape[2] if partial_lse is not None else
                          partitions_needed(s.page_size, s.max_pages_per_seq, partition_tokens))
    if partial_out is None:
        partial_out = torch.empty((s.batch, s.num_q_heads, max_partitions, s.head_dim),
                                  dtype=torch.float32, device=q.device)
    if partial_lse is None:
        partial_lse = torch.empty((s.batch, s.num_q_heads, max_partitions),
                                  dtype=torch.float32, device=q.device)
    _require(partial_out, "partial_out", dtype=torch.float32, ndim=4, device=q.device)
    _require(partial_lse, "partial_lse", dtype=torch.float32, ndim=3, device=q.device)
    if (tuple(partial_out.shape) != (s.batch, s.num_q_heads, max_partitions, s.head_dim)
            or tuple(partial_lse.shape) != (s.batch, s.num_q_heads, max_partitions)):
        raise ValueError("partial buffers have the wrong shape")
    scale = _default_scale(s.head_dim) if scale is None else float(scale)
    _check(lib.pkv_paged_decode_attention_partial(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), page_table.data_ptr(),
        context_lens.data_ptr(), scale, int(partition_tokens), partial_out.data_ptr(),
        partial_lse.data_ptr(), int(max_partitions), ctypes.byref(s), _stream(q.device)))
    return partial_out, partial_lse


def lse_merge(partial_out, partial_lse, context_lens, partition_tokens: int, page_size: int,
              max_pages_per_seq: int, out=None, dtype=None, lse_out=None):
    """Merge split-KV partials into ``out [B, Hq, D]``; optionally also writes ``lse_out``."""
    torch = _torch()
    _require(partial_out, "partial_out", dtype=torch.float32, ndim=4)
    dev = partial_out.device
    _require(partial_lse, "partial_lse", dtype=torch.float32, ndim=3, device=dev)
    _require(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=dev)
    B, Hq, P, D = partial_out.shape
    if tuple(partial_lse.shape) != (B, Hq, P):
        raise ValueError("partial_lse shape does not match partial_out")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=dtype or torch.float32, device=dev)
    _require(out, "out", ndim=3, device=dev)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B, Hq, D]")
    lse_ptr = None
    if lse_out is not None:
        _require(lse_out, "lse_out", dtype=torch.float32, ndim=2, device=dev)
        lse_ptr = lse_out.data_ptr()
    # KV-head count and pool size do not enter the merge; any valid values do.
    s = make_shape(B, Hq, Hq, D, page_size, 1, max_pages_per_seq, _dtype_code(out))
    _check(lib.pkv_lse_merge(partial_out.data_ptr(), partial_lse.data_ptr(),
                             context_lens.data_ptr(), int(partition_tokens), int(P),
                             out.data_ptr(), lse_ptr, ctypes.byref(s), _stream(dev)))
    return out


def paged_decode_attention_split(q, k_pool, v_pool, page_table, context_lens,
                                 partition_tokens: int, scale: Optional[float] = None,
                                 out=None, partial_out=None, partial_lse=None, lse_out=None):
    """Split-KV decode: the partial call followed by the merge call on the same stream."""
    po, pl = paged_decode_attention_partial(q, k_pool, v_pool, page_table, context_lens,
                                            partition_tokens, scale, partial_out, partial_lse)
    return lse_merge(po, pl, context_lens, partition_tokens, k_pool.shape[1],
                     page_table.shape[1], out=out if out is not None else _torch().empty_like(q),
                     lse_out=lse_out)


def paged_decode_cascade(q, k_pool, v_pool, prefix_pages, prefix_tokens: int, page_table,
                         context_lens, partition_tokens: int, scale: Optional[float] = None,
                         out=None, lse_out=None, partial_out=None, partial_lse=None):
    """Shared-prefix decode: tokens ``t < prefix_tokens`` of every sequence are read from
    ``prefix_pages`` (int32 ``[prefix_tokens / page_size]``), the rest through ``page_table``.
    Returns ``out [B, Hq, D]``; the partials (allocated when not given) are the workspace."""
    torch = _torch()
    s = _attention_shape(q, k_pool, v_pool, page_table, context_lens)
    _require(prefix_pages, "prefix_pages", dtype=torch.int32, ndim=1, device=q.device)
    if prefix_pages.shape[0] * s.page_size < prefix_tokens:
        raise ValueError("prefix_pages holds fewer than prefix_tokens / page_size ids")
    max_partitions = (partial_lse.shape[2] if partial_lse is not None else
                      partitions_needed(s.page_size, s.max_pages_per_seq, partition_tokens))
    if partial_out is None:
        partial_out = torch.empty((s.batch, s.num_q_heads, max_partitions, s.head_dim),
                                  dtype=torch.float32, device=q.device)
    if partial_lse is None:
        partial_lse = torch.empty((s.batch, s.num_q_heads, max_partitions),
                                  dtype=torch.float32, device=q.device)
    _require(partial_out, "partial_out", dtype=torch.float32, ndim=4, device=q.device)
    _require(partial_lse, "partial_lse", dtype=torch.float32, ndim=3, device=q.device)
    if (tuple(partial_out.shape) != (s.batch, s.num_q_heads, max_partitions, s.head_dim)
            or tuple(partial_lse.shape) != (s.batch, s.num_q_heads, max_partitions)):
        raise ValueError("partial buffers have the wrong shape")
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", dtype=q.dtype, ndim=3, device=q.device)
    lse_ptr = None
    if lse_out is not None:
        _require(lse_out, "lse_out", dtype=torch.float32, ndim=2, device=q.device)
        lse_ptr = lse_out.data_ptr()
    scale = _default_scale(s.head_dim) if scale is None else float(scale)
    _check(lib.pkv_paged_decode_cascade(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), prefix_pages.data_ptr(),
        int(prefix_tokens), page_table.data_ptr(), context_lens.data_ptr(), scale,
        int(partition_tokens), partial_out.data_ptr(), partial_lse.data_ptr(),
        int(max_partitions), out.data_ptr(), lse_ptr, ctypes.byref(s), _stream(q.device)))
    return out


def paged_decode_multi_query(q, k_pool, v_pool, page_table, context_lens, partition_tokens: int = 1024,
                             scale: Optional[float] = None, out=None, lse_out=None,
                             partial_out=None, partial_lse=None):
    """Causal decode of T new tokens per sequence: ``q [B, T, Hq, D]``; ``context_lens[b]``
    counts the T new tokens too.  Returns ``out [B, T, Hq, D]``."""
    torch = _torch()
    _require(q, "q", ndim=4)
    B, T, Hq, D = q.shape
    s = _attention_shape(torch.empty((B, Hq, D), dtype=q.dtype, device=q.device), k_pool,
                         v_pool, page_table, context_lens)   # shapes only
    maxp = (partial_lse.shape[3] if partial_lse is not None else
            partitions_needed(s.page_size, s.max_pages_per_seq, partition_tokens))
    if partial_out is None:
        partial_out = torch.empty((B, T, Hq, maxp, D), dtype=torch.float32, device=q.device)
    if partial_lse is None:
        partial_lse = torch.empty((B, T, Hq, maxp), dtype=torch.float32, device=q.device)
    _require(partial_out, "partial_out", dtype=torch.float32, ndim=5, device=q.device)
    _require(partial_lse, "partial_lse", dtype=torch.float32, ndim=4, device=q.device)
    if (tuple(partial_out.shape) != (B, T, Hq, maxp, D)
            or tuple(partial_lse.shape) != (B, T, Hq, maxp)):
        raise ValueError("partial buffers have the wrong shape")
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", dtype=q.dtype, ndim=4, device=q.device)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must be [B, T, Hq, D]")
    lse_ptr = None
    if lse_out is not None:
        _require(lse_out, "lse_out", dtype=torch.float32, ndim=3, device=q.device)
        lse_ptr = lse_out.data_ptr()
    scale = _default_scale(s.head_dim) if scale is None else float(scale)
    _check(lib.pkv_paged_decode_multi_query(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), page_table.data_ptr(),
        context_lens.data_ptr(), int(T), scale, int(partition_tokens), partial_out.data_ptr(),
        partial_lse.data_ptr(), int(maxp), out.data_ptr(), lse_ptr, ctypes.byref(s),
        _stream(q.device)))
    return out


def multi_query_step_workspace_bytes(q, k_pool, page_table) -> int:
    """Workspace bytes paged_decode_multi_query_step needs for ``q [B, T, Hq, D]``."""
    B, T, Hq, D = q.shape
    NP, PS, Hkv, _ = k_pool.shape
    s = make_shape(B, Hq, Hkv, D, PS, NP, page_table.shape[1], _dtype_code(q))
    return int(lib.pkv_multi_query_step_workspace_bytes(ctypes.byref(s), int(T)))


def paged_decode_multi_query_step(q, k_pool, v_pool, page_table, context_lens,
                                  scale: Optional[float] = None, out=None, lse_out=None,
                                  workspace=None):
    """Causal decode of T new tokens per sequence through the balanced step (one launch; the
    T x G query rows of a KV head are its columns): ``q [B, T, Hq, D]``, ``context_lens[b]``
    counts the T new tokens too.  Returns ``out [B, T, Hq, D]``."""
    torch = _torch()
    _require(q, "q", ndim=4)
    B, T, Hq, D = q.shape
    s = _attention_shape(torch.empty((B, Hq, D), dtype=q.dtype, device=q.device), k_pool,
                         v_pool, page_table, context_lens)   # shapes only
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", dtype=q.dtype, ndim=4, device=q.device)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must be [B, T, Hq, D]")
    lse_ptr = None
    if lse_out is not None:
        _require(lse_out, "lse_out", dtype=torch.float32, ndim=3, device=q.device)
        if tuple(lse_out.shape) != (B, T, Hq):
            raise ValueError("lse_out must be [B, T, Hq]")
        lse_ptr = lse_out.data_ptr()
    need = int(lib.pkv_multi_query_step_workspace_bytes(ctypes.byref(s), int(T)))
    if workspace is None:   # zero-filled once: the step leaves its counters at zero
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", dtype=torch.uint8, ndim=1, device=q.device)
    scale = _default_scale(s.head_dim) if scale is None else float(scale)
    _check(lib.pkv_paged_decode_multi_query_step(
        q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), page_table.data_ptr(),
        context_lens.data_ptr(), int(T), scale, workspace.data_ptr(), workspace.numel(),
        out.data_ptr(), lse_ptr, ctypes.byref(s), _stream(q.device)))
    return out


def decode_step_workspace_bytes(q, k_pool, page_table) -> int:
    """Workspace bytes paged_decode_step needs for these shapes on the current device."""
    NP, PS, Hkv, D = k_pool.shape
    s = make_shape(q.shape[0], q.shape[1], Hkv, D, PS, NP, page_table.shape[1], _dtype_code(q))
    return int(lib.pkv_decode_step_workspace_bytes(ctypes.byref(s)))


def paged_decode_step(q, k_pool, v_pool, page_table, context_lens, scale: Optional[float] = None,
                      k_new=None, v_new=None, out=None, lse_out=None, workspace=None,
                      rope_cos=None, rope_sin=None):
    """Balanced decode step: optional append of k_new/v_new at context_lens[b], then attention
    over context_lens[b] (+1 with the append).  With ``rope_cos`` / ``rope_sin`` (the float32
    rotary cache ``[positions, D/2]``; needs the append) the new key and the query are rotated
    at position context_lens[b] in the same launch.  Returns ``out [B, Hq, D]``."""
    torch = _torch()
    s = _attention_shape(q, k_pool, v_pool, page_table, context_lens)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    if k_new is not None:
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            _require(t, n, dtype=q.dtype, ndim=3, device=q.device)
            if tuple(t.shape) != (s.batch, s.num_kv_heads, s.head_dim):
                raise ValueError(f"{n} must be [B, Hkv, D]")
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", dtype=q.dtype, ndim=3, device=q.device)
    lse_ptr = None
    if lse_out is not None:
        _require(lse_out, "lse_out", dtype=torch.float32, ndim=2, device=q.device)
        lse_ptr = lse_out.data_ptr()
    need = int(lib.pkv_decode_step_workspace_bytes(ctypes.byref(s)))
    if workspace is None:   # zero-filled once: the step leaves its counters at zero
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", dtype=torch.uint8, ndim=1, device=q.device)
    scale = _default_scale(s.head_dim) if scale is None else float(scale)
    if rope_cos is not None or rope_sin is not None:
        if rope_cos is None or rope_sin is None or k_new is None:
            raise ValueError("the rotary step needs rope_cos, rope_sin and the appended rows")
        for t, n in ((rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
            _require(t, n, dtype=torch.float32, ndim=2, device=q.device)
            if t.shape[1] != s.head_dim // 2 or t.shape != rope_cos.shape:
                raise ValueError(f"{n} must be [positions, D/2]")
        _check(lib.pkv_paged_decode_step_rope(
            q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(),
            v_pool.data_ptr(), page_table.data_ptr(), context_lens.data_ptr(),
            rope_cos.data_ptr(), rope_sin.data_ptr(), int(rope_cos.shape[0]), scale,
            workspace.data_ptr(), workspace.numel(), out.data_ptr(), lse_ptr, ctypes.byref(s),
            _stream(q.device)))
        return out
    _check(lib.pkv_paged_decode_step(
        q.data_ptr(), None if k_new is None else k_new.data_ptr(),
        None if v_new is None else v_new.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        page_table.data_ptr(), context_lens.data_ptr(), scale, workspace.data_ptr(),
        workspace.numel(), out.data_ptr(), lse_ptr, ctypes.byref(s), _stream(q.device)))
    return out


def paged_decode_step_noalloc(q, k_pool, v_pool, page_table, context_lens, out, scale=None,
                              k_new=None, v_new=None, lse_out=None):
    """paged_decode_step with the library's static device scratch as its workspace (the C call
    allocates nothing; ``out`` is the caller's).  Same results as paged_decode_step."""
    torch = _torch()
    s = _attention_shape(q, k_pool, v_pool, page_table, context_lens)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    if k_new is not None:
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            _require(t, n, dtype=q.dtype, ndim=3, device=q.device)
            if tuple(t.shape) != (s.batch, s.num_kv_heads, s.head_dim):
                raise ValueError(f"{n} must be [B, Hkv, D]")
    _require(out, "out", dtype=q.dtype, ndim=3, device=q.device)
    lse_ptr = None
    if lse_out is not None:
        _require(lse_out, "lse_out", dtype=torch.float32, ndim=2, device=q.device)
        lse_ptr = lse_out.data_ptr()
    scale = _default_scale(s.head_dim) if scale is None else float(scale)
    _check(lib.pkv_paged_decode_step_noalloc(
        q.data_ptr(), None if k_new is None else k_new.data_ptr(),
        None if v_new is None else v_new.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        page_table.data_ptr(), context_lens.data_ptr(), scale, out.data_ptr(), lse_ptr,
        ctypes.byref(s), _stream(q.device)))
    return out


def paged_kv_append(k_new, v_new, k_pool, v_pool, page_table, context_lens) -> None:
    """Write each row's new K/V at position ``context_lens[b]`` (in place, stream-ordered)."""
    torch = _torch()
    _require(k_pool, "k_pool", ndim=4)
    dev = k_pool.device
    _require(v_pool, "v_pool", dtype=k_pool.dtype, ndim=4, device=dev)
    _require(k_new, "k_new", dtype=k_pool.dtype, ndim=3, device=dev)
    _require(v_new, "v_new", dtype=k_pool.dtype, ndim=3, device=dev)
    _require(page_table, "page_table", dtype=torch.int32, ndim=2, device=dev)
    _require(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=dev)
    NP, PS, Hkv, D = k_pool.shape
    B = k_new.shape[0]
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new / v_new must be [B, Hkv, D]")
    if tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("k_pool and v_pool shapes differ")
    s = make_shape(B, Hkv, Hkv, D, PS, NP, page_table.shape[1], _dtype_code(k_pool))
    _check(lib.pkv_paged_kv_append(k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(),
                                   v_pool.data_ptr(), page_table.data_ptr(),
                                   context_lens.data_ptr(), ctypes.byref(s), _stream(dev)))


def rope_kv_append(q, k_new, v_new, k_pool, v_pool, page_table, context_lens, rope_cos, rope_sin,
                   q_out=None):
    """Rotary embedding + append of the new token at position ``context_lens[b]``: q rotated into
    ``q_out`` (returned), k_new rotated and v_new written into the pools.  ``rope_cos`` /
    ``rope_sin`` are the float32 rotary cache ``[positions, D/2]``."""
    torch = _torch()
    s = _attention_shape(q, k_pool, v_pool, page_table, context_lens)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _require(t, n, dtype=q.dtype, ndim=3, device=q.device)
        if tuple(t.shape) != (s.batch, s.num_kv_heads, s.head_dim):
            raise ValueError(f"{n} must be [B, Hkv, D]")
    for t, n in ((rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
        _require(t, n, dtype=torch.float32, ndim=2, device=q.device)
        if t.shape[1] != s.head_dim // 2 or t.shape != rope_cos.shape:
            raise ValueError(f"{n} must be [positions, D/2]")
    if q_out is None:
        q_out = torch.empty_like(q)
    _require(q_out, "q_out", dtype=q.dtype, ndim=3, device=q.device)
    _check(lib.pkv_rope_kv_append(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        page_table.data_ptr(), context_lens.data_ptr(), rope_cos.data_ptr(), rope_sin.data_ptr(),
        int(rope_cos.shape[0]), q_out.data_ptr(), ctypes.byref(s), _stream(q.device)))
    return q_out


def validate_metadata(page_table, context_lens, num_pages: int, page_size: int,
                      extra_tokens: int = 0, check_append_unique: bool = False,
                      status=None, sync: bool = True):
    """Device-side metadata check.  Returns the status word (syncs) or the status tensor."""
    torch = _torch()
    _require(page_table, "page_table", dtype=torch.int32, ndim=2)
    dev = page_table.device
    _require(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=dev)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=dev)
    B, MP = page_table.shape
    s = make_shape(B, 1, 1, 64, page_size, num_pages, MP, PKV_F32)
    _check(lib.pkv_validate_metadata(page_table.data_ptr(), context_lens.data_ptr(),
                                     int(extra_tokens), 1 if check_append_unique else 0,
                                     status.data_ptr(), ctypes.byref(s), _stream(dev)))
    return int(status.item()) if sync else status


def partial_workspace_bytes(batch, num_q_heads, head_dim, max_partitions, page_size=16,
                            max_pages_per_seq=1) -> int:
    s = make_shape(batch, num_q_heads, num_q_heads, head_dim, page_size, 1, max_pages_per_seq, PKV_F32)
    return int(lib.pkv_partial_workspace_bytes(ctypes.byref(s), int(max_partitions)))


# ----------------------------------------------------------------------------------------------
# host page allocator
# ----------------------------------------------------------------------------------------------

def copy_pages(k_pool, v_pool, pairs) -> None:
    """Copy whole pages in both pools: ``pairs`` is a device int32 ``[n, 2]`` of (src, dst)."""
    torch = _torch()
    _require(k_pool, "k_pool", ndim=4)
    _require(v_pool, "v_pool", dtype=k_pool.dtype, ndim=4, device=k_pool.device)
    _require(pairs, "pairs", dtype=torch.int32, ndim=2, device=k_pool.device)
    NP, PS, Hkv, D = k_pool.shape
    s = make_shape(0, Hkv, Hkv, D, PS, NP, 1, _dtype_code(k_pool))
    _check(lib.pkv_copy_pages(k_pool.data_ptr(), v_pool.data_ptr(), pairs.data_ptr(),
                              int(pairs.shape[0]), ctypes.byref(s), _stream(k_pool.device)))


def read_stream(buf, sink) -> None:
    """Read every byte of the contiguous device tensor ``buf`` once (measurement of the device's
    read bandwidth); one word per workgroup of what was read is folded by XOR into ``sink`` (a
    device int32 tensor of one element or more, first element used)."""
    torch = _torch()
    _require(buf, "buf")
    _require(sink, "sink", dtype=torch.int32, device=buf.device)
    _check(lib.pkv_read_stream(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                               _stream(buf.device)))


def _page_check(rc: int) -> None:
    if rc != PKV_OK:
        raise PkvError(rc, lib.pkv_pages_last_error().decode())


class PageAllocator:
    """The library's host page allocator (reference-counted pages, forks, copy-on-write growth,
    prefix cache); see ``pkv_pages_*`` in include/pkv.h."""

    def __init__(self, num_pages: int, page_size: int):
        self._h = lib.pkv_pages_create(int(num_pages), int(page_size))
        if not self._h:
            raise PkvError(PKV_EINVAL, lib.pkv_pages_last_error().decode())
        self.page_size = page_size

    def close(self):
        if self._h:
            lib.pkv_pages_destroy(self._h)
            self._h = None

    __del__ = close

    def free_count(self) -> int:
        return int(lib.pkv_pages_free_count(self._h))

    def refcount(self, page: int) -> int:
        return int(lib.pkv_pages_refcount(self._h, int(page)))

    def create(self) -> int:
        out = _i32()
        _page_check(lib.pkv_pages_seq_create(self._h, ctypes.byref(out)))
        return out.value

    def fork(self, seq: int) -> int:
        out = _i32()
        _page_check(lib.pkv_pages_seq_fork(self._h, int(seq), ctypes.byref(out)))
        return out.value

    def release(self, seq: int) -> None:
        _page_check(lib.pkv_pages_seq_release(self._h, int(seq)))

    def reserve(self, seq: int, n_tokens: int):
        """Grow by n_tokens; returns the (src, dst) page copies to run before appending."""
        buf = (_i32 * 2)()
        n = _i32()
        _page_check(lib.pkv_pages_seq_reserve(self._h, int(seq), int(n_tokens), buf, 1,
                                              ctypes.byref(n)))
        return [(buf[0], buf[1])] if n.value else []

    def length(self, seq: int) -> int:
        out = _i32()
        _page_check(lib.pkv_pages_seq_length(self._h, int(seq), ctypes.byref(out)))
        return out.value

    def table(self, seq: int, max_pages: Optional[int] = None):
        n = _i32()
        if max_pages is None:
            lib.pkv_pages_seq_table(self._h, int(seq), (_i32 * 1)(), 0, ctypes.byref(n))
            max_pages = n.value
        row = (_i32 * max(max_pages, 1))()
        _page_check(lib.pkv_pages_seq_table(self._h, int(seq), row, int(max_pages), ctypes.byref(n)))
        return list(row[:max_pages])

    def prefix_insert(self, seq: int, tokens) -> None:
        arr = (_i32 * max(len(tokens), 1))(*tokens)
        _page_check(lib.pkv_pages_prefix_insert(self._h, int(seq), arr, len(tokens)))

    def create_with_prefix(self, tokens):
        arr = (_i32 * max(len(tokens), 1))(*tokens)
        sid, matched = _i32(), _i32()
        _page_check(lib.pkv_pages_seq_create_with_prefix(self._h, arr, len(tokens),
                                                         ctypes.byref(sid), ctypes.byref(matched)))
        return sid.value, matched.value

    def evict(self, max_pages: int) -> int:
        out = _i32()
        _page_check(lib.pkv_pages_prefix_evict(self._h, int(max_pages), ctypes.byref(out)))
        return out.value
