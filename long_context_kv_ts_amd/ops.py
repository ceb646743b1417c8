"""Thin Python binding of ``libts.so`` (the C ABI declared in ``include/ts.h``).

Argument marshalling only: torch tensors supply device memory, shapes and the
current HIP stream; every step of the computation runs in the library's
kernels. There is no fallback: if the library is missing or a call fails, an
exception is raised.

Entry points, named as the C functions without the ``ts_`` prefix:

* verify and partial-cache step: ``tree_verify_attn`` (and ``tree_verify_attn_noalloc``,
  its variant without a workspace), ``tree_verify_attn_partials``,
  ``tree_verify_attn_partials_and_importance``,
  ``attn_merge``, ``kv_importance_score``, ``attn_merge_and_importance``, ``kv_topk_select``, ``kv_gather``,
  ``partial_draft_attn``;
* decode step around them: ``build_draft_tree`` (with ``draft_tree_nodes``),
  ``sample_tokens``, ``accept_commit``, and the ``NgramTable`` class over
  ``ts_ngram_init`` / ``ts_ngram_update`` / ``ts_ngram_retrieve``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_LIB_PATH = os.environ.get("TS_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libts.so")
_lib = None

TS_OK, TS_ERR_INVALID_ARG, TS_ERR_UNSUPPORTED, TS_ERR_WORKSPACE, TS_ERR_HIP = range(5)
TS_F32, TS_BF16 = 0, 1

_c_void_p, _c_int, _c_i64, _c_f, _c_size = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                            ctypes.c_float, ctypes.c_size_t)

# name -> (restype, argtypes); must mirror include/ts.h
SIGNATURES = {
    "ts_last_error": (ctypes.c_char_p, []),
    "ts_abi_version": (_c_int, []),
    "ts_tree_verify_attn_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_i64, _c_int, _c_int]),
    "ts_tree_verify_attn": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_i64, _c_void_p, _c_void_p,
                                     _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                     _c_i64, _c_f, _c_int, _c_int, _c_void_p, _c_size, _c_void_p]),
    "ts_tree_verify_attn_noalloc": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_i64, _c_void_p, _c_void_p,
                                             _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                             _c_i64, _c_f, _c_int, _c_int, _c_void_p]),
    "ts_tree_verify_attn_num_splits": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_i64, _c_int, _c_int]),
    "ts_tree_verify_attn_partials": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_i64, _c_void_p,
                                              _c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p, _c_int,
                                              _c_int, _c_int, _c_int, _c_i64, _c_f, _c_int, _c_int,
                                              _c_void_p]),
    "ts_tree_verify_attn_partials_and_importance": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_i64, _c_void_p,
                                                             _c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p,
                                                             _c_int, _c_int, _c_int, _c_int, _c_i64, _c_f, _c_int,
                                                             _c_int, _c_void_p, _c_int, _c_int, _c_f, _c_void_p,
                                                             _c_void_p]),
    "ts_attn_merge": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                               _c_int, _c_void_p]),
    "ts_kv_importance_score": (_c_int, [_c_void_p, _c_void_p, _c_i64, _c_void_p, _c_int, _c_int,
                                        _c_int, _c_int, _c_i64, _c_int, _c_f, _c_int, _c_void_p]),
    "ts_attn_merge_and_importance": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_int, _c_int, _c_void_p,
                                              _c_void_p, _c_int, _c_void_p, _c_void_p, _c_i64, _c_void_p, _c_int,
                                              _c_int, _c_int, _c_int, _c_i64, _c_int, _c_f, _c_int, _c_void_p]),
    "ts_attn_merge_and_topk": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                                        _c_int, _c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p]),
    "ts_kv_topk_select": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p]),
    "ts_kv_gather": (_c_int, [_c_void_p, _c_void_p, _c_i64, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                              _c_i64, _c_void_p, _c_void_p, _c_int, _c_void_p]),
    "ts_kv_gather_and_draft_attn": (_c_int, [_c_void_p, _c_void_p, _c_i64, _c_void_p, _c_int, _c_int, _c_i64,
                                             _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                             _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_f, _c_int, _c_int,
                                             _c_void_p, _c_size, _c_void_p]),
    "ts_draft_tree_nodes": (_c_int, [_c_void_p, _c_int]),
    "ts_build_draft_tree_workspace": (_c_size, [_c_int, _c_int]),
    "ts_build_draft_tree": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                     _c_void_p, _c_int, _c_void_p, _c_size, _c_void_p]),
    "ts_accept_commit": (_c_int, [_c_void_p, _c_void_p, _c_void_p, ctypes.c_uint32, _c_int, _c_void_p,
                                  _c_void_p, _c_i64, _c_i64, _c_void_p, _c_void_p, _c_int, _c_int,
                                  _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "ts_sample_workspace": (_c_size, [_c_int, _c_int]),
    "ts_sample_tokens": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p, _c_int, _c_void_p, _c_void_p, _c_int,
                                  _c_int, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, _c_void_p,
                                  _c_void_p, _c_int, _c_void_p, _c_size, _c_void_p]),
    "ts_ngram_table_bytes": (_c_size, [_c_int, _c_int]),
    "ts_ngram_init": (_c_int, [_c_void_p, _c_size, _c_int, _c_int, _c_void_p]),
    "ts_ngram_update": (_c_int, [_c_void_p, _c_void_p, _c_i64, _c_i64, _c_void_p]),
    "ts_ngram_retrieve_workspace": (_c_size, [_c_int, _c_int]),
    "ts_ngram_retrieve": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p, _c_size, _c_void_p]),
    "ts_partial_draft_attn_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_i64, _c_int, _c_int]),
    "ts_partial_draft_attn": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                       _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_i64,
                                       _c_f, _c_int, _c_int, _c_void_p, _c_size, _c_void_p]),
}


class TsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[ts status {status}] {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libts.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m long_context_kv_ts_amd.build`")
        l = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def library_path() -> str:
    return _LIB_PATH


def _check(status: int) -> None:
    if status != TS_OK:
        raise TsError(status, lib().ts_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TS_BF16
    if t.dtype == torch.float32:
        return TS_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: Optional[torch.Tensor], name: str, dim: int, dtype=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _cache_stride(t: torch.Tensor, name: str) -> int:
    """Row stride (in tokens) of a [Hkv][stride][D] cache view whose last two
    dims are dense; lets callers pass cache[:, :L] of a larger allocation."""
    Hkv, L, D = t.shape
    if t.numel() == 0:
        return L
    if t.stride(2) != 1 or (L > 1 and t.stride(1) != D):
        raise ValueError(f"{name} must be dense in its last two dims")
    if Hkv > 1 and t.stride(0) % D:
        raise ValueError(f"{name} head stride must be a multiple of D")
    return t.stride(0) // D if Hkv > 1 else max(L, 1)


def _contig(t: torch.Tensor, name: str) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out(t: Optional[torch.Tensor], name: str, shape, dtype, device) -> Optional[torch.Tensor]:
    """Check a caller-supplied output buffer: the C ABI sees only its address,
    so a wrong size or type would become an out-of-bounds device write."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _workspace(t: Optional[torch.Tensor], name: str, need: int, device) -> Optional[torch.Tensor]:
    """Check a caller-supplied workspace: a contiguous device buffer of at least `need` bytes."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor")
    if t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.numel() * t.element_size() < need:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, {need} required")
    return t


def _parts(o_part, l_part, device=None) -> None:
    """Split partials: o_part [S][..][D] (fp32 or bf16) and l_part [S][..] fp32 on one GPU."""
    if not isinstance(o_part, torch.Tensor) or o_part.dim() < 2:
        raise ValueError("o_part must be a [S][..][D] tensor")
    if o_part.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"o_part: dtype {o_part.dtype}, expected float32 or bfloat16")
    _need(o_part, "o_part", o_part.dim(), o_part.dtype, device)
    _need(l_part, "l_part", o_part.dim() - 1, torch.float32, o_part.device)


def _part_code(o_part: torch.Tensor) -> int:
    return TS_BF16 if o_part.dtype == torch.bfloat16 else TS_F32


def _part_dtype(o_part, part_dtype) -> torch.dtype:
    """The partials' dtype: the given o_part's, else part_dtype (float32 or bfloat16)."""
    dt = o_part.dtype if o_part is not None else part_dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError(f"o_part: dtype {dt}, expected float32 or bfloat16")
    return dt


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


# ---------------------------------------------------------------------------
# workspace
# ---------------------------------------------------------------------------
def verify_workspace_bytes(T: int, Hq: int, Hkv: int, D: int, L: int, dtype: torch.dtype,
                           num_splits: int = 0) -> int:
    code = TS_BF16 if dtype == torch.bfloat16 else TS_F32
    n = lib().ts_tree_verify_attn_workspace(T, Hq, Hkv, D, L, code, num_splits)
    if n == 0:
        raise TsError(TS_ERR_INVALID_ARG, lib().ts_last_error().decode())
    return int(n)


def num_splits(T: int, Hq: int, Hkv: int, D: int, L: int, dtype: torch.dtype, num_splits: int = 0) -> int:
    code = TS_BF16 if dtype == torch.bfloat16 else TS_F32
    n = lib().ts_tree_verify_attn_num_splits(T, Hq, Hkv, D, L, code, num_splits)
    if n < 0:
        raise TsError(TS_ERR_INVALID_ARG, lib().ts_last_error().decode())
    return int(n)


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte-aligned blocks
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def tree_verify_attn(q, k_cache, v_cache, k_draft, v_draft, parent, *, scale=None, out=None,
                     lse=None, want_lse=True, num_splits: int = 0,
                     workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """ts_tree_verify_attn. q [T][Hq][D]; caches [Hkv][L][D] (a prefix view of a
    larger cache is allowed); drafts [Hkv][T][D]; parent int32 [T] on the GPU."""
    _need(q, "q", 3)
    dev = q.device
    T, Hq, D = q.shape
    _need(k_cache, "k_cache", 3, q.dtype, dev)
    _need(v_cache, "v_cache", 3, q.dtype, dev)
    _need(k_draft, "k_draft", 3, q.dtype, dev)
    _need(v_draft, "v_draft", 3, q.dtype, dev)
    _need(parent, "parent", 1, torch.int32, dev)
    Hkv, L, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if tuple(k_draft.shape) != (Hkv, T, D) or tuple(v_draft.shape) != (Hkv, T, D):
        raise ValueError(f"drafts must be [{Hkv}][{T}][{D}]")
    if parent.shape[0] != T:
        raise ValueError("parent must have T entries")
    for n, t in (("q", q), ("k_draft", k_draft), ("v_draft", v_draft), ("parent", parent)):
        _contig(t, n)
    stride = _cache_stride(k_cache, "k_cache")
    if _cache_stride(v_cache, "v_cache") != stride:
        raise ValueError("k_cache and v_cache must share the row stride")
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _out(out, "out", (T, Hq, D), q.dtype, dev)
    _out(lse, "lse", (T, Hq), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    need = verify_workspace_bytes(T, Hq, Hkv, D, L, q.dtype, num_splits)
    _workspace(workspace, "workspace", need, dev)
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    _check(lib().ts_tree_verify_attn(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), stride, k_draft.data_ptr(),
        v_draft.data_ptr(), parent.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, T, Hq, Hkv, D, L, float(scale), code,
        num_splits, workspace.data_ptr(), _nbytes(workspace), _stream(dev)))
    return out, lse


def tree_verify_attn_noalloc(q, k_cache, v_cache, k_draft, v_draft, parent, *, scale=None, out=None,
                             lse=None, want_lse=True, num_splits: int = 0):
    """ts_tree_verify_attn_noalloc: ts_tree_verify_attn with the split partials
    in the library's static device scratch instead of a workspace (the C call
    allocates nothing; pass `out`/`lse` to keep this wrapper from allocating
    them). Calls that overlap on one GPU race."""
    _need(q, "q", 3)
    dev = q.device
    T, Hq, D = q.shape
    _need(k_cache, "k_cache", 3, q.dtype, dev)
    _need(v_cache, "v_cache", 3, q.dtype, dev)
    _need(k_draft, "k_draft", 3, q.dtype, dev)
    _need(v_draft, "v_draft", 3, q.dtype, dev)
    _need(parent, "parent", 1, torch.int32, dev)
    Hkv, L, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if tuple(k_draft.shape) != (Hkv, T, D) or tuple(v_draft.shape) != (Hkv, T, D):
        raise ValueError(f"drafts must be [{Hkv}][{T}][{D}]")
    if parent.shape[0] != T:
        raise ValueError("parent must have T entries")
    for n, t in (("q", q), ("k_draft", k_draft), ("v_draft", v_draft), ("parent", parent)):
        _contig(t, n)
    stride = _cache_stride(k_cache, "k_cache")
    if _cache_stride(v_cache, "v_cache") != stride:
        raise ValueError("k_cache and v_cache must share the row stride")
    _out(out, "out", (T, Hq, D), q.dtype, dev)
    _out(lse, "lse", (T, Hq), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check(lib().ts_tree_verify_attn_noalloc(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), stride, k_draft.data_ptr(),
            v_draft.data_ptr(), parent.data_ptr(), out.data_ptr(),
            lse.data_ptr() if lse is not None else None, T, Hq, Hkv, D, L,
            float(1.0 / math.sqrt(D) if scale is None else scale), _dtype_code(q), num_splits, _stream(dev)))
    return out, lse


def tree_verify_attn_partials(q, k_cache, v_cache, k_draft, v_draft, parent, *, scale=None,
                              o_part=None, l_part=None, num_splits: int = 0, part_dtype=torch.float32):
    """ts_tree_verify_attn_partials -> (o_part [S][T][Hq][D] in part_dtype (float32, or
    bfloat16 for bf16 inputs; a given o_part's dtype wins), l_part [S][T][Hq] fp32)."""
    _need(q, "q", 3)
    dev = q.device
    T, Hq, D = q.shape
    _need(k_cache, "k_cache", 3, q.dtype, dev)
    _need(v_cache, "v_cache", 3, q.dtype, dev)
    _need(k_draft, "k_draft", 3, q.dtype, dev)
    _need(v_draft, "v_draft", 3, q.dtype, dev)
    _need(parent, "parent", 1, torch.int32, dev)
    Hkv, L, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if tuple(k_draft.shape) != (Hkv, T, D) or tuple(v_draft.shape) != (Hkv, T, D):
        raise ValueError(f"drafts must be [{Hkv}][{T}][{D}]")
    if parent.shape[0] != T:
        raise ValueError("parent must have T entries")
    for n, t in (("q", q), ("k_draft", k_draft), ("v_draft", v_draft), ("parent", parent)):
        _contig(t, n)
    stride = _cache_stride(k_cache, "k_cache")
    if _cache_stride(v_cache, "v_cache") != stride:
        raise ValueError("k_cache and v_cache must share the row stride")
    S = globals()["num_splits"](T, Hq, Hkv, D, L, q.dtype, num_splits)
    pdt = _part_dtype(o_part, part_dtype)
    _out(o_part, "o_part", (S, T, Hq, D), pdt, dev)
    _out(l_part, "l_part", (S, T, Hq), torch.float32, dev)
    if o_part is None:
        o_part = torch.empty((S, T, Hq, D), dtype=pdt, device=dev)
    if l_part is None:
        l_part = torch.empty((S, T, Hq), dtype=torch.float32, device=dev)
    _check(lib().ts_tree_verify_attn_partials(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), stride, k_draft.data_ptr(),
        v_draft.data_ptr(), parent.data_ptr(), o_part.data_ptr(), _part_code(o_part), l_part.data_ptr(), T, Hq, Hkv,
        D, L, float(1.0 / math.sqrt(D) if scale is None else scale), _dtype_code(q), num_splits,
        _stream(dev)))
    return o_part, l_part


def tree_verify_attn_partials_and_importance(q, k_cache, v_cache, k_draft, v_draft, parent, q_recent, chunk: int,
                                             *, scale=None, imp_scale=None, o_part=None, l_part=None, scores=None,
                                             num_splits: int = 0, part_dtype=torch.float32):
    """ts_tree_verify_attn_partials_and_importance: the verify split partials
    (o_part in part_dtype, as tree_verify_attn_partials) and the chunk
    importance of the same cache for the recent queries q_recent [R][Hq][D], in
    one launch where the shapes allow -> (o_part, l_part, scores)."""
    _need(q, "q", 3)
    dev = q.device
    T, Hq, D = q.shape
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_draft", k_draft), ("v_draft", v_draft),
                 ("q_recent", q_recent)):
        _need(t, n, 3, q.dtype, dev)
    _need(parent, "parent", 1, torch.int32, dev)
    Hkv, L, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if tuple(k_draft.shape) != (Hkv, T, D) or tuple(v_draft.shape) != (Hkv, T, D):
        raise ValueError(f"drafts must be [{Hkv}][{T}][{D}]")
    if parent.shape[0] != T:
        raise ValueError("parent must have T entries")
    R = q_recent.shape[0]
    if tuple(q_recent.shape[1:]) != (Hq, D):
        raise ValueError(f"q_recent must be [R][{Hq}][{D}]")
    for n, t in (("q", q), ("k_draft", k_draft), ("v_draft", v_draft), ("parent", parent), ("q_recent", q_recent)):
        _contig(t, n)
    stride = _cache_stride(k_cache, "k_cache")
    if _cache_stride(v_cache, "v_cache") != stride:
        raise ValueError("k_cache and v_cache must share the row stride")
    S = globals()["num_splits"](T, Hq, Hkv, D, L, q.dtype, num_splits)
    pdt = _part_dtype(o_part, part_dtype)
    _out(o_part, "o_part", (S, T, Hq, D), pdt, dev)
    _out(l_part, "l_part", (S, T, Hq), torch.float32, dev)
    _out(scores, "scores", (Hkv, L // max(int(chunk), 1)), torch.float32, dev)
    if o_part is None:
        o_part = torch.empty((S, T, Hq, D), dtype=pdt, device=dev)
    if l_part is None:
        l_part = torch.empty((S, T, Hq), dtype=torch.float32, device=dev)
    if scores is None:
        scores = torch.empty((Hkv, L // chunk), dtype=torch.float32, device=dev)
    sc = float(1.0 / math.sqrt(D) if scale is None else scale)
    isc = float(1.0 / math.sqrt(D) if imp_scale is None else imp_scale)
    _check(lib().ts_tree_verify_attn_partials_and_importance(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), stride, k_draft.data_ptr(), v_draft.data_ptr(),
        parent.data_ptr(), o_part.data_ptr(), _part_code(o_part), l_part.data_ptr(), T, Hq, Hkv, D, L, sc,
        _dtype_code(q), num_splits,
        q_recent.data_ptr(), R, int(chunk), isc, scores.data_ptr(), _stream(dev)))
    return o_part, l_part, scores


def attn_merge(o_part, l_part, *, out_dtype=torch.bfloat16, out=None, lse=None):
    """ts_attn_merge over the leading (parts) dim: o_part [S][..][D] (fp32 or bf16), l_part [S][..]."""
    _parts(o_part, l_part)
    dev = o_part.device
    _contig(o_part, "o_part")
    _contig(l_part, "l_part")
    S = o_part.shape[0]
    D = o_part.shape[-1]
    rows = o_part[0].numel() // D
    if tuple(l_part.shape) != tuple(o_part.shape[:-1]):
        raise ValueError("l_part does not match o_part")
    _out(out, "out", o_part.shape[1:], out.dtype if out is not None else out_dtype, dev)
    _out(lse, "lse", l_part.shape[1:], torch.float32, dev)
    if out is None:
        out = torch.empty(o_part.shape[1:], dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty(l_part.shape[1:], dtype=torch.float32, device=dev)
    _check(lib().ts_attn_merge(o_part.data_ptr(), _part_code(o_part), l_part.data_ptr(), S, rows, D, out.data_ptr(),
                               lse.data_ptr(), _dtype_code(out), _stream(dev)))
    return out, lse


def kv_importance_score(q_recent, k_cache, chunk: int, *, scale=None, scores=None):
    """ts_kv_importance_score -> scores [Hkv][L/chunk] fp32."""
    _need(q_recent, "q_recent", 3)
    dev = q_recent.device
    _need(k_cache, "k_cache", 3, q_recent.dtype, dev)
    _contig(q_recent, "q_recent")
    R, Hq, D = q_recent.shape
    Hkv, L, _ = k_cache.shape
    stride = _cache_stride(k_cache, "k_cache")
    _out(scores, "scores", (Hkv, L // max(int(chunk), 1)), torch.float32, dev)
    if scores is None:
        scores = torch.empty((Hkv, L // chunk), dtype=torch.float32, device=dev)
    _check(lib().ts_kv_importance_score(
        q_recent.data_ptr(), k_cache.data_ptr(), stride, scores.data_ptr(), R, Hq, Hkv, D, L,
        chunk, float(1.0 / math.sqrt(D) if scale is None else scale), _dtype_code(q_recent),
        _stream(dev)))
    return scores


def attn_merge_and_importance(o_part, l_part, q_recent, k_cache, chunk: int, *, out_dtype=torch.bfloat16,
                              out=None, lse=None, scale=None, scores=None):
    """ts_attn_merge_and_importance: attn_merge(o_part, l_part) and
    kv_importance_score(q_recent, k_cache, chunk) in one launch where the
    shapes allow -> (out, lse, scores), bit-identical to the two calls."""
    _need(q_recent, "q_recent", 3)
    dev = q_recent.device
    _parts(o_part, l_part, dev)
    _contig(o_part, "o_part")
    _contig(l_part, "l_part")
    S, Dv = o_part.shape[0], o_part.shape[-1]
    rows = o_part[0].numel() // Dv
    if tuple(l_part.shape) != tuple(o_part.shape[:-1]):
        raise ValueError("l_part does not match o_part")
    _need(k_cache, "k_cache", 3, q_recent.dtype, dev)
    _contig(q_recent, "q_recent")
    R, Hq, D = q_recent.shape
    Hkv, L, _ = k_cache.shape
    stride = _cache_stride(k_cache, "k_cache")
    _out(out, "out", o_part.shape[1:], out.dtype if out is not None else out_dtype, dev)
    _out(lse, "lse", l_part.shape[1:], torch.float32, dev)
    _out(scores, "scores", (Hkv, L // max(int(chunk), 1)), torch.float32, dev)
    if out is None:
        out = torch.empty(o_part.shape[1:], dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty(l_part.shape[1:], dtype=torch.float32, device=dev)
    if scores is None:
        scores = torch.empty((Hkv, L // chunk), dtype=torch.float32, device=dev)
    _check(lib().ts_attn_merge_and_importance(
        o_part.data_ptr(), _part_code(o_part), l_part.data_ptr(), S, rows, Dv, out.data_ptr(), lse.data_ptr(),
        _dtype_code(out), q_recent.data_ptr(), k_cache.data_ptr(), stride, scores.data_ptr(), R, Hq, Hkv, D, L, chunk,
        float(1.0 / math.sqrt(D) if scale is None else scale), _dtype_code(q_recent), _stream(dev)))
    return out, lse, scores


def attn_merge_and_topk(o_part, l_part, scores, k: int, *, out_dtype=torch.bfloat16, out=None, lse=None,
                        chunk_idx=None, chunk_score=None, want_scores=True):
    """ts_attn_merge_and_topk: attn_merge(o_part, l_part) and kv_topk_select(scores, k)
    in one launch where the merge allows -> (out, lse, chunk_idx, chunk_score),
    bit-identical to the two calls."""
    _parts(o_part, l_part)
    dev = o_part.device
    _contig(o_part, "o_part")
    _contig(l_part, "l_part")
    S, Dv = o_part.shape[0], o_part.shape[-1]
    rows = o_part[0].numel() // Dv
    if tuple(l_part.shape) != tuple(o_part.shape[:-1]):
        raise ValueError("l_part does not match o_part")
    _need(scores, "scores", 2, torch.float32, dev)
    _contig(scores, "scores")
    Hkv, n = scores.shape
    _out(out, "out", o_part.shape[1:], out.dtype if out is not None else out_dtype, dev)
    _out(lse, "lse", l_part.shape[1:], torch.float32, dev)
    _out(chunk_idx, "chunk_idx", (Hkv, k), torch.int32, dev)
    _out(chunk_score, "chunk_score", (Hkv, k), torch.float32, dev)
    if out is None:
        out = torch.empty(o_part.shape[1:], dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty(l_part.shape[1:], dtype=torch.float32, device=dev)
    if chunk_idx is None:
        chunk_idx = torch.empty((Hkv, k), dtype=torch.int32, device=dev)
    if chunk_score is None and want_scores:
        chunk_score = torch.empty((Hkv, k), dtype=torch.float32, device=dev)
    _check(lib().ts_attn_merge_and_topk(o_part.data_ptr(), _part_code(o_part), l_part.data_ptr(), S, rows, Dv,
                                        out.data_ptr(),
                                        lse.data_ptr(), _dtype_code(out), scores.data_ptr(), Hkv, n, k,
                                        chunk_idx.data_ptr(),
                                        chunk_score.data_ptr() if chunk_score is not None else None, _stream(dev)))
    return out, lse, chunk_idx, chunk_score


def kv_topk_select(scores, k: int, *, chunk_idx=None, chunk_score=None, want_scores=True):
    """ts_kv_topk_select -> (chunk_idx int32 [Hkv][k] ascending, chunk_score fp32 [Hkv][k])."""
    _need(scores, "scores", 2, torch.float32)
    _contig(scores, "scores")
    Hkv, n = scores.shape
    dev = scores.device
    _out(chunk_idx, "chunk_idx", (Hkv, k), torch.int32, dev)
    _out(chunk_score, "chunk_score", (Hkv, k), torch.float32, dev)
    if chunk_idx is None:
        chunk_idx = torch.empty((Hkv, k), dtype=torch.int32, device=dev)
    if chunk_score is None and want_scores:
        chunk_score = torch.empty((Hkv, k), dtype=torch.float32, device=dev)
    _check(lib().ts_kv_topk_select(scores.data_ptr(), Hkv, n, k, chunk_idx.data_ptr(),
                                   chunk_score.data_ptr() if chunk_score is not None else None,
                                   _stream(dev)))
    return chunk_idx, chunk_score


def kv_gather(k_cache, v_cache, chunk_idx, chunk: int, *, k_part=None, v_part=None):
    """ts_kv_gather -> (k_part, v_part) [Hkv][k*chunk][D]."""
    _need(k_cache, "k_cache", 3)
    dev = k_cache.device
    _need(v_cache, "v_cache", 3, k_cache.dtype, dev)
    _need(chunk_idx, "chunk_idx", 2, torch.int32, dev)
    _contig(chunk_idx, "chunk_idx")
    Hkv, L, D = k_cache.shape
    k = chunk_idx.shape[1]
    stride = _cache_stride(k_cache, "k_cache")
    if _cache_stride(v_cache, "v_cache") != stride:
        raise ValueError("k_cache and v_cache must share the row stride")
    if tuple(v_cache.shape) != (Hkv, L, D):
        raise ValueError("v_cache must have the shape of k_cache")
    _out(k_part, "k_part", (Hkv, k * chunk, D), k_cache.dtype, dev)
    _out(v_part, "v_part", (Hkv, k * chunk, D), k_cache.dtype, dev)
    if k_part is None:
        k_part = torch.empty((Hkv, k * chunk, D), dtype=k_cache.dtype, device=dev)
    if v_part is None:
        v_part = torch.empty((Hkv, k * chunk, D), dtype=k_cache.dtype, device=dev)
    _check(lib().ts_kv_gather(k_cache.data_ptr(), v_cache.data_ptr(), stride, chunk_idx.data_ptr(),
                              Hkv, k, chunk, D, L, k_part.data_ptr(), v_part.data_ptr(),
                              _dtype_code(k_cache), _stream(dev)))
    return k_part, v_part


def kv_gather_and_draft_attn(k_cache, v_cache, chunk_idx, chunk: int, q, k_new, v_new, *, scale=None,
                             k_part=None, v_part=None, out=None, lse=None, want_lse=True, num_splits: int = 0,
                             workspace=None):
    """ts_kv_gather_and_draft_attn: kv_gather(k_cache, v_cache, chunk_idx, chunk)
    then partial_draft_attn(q, k_part, v_part, k_new, v_new) in one pass where
    possible -> (k_part, v_part, out, lse), bit-identical to the two calls."""
    _need(k_cache, "k_cache", 3)
    dev = k_cache.device
    _need(v_cache, "v_cache", 3, k_cache.dtype, dev)
    _need(chunk_idx, "chunk_idx", 2, torch.int32, dev)
    _contig(chunk_idx, "chunk_idx")
    Hkv, L, D = k_cache.shape
    k = chunk_idx.shape[1]
    if chunk_idx.shape[0] != Hkv:
        raise ValueError(f"chunk_idx must be [{Hkv}][k]")
    stride = _cache_stride(k_cache, "k_cache")
    if _cache_stride(v_cache, "v_cache") != stride:
        raise ValueError("k_cache and v_cache must share the row stride")
    if tuple(v_cache.shape) != (Hkv, L, D):
        raise ValueError("v_cache must have the shape of k_cache")
    _need(q, "q", 3, k_cache.dtype, dev)
    _contig(q, "q")
    Tq, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q and the cache differ in head dim")
    for n, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t, n, 3, q.dtype, dev)
        _contig(t, n)
        if tuple(t.shape) != (Hkv, Tq, D):
            raise ValueError(f"{n} must be [{Hkv}][{Tq}][{D}]")
    P = k * chunk
    code = _dtype_code(q)
    _out(k_part, "k_part", (Hkv, P, D), q.dtype, dev)
    _out(v_part, "v_part", (Hkv, P, D), q.dtype, dev)
    _out(out, "out", (Tq, Hq, D), q.dtype, dev)
    _out(lse, "lse", (Tq, Hq), torch.float32, dev)
    if k_part is None:
        k_part = torch.empty((Hkv, P, D), dtype=q.dtype, device=dev)
    if v_part is None:
        v_part = torch.empty((Hkv, P, D), dtype=q.dtype, device=dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((Tq, Hq), dtype=torch.float32, device=dev)
    need = int(lib().ts_partial_draft_attn_workspace(Tq, Hq, Hkv, D, P, code, num_splits))
    if need == 0:
        raise TsError(TS_ERR_INVALID_ARG, lib().ts_last_error().decode())
    _workspace(workspace, "workspace", need, dev)
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    _check(lib().ts_kv_gather_and_draft_attn(
        k_cache.data_ptr(), v_cache.data_ptr(), stride, chunk_idx.data_ptr(), k, chunk, L, k_part.data_ptr(),
        v_part.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, Tq, Hq, Hkv, D,
        float(1.0 / math.sqrt(D) if scale is None else scale), code, num_splits, workspace.data_ptr(),
        _nbytes(workspace), _stream(dev)))
    return k_part, v_part, out, lse


def draft_tree_nodes(shape) -> int:
    """ts_draft_tree_nodes: node count of a tree shape [k_0, k_1, ...]."""
    arr = (ctypes.c_int32 * len(shape))(*[int(k) for k in shape])
    n = lib().ts_draft_tree_nodes(ctypes.cast(arr, ctypes.c_void_p), len(shape))
    if n < 0:
        raise TsError(TS_ERR_UNSUPPORTED, lib().ts_last_error().decode())
    return int(n)


def build_draft_tree(logits, shape, *, parent=None, draft_tok=None, cand=None, workspace=None):
    """ts_build_draft_tree -> (parent [T], draft_tok [T], cand [depth][16]) int32 device tensors.

    logits: [P][V] float32 or bfloat16 on the device; shape: host list of k_d."""
    _need(logits, "logits", 2)
    _contig(logits, "logits")
    dev = logits.device
    P, V = logits.shape
    T = draft_tree_nodes(shape)
    _out(parent, "parent", (T,), torch.int32, dev)
    _out(draft_tok, "draft_tok", (T,), torch.int32, dev)
    _out(cand, "cand", (len(shape), 16), torch.int32, dev)
    need = int(lib().ts_build_draft_tree_workspace(V, len(shape)))
    _workspace(workspace, "workspace", need, dev)
    if parent is None:
        parent = torch.empty(T, dtype=torch.int32, device=dev)
    if draft_tok is None:
        draft_tok = torch.empty(T, dtype=torch.int32, device=dev)
    if cand is None:
        cand = torch.empty((len(shape), 16), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    arr = (ctypes.c_int32 * len(shape))(*[int(k) for k in shape])
    _check(lib().ts_build_draft_tree(logits.data_ptr(), P, V, ctypes.cast(arr, ctypes.c_void_p), len(shape),
                                     parent.data_ptr(), draft_tok.data_ptr(), cand.data_ptr(),
                                     _dtype_code(logits), workspace.data_ptr(), _nbytes(workspace),
                                     _stream(dev)))
    return parent, draft_tok, cand


def accept_commit(parent, draft_tok, target_tok, rand_u32: int, k_cache, v_cache, L: int,
                  k_draft, v_draft, *, n_accepted=None, path=None, bonus=None):
    """ts_accept_commit -> (n_accepted [1], path [T], bonus [1]) int32 device tensors.

    k_cache, v_cache: [Hkv][capacity][D] (rows L .. L+n-1 are written in place;
    capacity >= L + T); k_draft, v_draft: [Hkv][T][D]; parent, draft_tok [T],
    target_tok [T+1] int32 on the device."""
    dev = k_cache.device
    for n, t, dims in (("parent", parent, 1), ("draft_tok", draft_tok, 1), ("target_tok", target_tok, 1)):
        _need(t, n, dims, torch.int32, dev)
        _contig(t, n)
    _need(k_cache, "k_cache", 3)
    _need(v_cache, "v_cache", 3, k_cache.dtype, dev)
    for n, t in (("k_draft", k_draft), ("v_draft", v_draft)):
        _need(t, n, 3, k_cache.dtype, dev)
        _contig(t, n)
    T = parent.shape[0]
    if draft_tok.shape[0] != T or target_tok.shape[0] != T + 1:
        raise ValueError("draft_tok must have T entries and target_tok T+1")
    Hkv, cap, D = k_cache.shape
    if k_draft.shape != (Hkv, T, D) or v_draft.shape != (Hkv, T, D):
        raise ValueError("k_draft / v_draft must be [Hkv][T][D]")
    stride = _cache_stride(k_cache, "k_cache")
    if _cache_stride(v_cache, "v_cache") != stride:
        raise ValueError("k_cache and v_cache must share the row stride")
    if cap < L + T:
        raise ValueError(f"cache capacity {cap} < L + T = {L + T}")
    if tuple(v_cache.shape) != (Hkv, cap, D):
        raise ValueError("v_cache must have the shape of k_cache")
    _out(n_accepted, "n_accepted", (1,), torch.int32, dev)
    _out(path, "path", (T,), torch.int32, dev)
    _out(bonus, "bonus", (1,), torch.int32, dev)
    if n_accepted is None:
        n_accepted = torch.empty(1, dtype=torch.int32, device=dev)
    if path is None:
        path = torch.empty(T, dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib().ts_accept_commit(parent.data_ptr(), draft_tok.data_ptr(), target_tok.data_ptr(),
                                  int(rand_u32) & 0xFFFFFFFF, T, k_cache.data_ptr(), v_cache.data_ptr(),
                                  stride, int(L), k_draft.data_ptr(), v_draft.data_ptr(), Hkv, D,
                                  _dtype_code(k_cache), n_accepted.data_ptr(), path.data_ptr(),
                                  bonus.data_ptr(), _stream(dev)))
    return n_accepted, path, bonus


def sample_tokens(logits, *, hist=None, parent=None, draft_tok=None, window: int = 1024,
                  penalty: float = 1.2, temperature: float = 1.0, min_p: float = 0.1, top_p: float = 1.0,
                  u=None, tok=None, workspace=None):
    """ts_sample_tokens -> tok [R] int32: the target's token for each of the
    R = T + 1 verified positions of logits [R][V] (row 0 after the committed
    context, row t+1 after draft t), with the windowed repetition penalty,
    temperature, min-p, top-p and the caller's uniforms u [R] (fp32, device)."""
    _need(logits, "logits", 2)
    _contig(logits, "logits")
    dev = logits.device
    R, V = logits.shape
    T = 0
    if parent is not None or draft_tok is not None:
        for n, t in (("parent", parent), ("draft_tok", draft_tok)):
            _need(t, n, 1, torch.int32, dev)
            _contig(t, n)
        T = parent.shape[0]
        if draft_tok.shape[0] != T:
            raise ValueError("parent and draft_tok must have T entries")
    n_hist = 0
    if hist is not None:
        _need(hist, "hist", 1, torch.int32, dev)
        _contig(hist, "hist")
        n_hist = hist.shape[0]
    if temperature > 0:
        _need(u, "u", 1, torch.float32, dev)
        _contig(u, "u")
        if u.shape[0] != R:
            raise ValueError("u must have one uniform per row")
    _out(tok, "tok", (R,), torch.int32, dev)
    need = int(lib().ts_sample_workspace(R, V))
    _workspace(workspace, "workspace", need, dev)
    if tok is None:
        tok = torch.empty(R, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    ptr = lambda t: t.data_ptr() if t is not None and t.numel() else None
    _check(lib().ts_sample_tokens(logits.data_ptr(), R, V, ptr(hist), n_hist, ptr(parent), ptr(draft_tok), T,
                                  int(window), float(penalty), float(temperature), float(min_p), float(top_p),
                                  ptr(u) if temperature > 0 else None, tok.data_ptr(), _dtype_code(logits),
                                  workspace.data_ptr(), _nbytes(workspace), _stream(dev)))
    return tok


class NgramTable:
    """The 4-gram table of the committed text (ts_ngram_*), in one device buffer.

    update(tokens, start, end) adds the 4-grams ending at positions start..end-1
    of the committed text `tokens` (int32, device); retrieve(first_tok, k) gives
    the k 4-grams starting with the device int32 first_tok[0], ranked by count
    then recency."""

    def __init__(self, device, capacity_log2: int = 18, max_entries: int = 131072):
        nbytes = int(lib().ts_ngram_table_bytes(capacity_log2, max_entries))
        if nbytes == 0:
            raise TsError(TS_ERR_UNSUPPORTED, f"capacity_log2={capacity_log2} max_entries={max_entries}")
        self.device = torch.device(device)
        self.capacity_log2, self.max_entries = capacity_log2, max_entries
        self.buf = alloc_workspace(nbytes, self.device)
        self.reset()

    def reset(self):
        _check(lib().ts_ngram_init(self.buf.data_ptr(), self.buf.numel(), self.capacity_log2, self.max_entries,
                                   _stream(self.device)))

    def update(self, tokens, start: int, end: int):
        _need(tokens, "tokens", 1, torch.int32, self.device)
        _contig(tokens, "tokens")
        if end > tokens.shape[0]:
            raise ValueError(f"end={end} past the {tokens.shape[0]} tokens")
        _check(lib().ts_ngram_update(self.buf.data_ptr(), tokens.data_ptr(), int(start), int(end),
                                     _stream(self.device)))

    def retrieve(self, first_tok, k: int = 20, *, out_tok=None, out_count=None, n_found=None, workspace=None):
        _need(first_tok, "first_tok", 1, torch.int32, self.device)
        dev = self.device
        _out(out_tok, "out_tok", (k, 4), torch.int32, dev)
        _out(out_count, "out_count", (k,), torch.int32, dev)
        _out(n_found, "n_found", (1,), torch.int32, dev)
        need = int(lib().ts_ngram_retrieve_workspace(self.max_entries, k))
        _workspace(workspace, "workspace", need, dev)
        if out_tok is None:
            out_tok = torch.empty((k, 4), dtype=torch.int32, device=dev)
        if out_count is None:
            out_count = torch.empty(k, dtype=torch.int32, device=dev)
        if n_found is None:
            n_found = torch.empty(1, dtype=torch.int32, device=dev)
        if workspace is None:
            workspace = alloc_workspace(need, dev)
        _check(lib().ts_ngram_retrieve(self.buf.data_ptr(), self.max_entries, first_tok.data_ptr(), int(k),
                                       out_tok.data_ptr(), out_count.data_ptr(), n_found.data_ptr(),
                                       workspace.data_ptr(), _nbytes(workspace), _stream(dev)))
        return out_tok, out_count, n_found

    def header(self) -> dict:
        """The table's header (synchronises the stream)."""
        h = self.buf[:16].view(torch.int32).cpu().tolist()
        return dict(capacity_log2=h[0], max_entries=h[1], n_entries=h[2], dropped=h[3])


def partial_draft_attn(q, k_part, v_part, k_new, v_new, *, scale=None, out=None, lse=None,
                       want_lse=True, num_splits: int = 0, workspace=None):
    """ts_partial_draft_attn: q [Tq][Hq][D] over partial cache [Hkv][P][D] plus
    the Tq new tokens [Hkv][Tq][D] under a causal chain."""
    _need(q, "q", 3)
    dev = q.device
    Tq, Hq, D = q.shape
    for n, t in (("k_part", k_part), ("v_part", v_part), ("k_new", k_new), ("v_new", v_new)):
        _need(t, n, 3, q.dtype, dev)
        _contig(t, n)
    _contig(q, "q")
    Hkv, P, Dk = k_part.shape
    if Dk != D or tuple(v_part.shape) != (Hkv, P, D):
        raise ValueError("partial cache shapes do not match q")
    if tuple(k_new.shape) != (Hkv, Tq, D) or tuple(v_new.shape) != (Hkv, Tq, D):
        raise ValueError(f"k_new / v_new must be [{Hkv}][{Tq}][{D}]")
    code = _dtype_code(q)
    _out(out, "out", (Tq, Hq, D), q.dtype, dev)
    _out(lse, "lse", (Tq, Hq), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((Tq, Hq), dtype=torch.float32, device=dev)
    need = int(lib().ts_partial_draft_attn_workspace(Tq, Hq, Hkv, D, P, code, num_splits))
    if need == 0:
        raise TsError(TS_ERR_INVALID_ARG, lib().ts_last_error().decode())
    _workspace(workspace, "workspace", need, dev)
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    _check(lib().ts_partial_draft_attn(
        q.data_ptr(), k_part.data_ptr(), v_part.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
        out.data_ptr(), lse.data_ptr() if lse is not None else None, Tq, Hq, Hkv, D, P,
        float(1.0 / math.sqrt(D) if scale is None else scale), code, num_splits,
        workspace.data_ptr(), _nbytes(workspace), _stream(dev)))
    return out, lse
