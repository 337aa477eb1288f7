"""Python binding of the MI355X fused exact-attention library (``libfa_mi355x.so``).

Argument marshalling only: every step of the computation runs in the HIP kernels
behind the C ABI declared in ``include/fa.h``.  PyTorch provides device memory and
the current stream.  There is no fallback: if the library is missing or a call is
rejected, a ``RuntimeError`` is raised.

The functions carry the C entry points' names:

    o, lse = fa_fwd(q, k, v, causal=False, softmax_scale=None)
    dq, dk, dv = fa_bwd(q, k, v, o, do, lse, causal=False, softmax_scale=None)

q: (B, Hq, N, D), k and v: (B, Hkv, N, D), contiguous CUDA(HIP) tensors of dtype
torch.float16 or torch.bfloat16 (or torch.float32 for the fp32 verification path of
fa_fwd and fa_bwd), D in {64, 128}, Hq a multiple of Hkv.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

__all__ = [
    "fa_fwd", "fa_fwd_splitkv", "fa_fwd_splitkv_parts", "fa_fwd_splitkv_workspace_size",
    "fa_merge_partials", "fa_bwd", "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq", "fa_bwd_postprocess",
    "fa_bwd_workspace_size", "fa_version", "fa_status_string", "library_path", "load_library",
    "EXPORTED_SYMBOLS", "FA_FP16", "FA_BF16", "FA_FP32",
]

FA_FP16 = 0
FA_BF16 = 1
FA_FP32 = 2
_LIB_NAME = "libfa_mi355x.so"
_lock = threading.Lock()
_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_SIGS = {
    "fa_version": ([], ctypes.c_int),
    "fa_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "fa_fwd": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_float,
                ctypes.c_int, ctypes.c_int, _vp], ctypes.c_int),
    "fa_fwd_splitkv_parts": ([_i64, _i64, _i64, _i64, _i64, ctypes.c_int], ctypes.c_int),
    "fa_fwd_splitkv_workspace_size": ([_i64, _i64, _i64, _i64, _i64, ctypes.c_int], ctypes.c_size_t),
    "fa_fwd_splitkv": ([_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, ctypes.c_int,
                        _i64, _i64, _i64, _i64, _i64, ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp],
                       ctypes.c_int),
    "fa_merge_partials": ([_vp, _vp, ctypes.c_int, _vp, _vp, _i64, _i64, ctypes.c_int, _vp], ctypes.c_int),
    "fa_bwd_workspace_size": ([_i64, _i64, _i64, _i64, _i64], ctypes.c_size_t),
    "fa_bwd": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                _i64, _i64, _i64, _i64, _i64, ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp],
               ctypes.c_int),
    "fa_bwd_preprocess": ([_vp, _vp, _vp, _vp, ctypes.c_size_t, _i64, _i64, _i64, _i64, _i64,
                           ctypes.c_int, _vp], ctypes.c_int),
    "fa_bwd_dkdv": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                     _i64, _i64, _i64, _i64, _i64, ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp],
                    ctypes.c_int),
    "fa_bwd_dq": ([_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                   _i64, _i64, _i64, _i64, _i64, ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp],
                  ctypes.c_int),
    "fa_bwd_postprocess": ([_vp, _vp, _vp, ctypes.c_size_t, _i64, _i64, _i64, _i64, _i64,
                            ctypes.c_int, _vp], ctypes.c_int),
}
EXPORTED_SYMBOLS = tuple(_SIGS)


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), _LIB_NAME)


def load_library():
    """Load (once) and return the ctypes handle; raises if the library is not built."""
    global _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build it with `python -m exact_attention_fa_amd._build` "
                    "(or __graft_entry__.build()); there is no non-HIP fallback")
            lib = ctypes.CDLL(path)
            for name, (args, res) in _SIGS.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = res
            _lib = lib
    return _lib


def fa_version() -> int:
    return load_library().fa_version()


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(status).decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed: {fa_status_string(rc)} (status {rc})")


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return FA_FP16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_FP32  # the fp32 verification path (fa_fwd, fa_bwd and its stages)
    raise RuntimeError(f"unsupported dtype {t.dtype}: float16, bfloat16 or float32 only")


def _dims(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise RuntimeError("q, k, v must be 4-D (B, H, N, D)")
    B, Hq, N, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise RuntimeError("k and v must be (B, Hkv, N, D) with the B, N, D of q")
    return B, Hq, k.shape[1], N, D


def _require(*tensors, dtype=None):
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise RuntimeError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise RuntimeError("tensors must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise RuntimeError(f"dtype mismatch: expected {dtype}, got {t.dtype}")


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _nbytes(t):
    return t.numel() * t.element_size()


def _scale(D, softmax_scale):
    return 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)


def fa_fwd(q, k, v, causal: bool = False, softmax_scale=None, out=None, lse=None):
    """Forward: returns (o, lse); o like q, lse float32 (B, Hq, N) in natural-log units."""
    import torch
    B, Hq, Hkv, N, D = _dims(q, k, v)
    _require(q, k, v, dtype=q.dtype)
    code = _dtype_code(q)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _require(o, dtype=q.dtype)
    _require(l, dtype=torch.float32)
    rc = load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, Hq, Hkv, N, D,
                               _scale(D, softmax_scale), int(bool(causal)), code, _stream(q))
    _check(rc, "fa_fwd")
    return o, l


def fa_fwd_splitkv_parts(B, Hq, Hkv, N, D, causal: bool = False) -> int:
    """The library's choice of key-range pieces for fa_fwd_splitkv (1: no split)."""
    return int(load_library().fa_fwd_splitkv_parts(B, Hq, Hkv, N, D, int(bool(causal))))


def fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, D, n_split: int) -> int:
    return int(load_library().fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, D, int(n_split)))


def fa_fwd_splitkv(q, k, v, causal: bool = False, softmax_scale=None, n_split: int = 0, workspace=None,
                   out=None, lse=None):
    """Forward over n_split key-range pieces merged through their LSEs (0: the library's
    choice); returns (o, lse) like fa_fwd."""
    import torch
    B, Hq, Hkv, N, D = _dims(q, k, v)
    _require(q, k, v, dtype=q.dtype)
    code = _dtype_code(q)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _require(o, dtype=q.dtype)
    _require(l, dtype=torch.float32)
    n = fa_fwd_splitkv_parts(B, Hq, Hkv, N, D, causal) if n_split == 0 else int(n_split)
    if workspace is None and 1 <= n <= 64:
        need = fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, D, n)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    nbytes = 0 if workspace is None else _nbytes(workspace)
    rc = load_library().fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), _ptr(workspace), nbytes,
                                       int(n_split), B, Hq, Hkv, N, D, _scale(D, softmax_scale),
                                       int(bool(causal)), code, _stream(q))
    _check(rc, "fa_fwd_splitkv")
    return o, l


def fa_merge_partials(o_parts, lse_parts, out, lse):
    """Merge fp32 partial results over disjoint key sets: o_parts (n, rows, D), lse_parts
    (n, rows) -> out (rows, D) in out's dtype, lse (rows,) float32 (any shapes with these
    element counts)."""
    import torch
    n = lse_parts.shape[0]
    rows = lse_parts.numel() // n
    D = o_parts.numel() // (n * rows)
    _require(o_parts, lse_parts, dtype=torch.float32)
    _require(out)
    _require(lse, dtype=torch.float32)
    rc = load_library().fa_merge_partials(_ptr(o_parts), _ptr(lse_parts), n, _ptr(out), _ptr(lse), rows, D,
                                          _dtype_code(out), _stream(out))
    _check(rc, "fa_merge_partials")


def fa_bwd_workspace_size(B, Hq, Hkv, N, D) -> int:
    return int(load_library().fa_bwd_workspace_size(B, Hq, Hkv, N, D))


def _workspace(q, shape, workspace):
    import torch
    need = fa_bwd_workspace_size(*shape)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    return workspace, workspace.numel() * workspace.element_size()


def fa_bwd(q, k, v, o, do, lse, causal: bool = False, softmax_scale=None, workspace=None,
           dq=None, dk=None, dv=None):
    """Backward: returns (dq, dk, dv) in the dtype of q."""
    import torch
    B, Hq, Hkv, N, D = _dims(q, k, v)
    _require(q, k, v, o, do, dtype=q.dtype)
    _require(lse, dtype=torch.float32)
    code = _dtype_code(q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _require(dq, dk, dv, dtype=q.dtype)
    ws, nbytes = _workspace(q, (B, Hq, Hkv, N, D), workspace)
    rc = load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                               _ptr(dk), _ptr(dv), _ptr(ws), nbytes, B, Hq, Hkv, N, D,
                               _scale(D, softmax_scale), int(bool(causal)), code, _stream(q))
    _check(rc, "fa_bwd")
    return dq, dk, dv


def fa_bwd_preprocess(o, do, lse, workspace, Hkv: int):
    B, Hq, N, D = o.shape
    _require(o, do, dtype=o.dtype)
    rc = load_library().fa_bwd_preprocess(_ptr(o), _ptr(do), _ptr(lse), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          B, Hq, Hkv, N, D, _dtype_code(o), _stream(o))
    _check(rc, "fa_bwd_preprocess")


def fa_bwd_dkdv(q, k, v, do, dk, dv, workspace, causal=False, softmax_scale=None):
    B, Hq, Hkv, N, D = _dims(q, k, v)
    rc = load_library().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dk), _ptr(dv),
                                    _ptr(workspace), _nbytes(workspace), B, Hq, Hkv, N, D,
                                    _scale(D, softmax_scale), int(bool(causal)), _dtype_code(q),
                                    _stream(q))
    _check(rc, "fa_bwd_dkdv")


def fa_bwd_dq(q, k, v, do, dq, workspace, causal=False, softmax_scale=None):
    B, Hq, Hkv, N, D = _dims(q, k, v)
    rc = load_library().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(workspace),
                                  _nbytes(workspace), B, Hq, Hkv, N, D, _scale(D, softmax_scale),
                                  int(bool(causal)), _dtype_code(q), _stream(q))
    _check(rc, "fa_bwd_dq")


def fa_bwd_postprocess(dk, dv, workspace, Hq: int):
    B, Hkv, N, D = dk.shape
    rc = load_library().fa_bwd_postprocess(_ptr(dk), _ptr(dv), _ptr(workspace), _nbytes(workspace),
                                           B, Hq, Hkv, N, D, _dtype_code(dk), _stream(dk))
    _check(rc, "fa_bwd_postprocess")
