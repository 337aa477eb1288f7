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
    "fa_merge_partials", "fa_bwd", "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq", "fa_bwd_dq_rows",
    "fa_bwd_postprocess", "fa_bwd_plan", "FA_BWD_PLAN_STAGES", "FA_BWD_PLAN_ROWS",
    "fa_bwd_workspace_size", "fa_version", "fa_status_string", "library_path", "load_library",
    "EXPORTED_SYMBOLS", "FA_FP16", "FA_BF16", "FA_FP32", "fa_bwd_noalloc", "FA_NOALLOC_SCRATCH_BYTES",
]

FA_FP16 = 0
FA_BF16 = 1
FA_FP32 = 2
FA_BWD_PLAN_STAGES = 0  # fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq, fa_bwd_postprocess
FA_BWD_PLAN_ROWS = 1    # fa_bwd_dq_rows, fa_bwd_dkdv
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
    "fa_bwd_dq_rows": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                        _i64, _i64, _i64, _i64, _i64, ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp],
                       ctypes.c_int),
    "fa_bwd_plan": ([_i64, _i64, _i64, _i64, _i64, ctypes.c_int], ctypes.c_int),
    "fa_bwd_postprocess": ([_vp, _vp, _vp, ctypes.c_size_t, _i64, _i64, _i64, _i64, _i64,
                            ctypes.c_int, _vp], ctypes.c_int),
    "fa_bwd_noalloc": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                        _i64, _i64, _i64, _i64, _i64, ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp],
                       ctypes.c_int),
}
FA_NOALLOC_SCRATCH_BYTES = 80 * 1024 * 1024  # the library's static backward workspace per GPU
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
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is None or t.dim() != 4:
            raise RuntimeError(f"{name} must be a 4-D tensor (B, H, N, D)")
    B, Hq, N, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise RuntimeError("k and v must be (B, Hkv, N, D) with the B, N, D of q")
    return B, Hq, k.shape[1], N, D


def _validate(*specs):
    """Checks tensor arguments before anything reaches the library: first the shape and dtype
    of every one, then device and contiguity.  The C ABI sees only pointers, so a wrongly
    shaped, typed, strided or host tensor would otherwise be read or written out of bounds.
    Each spec is (tensor, name, shape or None, numel or None, dtype or None); all tensors must
    share the first one's device."""
    # (kept cheap: a latency-bound call spends more time here than in its kernels)
    for t, name, shape, numel, dtype in specs:
        if t is None:
            raise RuntimeError(f"{name} is required")
        if shape is not None and t.shape != tuple(shape):
            raise RuntimeError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if numel is not None and t.numel() != numel:
            raise RuntimeError(f"{name} has {t.numel()} elements, expected {numel}")
        if dtype is not None and t.dtype != dtype:
            raise RuntimeError(f"{name}: dtype mismatch, expected {dtype}, got {t.dtype}")
    index = specs[0][0].get_device()
    for t, name, *_ in specs:
        if not t.is_cuda:
            raise RuntimeError(f"{name} must live on the GPU")
        if t.get_device() != index:
            raise RuntimeError(f"{name} is on {t.device}, expected {specs[0][0].device}")
        if not t.is_contiguous():
            raise RuntimeError(f"{name} must be contiguous")


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _nbytes(t):
    return t.numel() * t.element_size()


def _scale(D, softmax_scale):
    return 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)


def _qkv_specs(q, k, v):
    return [(q, "q", None, None, q.dtype), (k, "k", None, None, q.dtype), (v, "v", None, None, q.dtype)]


def fa_fwd(q, k, v, causal: bool = False, softmax_scale=None, out=None, lse=None):
    """Forward: returns (o, lse); o like q, lse float32 (B, Hq, N) in natural-log units."""
    import torch
    B, Hq, Hkv, N, D = _dims(q, k, v)
    code = _dtype_code(q)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _validate(*_qkv_specs(q, k, v), (o, "out", q.shape, None, q.dtype), (l, "lse", (B, Hq, N), None, torch.float32))
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
    code = _dtype_code(q)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _validate(*_qkv_specs(q, k, v), (o, "out", q.shape, None, q.dtype), (l, "lse", (B, Hq, N), None, torch.float32))
    n = fa_fwd_splitkv_parts(B, Hq, Hkv, N, D, causal) if n_split == 0 else int(n_split)
    if workspace is None and 1 <= n <= 64:
        need = fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, D, n)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    if workspace is not None:
        _validate((q, "q", None, None, None), (workspace, "workspace", None, None, None))
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
    if lse_parts.dim() < 1 or lse_parts.numel() == 0:
        raise RuntimeError("lse_parts must be (n_parts, rows)")
    n = lse_parts.shape[0]
    rows = lse_parts.numel() // n
    if o_parts.numel() % (n * rows) != 0:
        raise RuntimeError("o_parts must hold n_parts * rows * D elements")
    D = o_parts.numel() // (n * rows)
    _validate((o_parts, "o_parts", None, None, torch.float32), (lse_parts, "lse_parts", None, n * rows, torch.float32),
              (out, "out", None, rows * D, None), (lse, "lse", None, rows, torch.float32))
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
    code = _dtype_code(q)
    specs = [*_qkv_specs(q, k, v), (o, "o", q.shape, None, q.dtype), (do, "do", q.shape, None, q.dtype),
             (lse, "lse", (B, Hq, N), None, torch.float32)]
    for t, name, shape in ((dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", k.shape), (workspace, "workspace", None)):
        if t is not None:
            specs.append((t, name, shape, None, None if name == "workspace" else q.dtype))
    _validate(*specs)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws, nbytes = _workspace(q, (B, Hq, Hkv, N, D), workspace)
    rc = load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                               _ptr(dk), _ptr(dv), _ptr(ws), nbytes, B, Hq, Hkv, N, D,
                               _scale(D, softmax_scale), int(bool(causal)), code, _stream(q))
    _check(rc, "fa_bwd")
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, do, lse, causal: bool = False, softmax_scale=None, dq=None, dk=None, dv=None):
    """fa_bwd with the library's static scratch as workspace (the C entry point allocates
    nothing; outputs not given are allocated here by torch).  Returns (dq, dk, dv)."""
    import torch
    B, Hq, Hkv, N, D = _dims(q, k, v)
    code = _dtype_code(q)
    specs = [*_qkv_specs(q, k, v), (o, "o", q.shape, None, q.dtype), (do, "do", q.shape, None, q.dtype),
             (lse, "lse", (B, Hq, N), None, torch.float32)]
    specs += [(t, name, shape, None, q.dtype) for t, name, shape in ((dq, "dq", q.shape), (dk, "dk", k.shape),
                                                                     (dv, "dv", k.shape)) if t is not None]
    _validate(*specs)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    rc = load_library().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                                       _ptr(dk), _ptr(dv), B, Hq, Hkv, N, D, _scale(D, softmax_scale),
                                       int(bool(causal)), code, _stream(q))
    _check(rc, "fa_bwd_noalloc")
    return dq, dk, dv


def fa_bwd_preprocess(o, do, lse, workspace, Hkv: int):
    import torch
    if o is None or o.dim() != 4:
        raise RuntimeError("o must be a 4-D tensor (B, Hq, N, D)")
    B, Hq, N, D = o.shape
    _dtype_code(o)
    _validate((o, "o", None, None, o.dtype), (do, "do", o.shape, None, o.dtype),
              (lse, "lse", (B, Hq, N), None, torch.float32), (workspace, "workspace", None, None, None))
    rc = load_library().fa_bwd_preprocess(_ptr(o), _ptr(do), _ptr(lse), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          B, Hq, Hkv, N, D, _dtype_code(o), _stream(o))
    _check(rc, "fa_bwd_preprocess")


def fa_bwd_dkdv(q, k, v, do, dk, dv, workspace, causal=False, softmax_scale=None):
    """dk/dv may be None where the pass writes partials into the workspace (Hq > Hkv, or
    query-range pieces); the library then does not touch them."""
    B, Hq, Hkv, N, D = _dims(q, k, v)
    _dtype_code(q)
    specs = [*_qkv_specs(q, k, v), (do, "do", q.shape, None, q.dtype), (workspace, "workspace", None, None, None)]
    specs += [(x, name, k.shape, None, q.dtype) for x, name in ((dk, "dk"), (dv, "dv")) if x is not None]
    _validate(*specs)
    rc = load_library().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dk), _ptr(dv),
                                    _ptr(workspace), _nbytes(workspace), B, Hq, Hkv, N, D,
                                    _scale(D, softmax_scale), int(bool(causal)), _dtype_code(q),
                                    _stream(q))
    _check(rc, "fa_bwd_dkdv")


def fa_bwd_dq(q, k, v, do, dq, workspace, causal=False, softmax_scale=None):
    B, Hq, Hkv, N, D = _dims(q, k, v)
    _dtype_code(q)
    _validate(*_qkv_specs(q, k, v), (do, "do", q.shape, None, q.dtype), (dq, "dq", q.shape, None, q.dtype),
              (workspace, "workspace", None, None, None))
    rc = load_library().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(workspace),
                                  _nbytes(workspace), B, Hq, Hkv, N, D, _scale(D, softmax_scale),
                                  int(bool(causal)), _dtype_code(q), _stream(q))
    _check(rc, "fa_bwd_dq")


def fa_bwd_dq_rows(q, k, v, o, do, lse, dq, workspace, causal=False, softmax_scale=None):
    """fa_bwd_preprocess and fa_bwd_dq as one pass (the row values are formed where the dQ pass
    holds each row, and stored in the workspace for fa_bwd_dkdv)."""
    import torch
    B, Hq, Hkv, N, D = _dims(q, k, v)
    _dtype_code(q)
    _validate(*_qkv_specs(q, k, v), (o, "o", q.shape, None, q.dtype), (do, "do", q.shape, None, q.dtype),
              (lse, "lse", (B, Hq, N), None, torch.float32), (dq, "dq", q.shape, None, q.dtype),
              (workspace, "workspace", None, None, None))
    rc = load_library().fa_bwd_dq_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                                       _ptr(workspace), _nbytes(workspace), B, Hq, Hkv, N, D,
                                       _scale(D, softmax_scale), int(bool(causal)), _dtype_code(q), _stream(q))
    _check(rc, "fa_bwd_dq_rows")


def fa_bwd_plan(B: int, Hq: int, Hkv: int, N: int, D: int, dtype: int) -> int:
    """The stage order fa_bwd enqueues: FA_BWD_PLAN_ROWS (fa_bwd_dq_rows, fa_bwd_dkdv) or
    FA_BWD_PLAN_STAGES (fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq, fa_bwd_postprocess)."""
    rc = load_library().fa_bwd_plan(B, Hq, Hkv, N, D, dtype)
    if rc < 0:
        _check(-rc, "fa_bwd_plan")
    return rc


def fa_bwd_postprocess(dk, dv, workspace, Hq: int):
    if dk is None or dk.dim() != 4:
        raise RuntimeError("dk must be a 4-D tensor (B, Hkv, N, D)")
    B, Hkv, N, D = dk.shape
    _dtype_code(dk)
    _validate((dk, "dk", None, None, dk.dtype), (dv, "dv", dk.shape, None, dk.dtype),
              (workspace, "workspace", None, None, None))
    rc = load_library().fa_bwd_postprocess(_ptr(dk), _ptr(dv), _ptr(workspace), _nbytes(workspace),
                                           B, Hq, Hkv, N, D, _dtype_code(dk), _stream(dk))
    _check(rc, "fa_bwd_postprocess")
