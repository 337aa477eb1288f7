"""C-ABI checks that need no GPU: the library loads, exports what include/fa.h declares,
and rejects invalid calls with the documented status before touching the device."""
import ctypes
import os
import re

import pytest

import exact_attention_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

STATUS = {
    "FA_OK": 0, "FA_ERR_NULL_POINTER": 1, "FA_ERR_BAD_SHAPE": 2, "FA_ERR_HEAD_DIM": 3,
    "FA_ERR_GQA": 4, "FA_ERR_DTYPE": 5, "FA_ERR_SCALE": 6, "FA_ERR_ALIGNMENT": 7,
    "FA_ERR_WORKSPACE": 8, "FA_ERR_HIP": 9, "FA_ERR_TOO_LARGE": 10, "FA_ERR_ALIAS": 11,
    "FA_ERR_SPLIT": 12, "FA_ERR_SCRATCH": 13,
}

# Fake, aligned, non-null "device" addresses: every call below fails validation before any
# HIP call, so they are never dereferenced.
A = 1 << 32
MB = 1 << 20


def ptr(i):
    return ctypes.c_void_p(A + i * 64 * 1024 * MB)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        pytest.fail("libfa_mi355x.so is not built (run __graft_entry__.build())")
    return fa.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\*?\s*(fa_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_entry_points():
    names = declared_functions()
    assert set(names) == set(fa.EXPORTED_SYMBOLS), names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {fa.library_path()}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_header_status_values_match():
    text = open(HEADER).read()
    for name, val in STATUS.items():
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name


def test_version_and_strings(lib):
    assert fa.fa_version() == 10100
    for code in range(14):
        s = fa.fa_status_string(code)
        assert s and s != "unknown status"
    assert fa.fa_status_string(999) == "unknown status"


def fwd(lib, q=0, k=1, v=2, o=3, l=4, B=1, Hq=2, Hkv=2, N=256, D=64, scale=0.125, causal=0, dtype=0):
    P = lambda x: x if isinstance(x, ctypes.c_void_p) else ptr(x)
    return lib.fa_fwd(P(q), P(k), P(v), P(o), P(l), B, Hq, Hkv, N, D, scale, causal, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), "FA_ERR_DTYPE"),
    (dict(dtype=-1), "FA_ERR_DTYPE"),
    (dict(B=0), "FA_ERR_BAD_SHAPE"),
    (dict(Hq=0), "FA_ERR_BAD_SHAPE"),
    (dict(Hkv=-1), "FA_ERR_BAD_SHAPE"),
    (dict(N=0), "FA_ERR_BAD_SHAPE"),
    (dict(D=32), "FA_ERR_HEAD_DIM"),
    (dict(D=96), "FA_ERR_HEAD_DIM"),
    (dict(D=256), "FA_ERR_HEAD_DIM"),
    (dict(Hq=6, Hkv=4), "FA_ERR_GQA"),
    (dict(scale=float("nan")), "FA_ERR_SCALE"),
    (dict(scale=float("inf")), "FA_ERR_SCALE"),
    # a finite negative scale passes validation: the call fails later, at the null pointer
    (dict(scale=-0.5, q=ctypes.c_void_p(0)), "FA_ERR_NULL_POINTER"),
    (dict(scale=-1e30, q=ctypes.c_void_p(0)), "FA_ERR_NULL_POINTER"),
    (dict(scale=float("-inf")), "FA_ERR_SCALE"),
    (dict(N=1 << 26, D=128), "FA_ERR_TOO_LARGE"),
    (dict(B=1 << 20, Hq=1 << 12, Hkv=1 << 12), "FA_ERR_TOO_LARGE"),
    (dict(q=ctypes.c_void_p(0)), "FA_ERR_NULL_POINTER"),
    (dict(l=ctypes.c_void_p(0)), "FA_ERR_NULL_POINTER"),
    (dict(k=ctypes.c_void_p(A + 8)), "FA_ERR_ALIGNMENT"),
    (dict(l=ctypes.c_void_p(A + 2)), "FA_ERR_ALIGNMENT"),
    (dict(o=0), "FA_ERR_ALIAS"),
    (dict(l=ctypes.c_void_p(A + 1024)), "FA_ERR_ALIAS"),
])
def test_fwd_rejects(lib, kw, status):
    assert fwd(lib, **kw) == STATUS[status]


def test_workspace_size(lib):
    B, Hq, Hkv, N, D = 1, 16, 4, 4000, 128
    up = lambda x: (x + 255) // 256 * 256
    rows = B * Hq * N
    mha = 2 * up(rows * 4)
    assert fa.fa_bwd_workspace_size(B, Hq, Hq, N, D) == mha
    assert fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D) == mha + 2 * up(rows * D * 4)
    assert fa.fa_bwd_workspace_size(0, Hq, Hkv, N, D) == 0
    # one head of a long sequence: the dK/dV pass takes 2 query-range pieces and the dQ pass
    # 2 key-range pieces, each with fp32 partials
    r1 = 16384
    assert fa.fa_bwd_workspace_size(1, 1, 1, r1, D) == 2 * up(r1 * 4) + 2 * up(2 * r1 * D * 4) + up(2 * r1 * D * 4)
    assert fa.fa_bwd_workspace_size(B, Hq, Hkv, N, 96) == 0


def bwd(lib, ws_bytes=None, B=1, Hq=2, Hkv=2, N=256, D=64, scale=0.125, dtype=0, **over):
    names = ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"]
    ptrs = {n: ptr(i) for i, n in enumerate(names)}
    ptrs.update(over)
    if ws_bytes is None:
        ws_bytes = fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D)
    return lib.fa_bwd(*[ptrs[n] for n in names], ws_bytes, B, Hq, Hkv, N, D, scale, 0, dtype, None)


def test_fp32_sizes_in_alias_checks(lib):
    # float32 buffers are twice as long: o right after q's 16-bit extent overlaps q in fp32
    B, Hq, N, D = 1, 2, 256, 64
    q16 = B * Hq * N * D * 2
    qp, op = ctypes.c_void_p(A), ctypes.c_void_p(A + q16)
    assert fwd(lib, q=qp, o=op, dtype=2) == STATUS["FA_ERR_ALIAS"]


def test_bwd_rejects(lib):
    need = fa.fa_bwd_workspace_size(1, 2, 2, 256, 64)
    assert bwd(lib, ws_bytes=need - 1) == STATUS["FA_ERR_WORKSPACE"]
    assert bwd(lib, D=80) == STATUS["FA_ERR_HEAD_DIM"]
    assert bwd(lib, dtype=7) == STATUS["FA_ERR_DTYPE"]
    assert bwd(lib, scale=float("nan")) == STATUS["FA_ERR_SCALE"]
    assert bwd(lib, scale=-1.0, dq=ctypes.c_void_p(0)) == STATUS["FA_ERR_NULL_POINTER"]  # accepted scale
    assert bwd(lib, dq=ctypes.c_void_p(0)) == STATUS["FA_ERR_NULL_POINTER"]
    assert bwd(lib, dv=ctypes.c_void_p(A + 4)) == STATUS["FA_ERR_ALIGNMENT"]
    assert bwd(lib, dq=ptr(0)) == STATUS["FA_ERR_ALIAS"]
    assert bwd(lib, ws=ptr(1)) == STATUS["FA_ERR_ALIAS"]
    assert bwd(lib, Hq=3, Hkv=2) == STATUS["FA_ERR_GQA"]


def test_stage_entry_points_reject(lib):
    B, Hq, Hkv, N, D = 1, 4, 2, 100, 128
    need = fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D)
    assert lib.fa_bwd_preprocess(ptr(0), ptr(1), ptr(3), ptr(2), need - 16, B, Hq, Hkv, N, D, 1, None) == \
        STATUS["FA_ERR_WORKSPACE"]
    assert lib.fa_bwd_preprocess(ptr(0), ctypes.c_void_p(0), ptr(3), ptr(2), need, B, Hq, Hkv, N, D, 1, None) == \
        STATUS["FA_ERR_NULL_POINTER"]
    assert lib.fa_bwd_preprocess(ptr(0), ptr(1), ctypes.c_void_p(A + 2), ptr(2), need, B, Hq, Hkv, N, D, 1,
                                 None) == STATUS["FA_ERR_ALIGNMENT"]
    assert lib.fa_bwd_dkdv(ptr(0), ptr(1), ptr(2), ptr(3), None, None, ptr(5), need,
                           B, Hq, Hkv, N, 32, 0.1, 1, 1, None) == STATUS["FA_ERR_HEAD_DIM"]
    # MHA writes dk/dv in the dK/dV stage; GQA writes them in the postprocess
    assert lib.fa_bwd_dkdv(ptr(0), ptr(1), ptr(2), ptr(3), None, None, ptr(5),
                           fa.fa_bwd_workspace_size(B, 2, 2, N, D), B, 2, 2, N, D, 0.1, 1, 1,
                           None) == STATUS["FA_ERR_NULL_POINTER"]
    assert lib.fa_bwd_dq(ptr(0), ptr(1), ptr(2), ptr(3), None, ptr(5), need, B, Hq, Hkv, N, D, 0.1, 1, 1,
                         None) == STATUS["FA_ERR_NULL_POINTER"]
    assert lib.fa_bwd_dq(ptr(0), ptr(1), ptr(2), ptr(3), ptr(0), ptr(5), need, B, Hq, Hkv, N, D, 0.1, 1, 1,
                         None) == STATUS["FA_ERR_ALIAS"]
    assert lib.fa_bwd_dq(ptr(0), ptr(1), ptr(2), ptr(3), ptr(4), ptr(5), need, B, Hq, Hkv, N, D,
                         float("inf"), 1, 1, None) == STATUS["FA_ERR_SCALE"]
    # a negative scale is accepted: the call fails later, at the aliased output
    assert lib.fa_bwd_dq(ptr(0), ptr(1), ptr(2), ptr(3), ptr(0), ptr(5), need, B, Hq, Hkv, N, D, -0.1, 1, 1,
                         None) == STATUS["FA_ERR_ALIAS"]
    assert lib.fa_bwd_postprocess(None, ptr(2), ptr(5), need, B, Hq, Hkv, N, D, 1, None) == \
        STATUS["FA_ERR_NULL_POINTER"]
    assert lib.fa_bwd_postprocess(ptr(1), ptr(2), ptr(1), need, B, Hq, Hkv, N, D, 1, None) == \
        STATUS["FA_ERR_ALIAS"]


def test_bwd_plan(lib):
    ROWS, STAGES = fa.FA_BWD_PLAN_ROWS, fa.FA_BWD_PLAN_STAGES
    text = open(HEADER).read()
    assert re.search(rf"\bFA_BWD_PLAN_STAGES\s*=\s*{STAGES}\b", text)
    assert re.search(rf"\bFA_BWD_PLAN_ROWS\s*=\s*{ROWS}\b", text)
    # MHA grids whose dK/dV pass writes dk/dv directly: the dQ pass first, forming the row values
    assert fa.fa_bwd_plan(1, 16, 16, 16384, 128, fa.FA_BF16) == ROWS
    assert fa.fa_bwd_plan(4, 16, 16, 4096, 128, fa.FA_BF16) == ROWS
    assert fa.fa_bwd_plan(1, 2, 2, 256, 64, fa.FA_FP16) == ROWS
    # partials: grouped-query heads, or one head cut into query-range pieces
    assert fa.fa_bwd_plan(1, 16, 4, 4096, 128, fa.FA_FP16) == STAGES
    assert fa.fa_bwd_plan(1, 1, 1, 16384, 128, fa.FA_BF16) == STAGES
    # the fp32 path keeps the four stages
    assert fa.fa_bwd_plan(1, 16, 16, 4096, 128, fa.FA_FP32) == STAGES
    # invalid arguments: the negated status
    assert lib.fa_bwd_plan(1, 16, 16, 4096, 96, 1) == -STATUS["FA_ERR_HEAD_DIM"]
    assert lib.fa_bwd_plan(1, 16, 16, 4096, 128, 5) == -STATUS["FA_ERR_DTYPE"]
    assert lib.fa_bwd_plan(0, 16, 16, 4096, 128, 1) == -STATUS["FA_ERR_BAD_SHAPE"]
    with pytest.raises(RuntimeError, match="head"):
        fa.fa_bwd_plan(1, 16, 16, 4096, 96, fa.FA_BF16)


def test_dq_rows_rejects(lib):
    B, Hq, Hkv, N, D = 1, 4, 4, 100, 128
    need = fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D)

    def rows(ws_bytes=need, scale=0.1, dtype=1, Dh=D, **over):
        names = ["q", "k", "v", "o", "do", "lse", "dq", "ws"]
        ptrs = {n: ptr(i) for i, n in enumerate(names)}
        ptrs.update(over)
        return lib.fa_bwd_dq_rows(*[ptrs[n] for n in names], ws_bytes, B, Hq, Hkv, N, Dh, scale, 1, dtype, None)
    assert rows(ws_bytes=need - 1) == STATUS["FA_ERR_WORKSPACE"]
    assert rows(Dh=80) == STATUS["FA_ERR_HEAD_DIM"]
    assert rows(dtype=4) == STATUS["FA_ERR_DTYPE"]
    assert rows(scale=float("nan")) == STATUS["FA_ERR_SCALE"]
    assert rows(o=ctypes.c_void_p(0)) == STATUS["FA_ERR_NULL_POINTER"]
    assert rows(lse=ctypes.c_void_p(0)) == STATUS["FA_ERR_NULL_POINTER"]
    assert rows(lse=ctypes.c_void_p(A + 2)) == STATUS["FA_ERR_ALIGNMENT"]
    assert rows(dq=ptr(3)) == STATUS["FA_ERR_ALIAS"]   # dq over o
    assert rows(ws=ptr(5)) == STATUS["FA_ERR_ALIAS"]   # the workspace over lse
    assert rows(scale=-0.1, dq=ptr(0)) == STATUS["FA_ERR_ALIAS"]  # a negative scale passes


def test_splitkv_workspace_and_parts(lib):
    B, Hq, Hkv, N, D = 1, 2, 1, 3000, 128
    up = lambda x: (x + 255) // 256 * 256
    rows = B * Hq * N
    assert fa.fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, D, 3) == up(3 * rows * D * 4) + up(3 * rows * 4)
    assert fa.fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, D, 1) == 0
    assert fa.fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, D, 0) == 0
    assert fa.fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, D, 65) == 0
    assert fa.fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, 80, 2) == 0
    # grids that fill the GPU take no pieces; one head of a long sequence takes several
    assert fa.fa_fwd_splitkv_parts(4, 16, 16, 4096, 128, False) == 1
    assert fa.fa_fwd_splitkv_parts(1, 1, 1, 16384, 128, False) == 2
    assert fa.fa_fwd_splitkv_parts(1, 1, 1, 8192, 64, True) == 4
    assert fa.fa_fwd_splitkv_parts(1, 16, 4, 2048, 64, True) == 1
    assert fa.fa_fwd_splitkv_parts(1, 1, 1, 100, 64, False) == 1
    assert fa.fa_fwd_splitkv_parts(1, 1, 1, 100, 96, False) == 0


def splitkv(lib, n_split=2, ws_bytes=None, B=1, Hq=2, Hkv=2, N=4096, D=128, scale=0.1, dtype=1, **over):
    names = ["q", "k", "v", "o", "lse", "ws"]
    ptrs = {n: ptr(i) for i, n in enumerate(names)}
    ptrs.update({n: x if isinstance(x, ctypes.c_void_p) else ptr(x) for n, x in over.items()})
    if ws_bytes is None:
        ws_bytes = fa.fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, D, max(n_split, 1))
    return lib.fa_fwd_splitkv(*[ptrs[n] for n in names[:5]], ptrs["ws"], ws_bytes, n_split, B, Hq, Hkv, N, D,
                              scale, 0, dtype, None)


def test_splitkv_rejects(lib):
    assert splitkv(lib, n_split=-1) == STATUS["FA_ERR_SPLIT"]
    assert splitkv(lib, n_split=65) == STATUS["FA_ERR_SPLIT"]
    assert splitkv(lib, n_split=3, ws_bytes=fa.fa_fwd_splitkv_workspace_size(1, 2, 2, 4096, 128, 3) - 1) == \
        STATUS["FA_ERR_WORKSPACE"]
    assert splitkv(lib, ws=ctypes.c_void_p(0)) == STATUS["FA_ERR_NULL_POINTER"]
    assert splitkv(lib, ws=ctypes.c_void_p(A + 64)) == STATUS["FA_ERR_ALIGNMENT"]
    assert splitkv(lib, ws=ptr(3)) == STATUS["FA_ERR_ALIAS"]
    assert splitkv(lib, D=96) == STATUS["FA_ERR_HEAD_DIM"]
    assert splitkv(lib, scale=float("nan")) == STATUS["FA_ERR_SCALE"]
    # a resolved count of 1 is fa_fwd's own validation (no workspace needed)
    assert splitkv(lib, n_split=1, ws=ctypes.c_void_p(0), o=0) == STATUS["FA_ERR_ALIAS"]


def test_merge_rejects(lib):
    def merge(op=0, lp=1, n=2, o=2, l=3, rows=100, D=128, dtype=1):
        P = lambda x: x if isinstance(x, ctypes.c_void_p) else ptr(x)
        return lib.fa_merge_partials(P(op), P(lp), n, P(o), P(l), rows, D, dtype, None)
    assert merge(n=0) == STATUS["FA_ERR_SPLIT"]
    assert merge(n=65) == STATUS["FA_ERR_SPLIT"]
    assert merge(rows=0) == STATUS["FA_ERR_BAD_SHAPE"]
    assert merge(D=32) == STATUS["FA_ERR_HEAD_DIM"]
    assert merge(dtype=3) == STATUS["FA_ERR_DTYPE"]
    assert merge(dtype=2) == STATUS["FA_ERR_DTYPE"]  # the fp32 path has no pieces to merge
    assert merge(op=ctypes.c_void_p(0)) == STATUS["FA_ERR_NULL_POINTER"]
    assert merge(op=ctypes.c_void_p(A + 4)) == STATUS["FA_ERR_ALIGNMENT"]
    assert merge(o=0) == STATUS["FA_ERR_ALIAS"]


def test_python_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    with pytest.raises(RuntimeError):
        fa.fa_fwd(q, q, q)


def test_noalloc_rejects_before_any_device_call(lib):
    """fa_bwd_noalloc: invalid shapes report fa_bwd's status, and a call that needs more than
    the static scratch returns FA_ERR_SCRATCH, both before any HIP call (no GPU here)."""
    names = ["q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"]
    p = [ptr(i) for i in range(len(names))]
    call = lambda B, Hq, Hkv, N, D: lib.fa_bwd_noalloc(*p, B, Hq, Hkv, N, D, 0.1, 1, 1, None)
    assert call(1, 2, 2, 256, 80) == STATUS["FA_ERR_HEAD_DIM"]
    assert call(0, 2, 2, 256, 64) == STATUS["FA_ERR_BAD_SHAPE"]
    assert call(1, 6, 4, 256, 64) == STATUS["FA_ERR_GQA"]
    # grouped heads at N = 8192, D = 128: 128 MiB of fp32 dK/dV partials
    assert fa.fa_bwd_workspace_size(1, 16, 4, 8192, 128) > fa.FA_NOALLOC_SCRATCH_BYTES
    assert call(1, 16, 4, 8192, 128) == STATUS["FA_ERR_SCRATCH"]
    # every configured workload fits
    from exact_attention_fa_amd.inputs import WORKLOADS
    for shapes in WORKLOADS.values():
        for sh in shapes:
            assert fa.fa_bwd_workspace_size(sh.B, sh.Hq, sh.Hkv, sh.N, sh.D) <= fa.FA_NOALLOC_SCRATCH_BYTES, sh

