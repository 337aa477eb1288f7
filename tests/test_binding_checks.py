"""The Python binding checks every tensor argument (shape, dtype, device, contiguity) before
anything reaches the C ABI, which sees only pointers and cannot tell a wrongly shaped or host
buffer from a good one.  No GPU: the library handle is replaced by one that fails the test if
it is ever reached."""
import pytest
import torch

import exact_attention_fa_amd as fa


@pytest.fixture
def no_lib(monkeypatch):
    def unreachable():
        raise AssertionError("the library was reached before the arguments were checked")
    monkeypatch.setattr(fa, "load_library", unreachable)


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


B, Hq, Hkv, N, D = 2, 4, 2, 48, 64
Q, K, LSE = (B, Hq, N, D), (B, Hkv, N, D), (B, Hq, N)


def good():
    return dict(q=t(*Q), k=t(*K), v=t(*K), o=t(*Q), do=t(*Q), lse=t(*LSE, dtype=torch.float32))


BAD_FWD = [
    ("out", t(B, Hq, N - 1, D), "shape"),
    ("out", t(*Q, dtype=torch.float16), "dtype"),
    ("lse", t(B, Hq, N + 1, dtype=torch.float32), "shape"),
    ("lse", t(*LSE), "dtype"),
]


@pytest.mark.parametrize("name,val,what", BAD_FWD, ids=[f"{n}-{w}" for n, _, w in BAD_FWD])
@pytest.mark.parametrize("fn", ["fa_fwd", "fa_fwd_splitkv"])
def test_forward_outputs_checked(no_lib, fn, name, val, what):
    g = good()
    kw = {"out": val} if name == "out" else {"lse": val}
    with pytest.raises(RuntimeError, match=what):
        getattr(fa, fn)(g["q"], g["k"], g["v"], **kw)


def test_forward_inputs_checked(no_lib):
    g = good()
    with pytest.raises(RuntimeError, match="4-D"):
        fa.fa_fwd(g["q"][0], g["k"], g["v"])
    with pytest.raises(RuntimeError, match="B, N, D"):
        fa.fa_fwd(g["q"], t(B, Hkv, N + 1, D), t(B, Hkv, N + 1, D))
    with pytest.raises(RuntimeError, match="dtype"):
        fa.fa_fwd(g["q"], t(*K, dtype=torch.float16), t(*K, dtype=torch.float16))
    with pytest.raises(RuntimeError, match="GPU"):  # right shapes, host memory
        fa.fa_fwd(g["q"], g["k"], g["v"])
    with pytest.raises(RuntimeError, match="unsupported dtype"):
        fa.fa_fwd(t(*Q, dtype=torch.float64), t(*K, dtype=torch.float64), t(*K, dtype=torch.float64))


BAD_BWD = [
    ("o", t(B, Hq, N, D + 1), "shape"),
    ("do", t(B, Hq - 1, N, D), "shape"),
    ("lse", t(B, Hq, N, dtype=torch.float32)[:, :, :-1], "shape"),
    ("lse", t(*LSE), "dtype"),
    ("dq", t(*K), "shape"),
    ("dk", t(*Q), "shape"),
    ("dv", t(B, Hkv, N, D, dtype=torch.float16), "dtype"),
]


@pytest.mark.parametrize("name,val,what", BAD_BWD, ids=[f"{n}-{w}" for n, _, w in BAD_BWD])
def test_backward_buffers_checked(no_lib, name, val, what):
    g = good()
    args = dict(q=g["q"], k=g["k"], v=g["v"], o=g["o"], do=g["do"], lse=g["lse"])
    extra = {}
    if name in args:
        args[name] = val
    else:
        extra[name] = val
    with pytest.raises(RuntimeError, match=what):
        fa.fa_bwd(args["q"], args["k"], args["v"], args["o"], args["do"], args["lse"], **extra)


def test_backward_host_memory_refused(no_lib):
    g = good()
    with pytest.raises(RuntimeError, match="GPU"):
        fa.fa_bwd(g["q"], g["k"], g["v"], g["o"], g["do"], g["lse"])


def test_stage_wrappers_checked(no_lib):
    g = good()
    ws = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(RuntimeError, match="shape"):
        fa.fa_bwd_preprocess(g["o"], t(B, Hq, N, D - 8), g["lse"], ws, Hkv)
    with pytest.raises(RuntimeError, match="shape"):
        fa.fa_bwd_preprocess(g["o"], g["do"], t(B, Hq, 2 * N, dtype=torch.float32), ws, Hkv)
    with pytest.raises(RuntimeError, match="GPU"):
        fa.fa_bwd_preprocess(g["o"], g["do"], g["lse"], ws, Hkv)
    with pytest.raises(RuntimeError, match="shape"):
        fa.fa_bwd_dkdv(g["q"], g["k"], g["v"], t(B, Hq, N - 2, D), None, None, ws)
    with pytest.raises(RuntimeError, match="shape"):
        fa.fa_bwd_dkdv(g["q"], g["k"], g["v"], g["do"], t(*Q), t(*K), ws)
    with pytest.raises(RuntimeError, match="shape"):
        fa.fa_bwd_dq(g["q"], g["k"], g["v"], g["do"], t(*K), ws)
    with pytest.raises(RuntimeError, match="dtype"):
        fa.fa_bwd_dq(g["q"], g["k"], g["v"], g["do"], t(*Q, dtype=torch.float16), ws)
    with pytest.raises(RuntimeError, match="shape"):
        fa.fa_bwd_postprocess(t(*K), t(B, Hkv, N, D // 2), ws, Hq)
    with pytest.raises(RuntimeError, match="GPU"):
        fa.fa_bwd_postprocess(t(*K), t(*K), ws, Hq)
    with pytest.raises(RuntimeError, match="required"):
        fa.fa_bwd_dq(g["q"], g["k"], g["v"], g["do"], None, ws)


def test_merge_checked(no_lib):
    n, rows = 3, 40
    op, lp = t(n, rows, D, dtype=torch.float32), t(n, rows, dtype=torch.float32)
    with pytest.raises(RuntimeError, match="elements"):
        fa.fa_merge_partials(op, lp, t(rows + 1, D), t(rows, dtype=torch.float32))
    with pytest.raises(RuntimeError, match="elements"):
        fa.fa_merge_partials(op, lp, t(rows, D), t(rows - 1, dtype=torch.float32))
    with pytest.raises(RuntimeError, match="dtype"):
        fa.fa_merge_partials(op.half(), lp, t(rows, D), t(rows, dtype=torch.float32))
    with pytest.raises(RuntimeError, match="GPU"):
        fa.fa_merge_partials(op, lp, t(rows, D), t(rows, dtype=torch.float32))
