"""GPU parity of the fp32 verification path (dtype FA_FP32) against the CPU oracle, and its
use as a checker of the 16-bit path, through the C ABI.

Tolerances for fp32 inputs (fp32 products and sums on both sides of the GPU computation;
the oracle is fp64): O and LSE max-abs <= 2e-5, gradients per-tensor max-abs relative
<= 2e-4 -- a few hundred fp32 roundings of accumulated error, far below the 16-bit bounds.
"""
import sys
import zlib

import numpy as np
import pytest

from exact_attention_fa_amd.inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu

TOL_O32, TOL_LSE32, TOL_GRAD32 = 2e-5, 2e-5, 2e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import exact_attention_fa_amd as fa
    fa.load_library()


F32 = [
    # (B, Hq, Hkv, N, D, causal)
    (1, 2, 2, 256, 64, False),
    (1, 2, 2, 256, 64, True),
    (1, 4, 2, 333, 128, False),
    (2, 3, 1, 129, 64, True),
    (1, 2, 1, 1000, 128, True),
    (1, 1, 1, 1, 128, False),
]


@pytest.mark.parametrize("dims", F32, ids=[f"B{b}H{hq}/{hk}N{n}D{d}{'c' if cz else ''}" for b, hq, hk, n, d, cz in F32])
def test_f32_full(dims):
    import torch
    import exact_attention_fa_amd as fa
    from parity_util import attention_backward, attention_forward, f64
    B, Hq, Hkv, N, D, causal = dims
    shape = Shape(B, Hq, Hkv, N, D, "fp32", causal)
    log("fp32", shape)
    q, k, v, do = make_inputs(shape, seed=zlib.crc32(repr(dims).encode()) % (1 << 31))
    dev = torch.device("cuda", 0)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, dod, lse, causal=causal)
    torch.cuda.synchronize()
    assert o.dtype == torch.float32 and dq.dtype == torch.float32
    o_r, l_r = attention_forward(f64(q), f64(k), f64(v), shape.scale, causal)
    eo, el = float(np.abs(f64(o) - o_r).max()), float(np.abs(f64(lse) - l_r).max())
    assert eo <= TOL_O32 and el <= TOL_LSE32, (eo, el)
    refs = attention_backward(f64(q), f64(k), f64(v), f64(do), shape.scale, causal)
    errs = {}
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        e = float(np.abs(f64(g) - r).max() / max(np.abs(r).max(), 1e-2))
        errs[name] = e
        assert np.isfinite(f64(g)).all() and e <= TOL_GRAD32, (name, e)
    log("  errors", eo, el, errs)


def test_f32_negative_scale():
    """The fp32 path keeps its running max in scaled units, so a negative scale is exact too."""
    import torch
    import exact_attention_fa_amd as fa
    from parity_util import attention_backward, attention_forward, f64
    shape = Shape(1, 4, 2, 300, 64, "fp32", True)
    q, k, v, do = make_inputs(shape, seed=4242)
    dev = torch.device("cuda", 0)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=True, softmax_scale=-0.2)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, dod, lse, causal=True, softmax_scale=-0.2)
    torch.cuda.synchronize()
    o_r, l_r = attention_forward(f64(q), f64(k), f64(v), -0.2, True)
    assert float(np.abs(f64(o) - o_r).max()) <= TOL_O32 and float(np.abs(f64(lse) - l_r).max()) <= TOL_LSE32
    for g, r in zip((dq, dk, dv), attention_backward(f64(q), f64(k), f64(v), f64(do), -0.2, True)):
        assert float(np.abs(f64(g) - r).max() / max(np.abs(r).max(), 1e-2)) <= TOL_GRAD32


def test_f32_checks_the_16bit_path():
    """Gradient checking: the fp32 path on the bf16 inputs (upcast) against the bf16 kernels;
    the difference stays within the 16-bit tolerances."""
    import torch
    import exact_attention_fa_amd as fa
    shape = Shape(2, 8, 2, 1000, 128, "bf16", True)
    q, k, v, do = (x.cuda() for x in make_inputs(shape, seed=31337))
    o16, l16 = fa.fa_fwd(q, k, v, causal=True)
    g16 = fa.fa_bwd(q, k, v, o16, do, l16, causal=True)
    q32, k32, v32, do32 = (x.float() for x in (q, k, v, do))
    o32, l32 = fa.fa_fwd(q32, k32, v32, causal=True)
    g32 = fa.fa_bwd(q32, k32, v32, o32, do32, l32, causal=True)
    torch.cuda.synchronize()
    assert float((o16.float() - o32).abs().max()) <= 1e-2
    assert float((l16 - l32).abs().max()) <= 1e-3
    for a, b in zip(g16, g32):
        assert float((a.float() - b).abs().max() / b.abs().max().clamp_min(1e-2)) <= 2e-2


def test_f32_splitkv_runs_as_fwd():
    import torch
    import exact_attention_fa_amd as fa
    shape = Shape(1, 1, 1, 2048, 64, "fp32", False)
    q, k, v, _ = (x.cuda() if x is not None else None for x in make_inputs(shape, seed=5, with_grad=False))
    o1, l1 = fa.fa_fwd(q, k, v)
    o2, l2 = fa.fa_fwd_splitkv(q, k, v, n_split=4, workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_f32_stage_orders_match_fa_bwd():
    """The fp32 path's stages, in either order (the four stages; fa_bwd_dq_rows, which on this
    path enqueues the preprocess and the dQ pass, then the dK/dV pass), give fa_bwd's bits."""
    import torch
    import exact_attention_fa_amd as fa
    shape = Shape(1, 4, 2, 333, 128, "fp32", True)
    q, k, v, do = (x.cuda() for x in make_inputs(shape, seed=515))
    B, Hq, Hkv, N, D = shape.B, shape.Hq, shape.Hkv, shape.N, shape.D
    assert fa.fa_bwd_plan(B, Hq, Hkv, N, D, fa.FA_FP32) == fa.FA_BWD_PLAN_STAGES
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    ref = fa.fa_bwd(q, k, v, o, do, lse, causal=True)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D), dtype=torch.uint8, device="cuda")
    for rows in (False, True):
        dq, dk, dv = (torch.full_like(t, float("nan")) for t in ref)
        ws.fill_(0xFF)
        if rows:
            fa.fa_bwd_dq_rows(q, k, v, o, do, lse, dq, ws, causal=True)
            fa.fa_bwd_dkdv(q, k, v, do, dk, dv, ws, causal=True)
        else:
            fa.fa_bwd_preprocess(o, do, lse, ws, Hkv)
            fa.fa_bwd_dkdv(q, k, v, do, dk, dv, ws, causal=True)
            fa.fa_bwd_dq(q, k, v, do, dq, ws, causal=True)
        fa.fa_bwd_postprocess(dk, dv, ws, Hq)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert torch.equal(a, b), (rows, name)
