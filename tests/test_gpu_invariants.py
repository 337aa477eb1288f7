"""GPU checks that do not rely on the oracle's arithmetic: properties of the definition,
the pages' printed softmax numbers, determinism, error behaviour."""
import json
import math
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import exact_attention_fa_amd as fa
    fa.load_library()
    return torch, fa


def inputs(shape, seed):
    from exact_attention_fa_amd.inputs import make_inputs
    import torch
    return [t.to("cuda") for t in make_inputs(shape, seed)]


def test_page_softmax_table_on_gpu(torch_fa):
    """FlashStieltjes page, 'Why touch softmax' figure data table (softmax column): 64 keys
    whose scores fall by 0.25 per key.  The GPU's fp32 LSE must reproduce every printed weight
    through p_j = exp(s_j - LSE), and its fp16 O (with V = identity, so O is the probability
    row) the weights that fp16 can hold."""
    torch, fa = torch_fa
    g = json.load(open(os.path.join(GOLDEN, "softmax_geometric_scores.json")))
    n = g["n_keys"]
    q = torch.zeros(1, 1, n, 64, dtype=torch.float16, device="cuda")
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, n, 64, dtype=torch.float16, device="cuda")
    k[0, 0, :, 0] = g["score_step"] * torch.arange(n, dtype=torch.float32, device="cuda")
    v = torch.eye(n, 64, dtype=torch.float16, device="cuda").reshape(1, 1, n, 64)
    o, lse = fa.fa_fwd(q, k, v, causal=False, softmax_scale=1.0)
    torch.cuda.synchronize()
    lse0 = float(lse[0, 0, 0])
    row = o[0, 0, 0].float().cpu().numpy()
    for r in g["rows"]:
        j = int(round(r["gap"] / -g["score_step"]))
        p_lse = math.exp(g["score_step"] * j - lse0)
        assert float(f"{p_lse:.{r['sig_digits']}g}") == pytest.approx(r["softmax"], rel=1e-9), (r, p_lse)
        if r["softmax"] > 1e-3:
            assert float(f"{row[j]:.{r['sig_digits']}g}") == pytest.approx(r["softmax"], rel=1e-9), (r, row[j])


@pytest.mark.parametrize("causal", [False, True])
def test_forward_bitwise_deterministic(torch_fa, causal):
    torch, fa = torch_fa
    from exact_attention_fa_amd.inputs import Shape
    q, k, v, _ = inputs(Shape(2, 8, 2, 1500, 128, "bf16", causal), 5)
    o1, l1 = fa.fa_fwd(q, k, v, causal=causal)
    o2, l2 = fa.fa_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_gives_value_means(torch_fa, causal):
    torch, fa = torch_fa
    from exact_attention_fa_amd.inputs import Shape
    N = 700
    q, k, v, _ = inputs(Shape(1, 4, 2, N, 64, "fp16", causal), 9)
    o, lse = fa.fa_fwd(q, k, v, causal=causal, softmax_scale=0.0)
    torch.cuda.synchronize()
    vv = v.double().cpu().numpy()
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    for h in range(4):
        vh = vv[0, h // 2]
        ref = np.cumsum(vh, axis=0) / cnt[:, None] if causal else np.broadcast_to(vh.mean(0), vh.shape)
        assert np.abs(o[0, h].double().cpu().numpy() - ref).max() < 5e-3
        assert np.abs(lse[0, h].double().cpu().numpy() - np.log(cnt)).max() < 1e-4


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_identities(torch_fa, causal):
    """sum_j dK_j = 0 (rows of dS sum to zero) and sum_j dV_j = sum over the group of sum_i dO_i."""
    torch, fa = torch_fa
    from exact_attention_fa_amd.inputs import Shape
    q, k, v, do = inputs(Shape(1, 8, 2, 1100, 128, "bf16", causal), 13)
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    dk64 = dk.double()
    resid = dk64.sum(dim=2).abs()
    scale = dk64.abs().sum(dim=2)
    assert float((resid / scale).max()) < 2e-2
    tot = do.double().reshape(1, 2, 4, 1100, 128).sum(dim=(2, 3))
    assert float((dv.double().sum(dim=2) - tot).abs().max()) < 2e-2 * float(tot.abs().max()) + 0.05


def test_constant_values_give_zero_dq_dk(torch_fa):
    torch, fa = torch_fa
    from exact_attention_fa_amd.inputs import Shape
    q, k, v, do = inputs(Shape(1, 4, 4, 600, 64, "bf16", True), 17)
    o_r, l_r = fa.fa_fwd(q, k, v, causal=True)
    dq_r, dk_r, _ = fa.fa_bwd(q, k, v, o_r, do, l_r, causal=True)
    vc = v[:, :, :1].expand_as(v).contiguous()
    o, lse = fa.fa_fwd(q, k, vc, causal=True)
    dq, dk, dv = fa.fa_bwd(q, k, vc, o, do, lse, causal=True)
    torch.cuda.synchronize()
    assert float((o.float() - vc.float()).abs().max()) < 1e-2
    assert float(dq.float().abs().max()) < 2e-2 * float(dq_r.float().abs().max())
    assert float(dk.float().abs().max()) < 2e-2 * float(dk_r.float().abs().max())


def test_rejected_call_writes_nothing(torch_fa):
    torch, fa = torch_fa
    q = torch.randn(1, 2, 100, 64, device="cuda").half()
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 2, 100), 3.0, device="cuda")
    with pytest.raises(RuntimeError, match="softmax_scale"):
        fa.fa_fwd(q, q, q, softmax_scale=float("nan"), out=o, lse=lse)
    with pytest.raises(RuntimeError, match="head dim"):
        x = torch.randn(1, 2, 100, 96, device="cuda").half()
        fa.fa_fwd(x, x, x)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 3.0).all())


def test_no_drift_along_sequence(torch_fa):
    """'FlashAttention for Tesla P100', section 'Driving a real model': the error of the online
    softmax does not grow with the position in the sequence.  Binned by position, the largest
    error of the last bin stays within twice that of the first bin (plus the output rounding)."""
    torch, fa = torch_fa
    from exact_attention_fa_amd.inputs import WORKLOADS, make_inputs, workload_seed
    from oracle import attention_forward
    shape = WORKLOADS["fwd_bf16_long"][0]            # N = 8192
    q, k, v, _ = make_inputs(shape, workload_seed("fwd_bf16_long", 0), with_grad=False)
    o, _ = fa.fa_fwd(q[:, :1].cuda(), k[:, :1].cuda(), v[:, :1].cuda())
    torch.cuda.synchronize()
    rows = np.arange(0, shape.N, 32)
    f = lambda t: t.double().cpu().numpy()
    o_ref, _ = attention_forward(f(q[:, :1]), f(k[:, :1]), f(v[:, :1]), shape.scale, False, rows=rows)
    err = np.abs(f(o)[0, 0, rows] - o_ref[0, 0]).max(axis=-1)
    bins = err.reshape(8, -1).max(axis=1)
    log("per-bin max error", bins)
    assert bins[-1] <= 2 * bins[0] + 2e-3


@pytest.mark.parametrize("causal", [False, True])
def test_backward_bitwise_deterministic(torch_fa, causal):
    """No atomics anywhere in the backward: repeated runs give identical bits."""
    torch, fa = torch_fa
    from exact_attention_fa_amd.inputs import Shape
    q, k, v, do = inputs(Shape(1, 8, 2, 1300, 128, "bf16", causal), 21)
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    g1 = fa.fa_bwd(q, k, v, o, do, lse, causal=causal)
    g2 = fa.fa_bwd(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


STAGE_SHAPES = [
    (2, 8, 4, 700, 64, "fp16", True),      # dQ key-range pieces: separate partial sums
    (1, 16, 4, 2048, 128, "fp16", True),   # one-round causal grid: the dQ pass runs the sums
    (2, 16, 4, 4096, 128, "bf16", False),  # 256-query dQ workgroups with the sums
    (2, 16, 4, 4096, 64, "fp16", False),   # 4-wave dQ workgroups (two per CU) with the sums
    # no dK/dV partials: the dQ pass runs first and forms the row values itself
    (2, 16, 16, 4096, 128, "bf16", False),  # 256-query dQ workgroups
    (1, 32, 32, 4096, 128, "fp16", True),   # 256-query dQ workgroups, causal
    (1, 16, 16, 2000, 128, "bf16", True),   # split 128-query workgroups, ragged tail
    (2, 16, 16, 2048, 64, "fp16", False),   # 4-wave dQ workgroups
    (4, 16, 16, 1000, 128, "bf16", False),  # 4-wave dQ workgroups, D=128, ragged tail
    (1, 2, 2, 512, 64, "fp16", False),      # dQ key-range pieces (the first piece stores the rows)
    (1, 2, 2, 256, 64, "fp16", True),       # the tiny causal workload
]


@pytest.mark.parametrize("dims", STAGE_SHAPES, ids=[f"B{b}H{hq}/{hk}N{n}D{d}{t}{'c' if cz else ''}"
                                                    for b, hq, hk, n, d, t, cz in STAGE_SHAPES])
def test_backward_stages_equal_fused_call(torch_fa, dims):
    """The exported stages, run in order on one stream, reproduce fa_bwd bit for bit (fa_bwd
    runs the grouped-query partial sums inside its dQ pass where the grid allows, and where
    the dK/dV pass writes no partials it runs the dQ pass first, forming the preprocess's row
    values there)."""
    torch, fa = torch_fa
    from exact_attention_fa_amd.inputs import Shape
    shape = Shape(*dims)
    B, Hq, Hkv, N, D, causal = shape.B, shape.Hq, shape.Hkv, shape.N, shape.D, shape.causal
    q, k, v, do = inputs(shape, 23)
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D), dtype=torch.uint8, device="cuda")
    dq2, dk2, dv2 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    fa.fa_bwd_preprocess(o, do, lse, ws, Hkv)
    fa.fa_bwd_dkdv(q, k, v, do, dk2, dv2, ws, causal=causal)
    fa.fa_bwd_dq(q, k, v, do, dq2, ws, causal=causal)
    fa.fa_bwd_postprocess(dk2, dv2, ws, Hq)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    # the combined stage in place of the preprocess and the dQ pass (fa_bwd's own order where
    # fa_bwd_plan says so), on a workspace that holds the last run's values
    plan = fa.fa_bwd_plan(B, Hq, Hkv, N, D, fa.FA_BF16 if q.dtype == torch.bfloat16 else fa.FA_FP16)
    assert plan == (fa.FA_BWD_PLAN_ROWS if Hq == Hkv else fa.FA_BWD_PLAN_STAGES), plan
    dq3, dk3, dv3 = (torch.full_like(t, float("nan")) for t in (dq, dk, dv))
    ws.fill_(0xFF)
    fa.fa_bwd_dq_rows(q, k, v, o, do, lse, dq3, ws, causal=causal)
    fa.fa_bwd_dkdv(q, k, v, do, dk3, dv3, ws, causal=causal)
    fa.fa_bwd_postprocess(dk3, dv3, ws, Hq)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq3) and torch.equal(dk, dk3) and torch.equal(dv, dv3)


@pytest.mark.parametrize("scale", [-0.15, 0.0])
def test_backward_stage_orders_other_scales(torch_fa, scale):
    """Both stage orders reproduce fa_bwd bit for bit at a negative and a zero softmax scale
    (MHA: fa_bwd forms the row values in its dQ pass; GQA: the preprocess runs first)."""
    torch, fa = torch_fa
    from exact_attention_fa_amd.inputs import Shape
    for dims in [(1, 8, 8, 1500, 128, "bf16", True), (1, 8, 2, 900, 64, "fp16", False)]:
        shape = Shape(*dims)
        B, Hq, Hkv, N, D, causal = shape.B, shape.Hq, shape.Hkv, shape.N, shape.D, shape.causal
        q, k, v, do = inputs(shape, 29)
        o, lse = fa.fa_fwd(q, k, v, causal=causal, softmax_scale=scale)
        ref = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, softmax_scale=scale)
        ws = torch.empty(fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D), dtype=torch.uint8, device="cuda")
        for rows in (False, True):
            dq, dk, dv = (torch.full_like(t, float("nan")) for t in ref)
            ws.fill_(0xFF)
            if rows:
                fa.fa_bwd_dq_rows(q, k, v, o, do, lse, dq, ws, causal=causal, softmax_scale=scale)
                fa.fa_bwd_dkdv(q, k, v, do, dk, dv, ws, causal=causal, softmax_scale=scale)
            else:
                fa.fa_bwd_preprocess(o, do, lse, ws, Hkv)
                fa.fa_bwd_dkdv(q, k, v, do, dk, dv, ws, causal=causal, softmax_scale=scale)
                fa.fa_bwd_dq(q, k, v, do, dq, ws, causal=causal, softmax_scale=scale)
            fa.fa_bwd_postprocess(dk, dv, ws, Hq)
            torch.cuda.synchronize()
            for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
                assert torch.equal(a, b), (dims, scale, rows, name)


def test_concurrent_streams_match_one_stream(torch_fa):
    """The library keeps no mutable global state: the same calls enqueued on two streams at
    once (separate outputs and workspaces) give the bits of a single-stream run."""
    torch, fa = torch_fa
    from exact_attention_fa_amd.inputs import Shape
    shapes = [Shape(2, 8, 2, 1500, 128, "bf16", True), Shape(1, 4, 4, 2100, 64, "fp16", False)]
    data = [inputs(s, 31 + i) for i, s in enumerate(shapes)]
    ref = []
    for (q, k, v, do), s in zip(data, shapes):
        o, lse = fa.fa_fwd(q, k, v, causal=s.causal)
        ref.append((o, lse, *fa.fa_bwd(q, k, v, o, do, lse, causal=s.causal)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    out = [None, None]
    for rep in range(3):
        for i, ((q, k, v, do), s) in enumerate(zip(data, shapes)):
            with torch.cuda.stream(streams[i]):
                o, lse = fa.fa_fwd(q, k, v, causal=s.causal)
                out[i] = (o, lse, *fa.fa_bwd(q, k, v, o, do, lse, causal=s.causal))
        torch.cuda.synchronize()
        for i in range(2):
            for a, b in zip(out[i], ref[i]):
                assert torch.equal(a, b), f"stream {i}, repetition {rep}"


def test_graph_replay_matches_eager(torch_fa):
    """fa_fwd and the fa_bwd stages captured in a HIP graph: every replay, with new inputs
    copied in and eager work in between, gives the bits of the eager calls."""
    torch, fa = torch_fa
    from exact_attention_fa_amd.inputs import Shape
    shape = Shape(1, 8, 2, 1200, 128, "bf16", True)
    B, Hq, Hkv, N, D = shape.B, shape.Hq, shape.Hkv, shape.N, shape.D
    q, k, v, do = (t.clone() for t in inputs(shape, 41))
    o, lse = torch.empty_like(q), torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D), dtype=torch.uint8, device="cuda")

    def step():
        fa.fa_fwd(q, k, v, causal=True, out=o, lse=lse)
        fa.fa_bwd_preprocess(o, do, lse, ws, Hkv)
        fa.fa_bwd_dkdv(q, k, v, do, dk, dv, ws, causal=True)
        fa.fa_bwd_dq(q, k, v, do, dq, ws, causal=True)
        fa.fa_bwd_postprocess(dk, dv, ws, Hq)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        new = inputs(shape, 50 + rep)
        for dst, src in zip((q, k, v, do), new):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv)]
        e_o, e_l = fa.fa_fwd(q, k, v, causal=True)
        e_g = fa.fa_bwd(q, k, v, e_o, do, e_l, causal=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, (e_o, e_l, *e_g)):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
