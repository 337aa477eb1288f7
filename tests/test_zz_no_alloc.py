"""fa_bwd_noalloc (the backward whose workspace is the library's static scratch array) against
fa_bwd with a caller-owned workspace, through the C ABI: two calls in a row, the second on a
smaller problem (the array keeps the first call's contents), each compared bit for bit with
fa_bwd and within the parity tolerances with the oracle; a call too large for the array is
refused before anything is enqueued."""
import sys

import pytest

from exact_attention_fa_amd.inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_noalloc_matches_fa_bwd_two_calls():
    import torch
    import exact_attention_fa_amd as fa
    from parity_util import assert_grad_close, attention_backward, f64
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    fa.load_library()
    # first the largest configured workspace (grouped-query heads, fp32 dK/dV partials: 64.5 MiB),
    # then a smaller problem with query- and key-range pieces, then a plain MHA one
    shapes = [Shape(1, 16, 4, 4096, 128, "fp16", True), Shape(1, 1, 1, 3000, 128, "bf16", True),
              Shape(2, 4, 4, 333, 64, "bf16", False)]
    for i, shape in enumerate(shapes):
        need = fa.fa_bwd_workspace_size(shape.B, shape.Hq, shape.Hkv, shape.N, shape.D)
        log("call", i, shape, "workspace", need)
        assert need <= fa.FA_NOALLOC_SCRATCH_BYTES
        qc, kc, vc, doc = make_inputs(shape, seed=900 + i)
        q, k, v, do = (t.cuda() for t in (qc, kc, vc, doc))
        o, lse = fa.fa_fwd(q, k, v, causal=shape.causal)
        ref = fa.fa_bwd(q, k, v, o, do, lse, causal=shape.causal)
        # outputs prefilled with NaN, so an element left unwritten shows
        outs = [torch.full_like(t, float("nan")) for t in ref]
        got = fa.fa_bwd_noalloc(q, k, v, o, do, lse, causal=shape.causal, dq=outs[0], dk=outs[1], dv=outs[2])
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"call {i}: {name} differs from fa_bwd"
        oracle = attention_backward(f64(qc), f64(kc), f64(vc), f64(doc), shape.scale, shape.causal)
        for name, g, r in zip(("dq", "dk", "dv"), got, oracle):
            assert_grad_close(f64(g), r, name, f"call {i}")


def test_noalloc_refuses_oversized_call():
    import torch
    import exact_attention_fa_amd as fa
    shape = Shape(1, 16, 4, 8192, 128, "bf16", True)  # 128.5 MiB of workspace
    assert fa.fa_bwd_workspace_size(shape.B, shape.Hq, shape.Hkv, shape.N, shape.D) > fa.FA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(1, 16, 8192, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 4, 8192, 128, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 16, 8192, dtype=torch.float32, device="cuda")
    dq = torch.full_like(q, 7.0)
    with pytest.raises(RuntimeError, match="80 MiB"):
        fa.fa_bwd_noalloc(q, k, k, q, q, lse, causal=True, dq=dq)
    torch.cuda.synchronize()
    assert bool((dq == 7.0).all())


def test_noalloc_graph_replay_matches_eager():
    """The callers this entry point is for capture it: fa_fwd and fa_bwd_noalloc in a HIP graph,
    replayed three times with new inputs copied in and eager fa_bwd calls in between, give the
    bits of the eager calls each time."""
    import torch
    import exact_attention_fa_amd as fa
    shape = Shape(2, 8, 2, 700, 128, "bf16", True)
    B, Hq, Hkv, N, D = shape.B, shape.Hq, shape.Hkv, shape.N, shape.D
    q, k, v, do = (t.cuda() for t in make_inputs(shape, seed=77))
    o, lse = torch.empty_like(q), torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        fa.fa_fwd(q, k, v, causal=True, out=o, lse=lse)
        fa.fa_bwd_noalloc(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # first call on the device resolves the scratch array's address, outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        new = make_inputs(shape, seed=80 + rep)
        for dst, src in zip((q, k, v, do), new):
            dst.copy_(src)
        log("replay", rep, shape)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv)]
        e_o, e_l = fa.fa_fwd(q, k, v, causal=True)
        e_g = fa.fa_bwd(q, k, v, e_o, do, e_l, causal=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, (e_o, e_l, *e_g)):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
