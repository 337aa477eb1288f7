"""The torch.library registration: shape propagation without a GPU; on the GPU, autograd
against the CPU oracle and the direct C-ABI calls, and torch.compile without a graph break."""
import pytest
import torch


def test_ops_registered_and_fake_shapes():
    from torch._subclasses.fake_tensor import FakeTensorMode
    import exact_attention_fa_amd.torch_op  # noqa: F401  (registers the ops)
    assert hasattr(torch.ops.fa_mi355x, "fwd") and hasattr(torch.ops.fa_mi355x, "bwd")
    with FakeTensorMode():
        q = torch.empty(2, 8, 100, 64, dtype=torch.bfloat16)
        k = torch.empty(2, 2, 100, 64, dtype=torch.bfloat16)
        o, lse = torch.ops.fa_mi355x.fwd(q, k, k, True, 0.125)
        assert o.shape == q.shape and o.dtype == q.dtype
        assert lse.shape == (2, 8, 100) and lse.dtype == torch.float32
        dq, dk, dv = torch.ops.fa_mi355x.bwd(q, k, k, o, o, lse, True, 0.125)
        assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == k.shape


def test_op_refuses_cpu_tensors():
    from exact_attention_fa_amd.torch_op import attention
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    with pytest.raises(RuntimeError):
        attention(q, q, q)


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [False, True])
def test_autograd_matches_oracle_and_direct_calls(causal):
    """Forward and autograd backward of the registered op against the CPU oracle (the parity
    tolerances), and bit for bit against the direct C-ABI calls it wraps."""
    import exact_attention_fa_amd as fa
    from exact_attention_fa_amd.torch_op import attention
    from exact_attention_fa_amd.inputs import Shape, make_inputs
    from parity_util import TOL_O, assert_fwd_close, assert_grad_close, f64
    from oracle import attention_backward, attention_forward
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    shape = Shape(2, 8, 2, 300, 128, "bf16", causal)
    qc, kc, vc, doc = make_inputs(shape, 31)
    q, k, v, do = (t.cuda() for t in (qc, kc, vc, doc))
    qr, kr, vr = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = attention(qr, kr, vr, causal=causal)
    o.backward(do)
    torch.cuda.synchronize()
    o_r, l_r = attention_forward(f64(qc), f64(kc), f64(vc), shape.scale, causal)
    eo = float(abs(f64(o) - o_r).max())  # the op returns O only; its LSE is checked below via fa_fwd
    assert eo <= TOL_O, f"torch op: O max-abs error {eo:.3e}"
    refs = attention_backward(f64(qc), f64(kc), f64(vc), f64(doc), shape.scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), (qr.grad, kr.grad, vr.grad), refs):
        assert_grad_close(f64(g), r, name, "torch op")
    o2, lse2 = fa.fa_fwd(q, k, v, causal=causal)
    dq2, dk2, dv2 = fa.fa_bwd(q, k, v, o2, do, lse2, causal=causal)
    torch.cuda.synchronize()
    assert_fwd_close(f64(o2), f64(lse2), o_r, l_r, "fa_fwd under the op")
    assert torch.equal(o.detach(), o2)
    assert torch.equal(qr.grad, dq2) and torch.equal(kr.grad, dk2) and torch.equal(vr.grad, dv2)


@pytest.mark.gpu
def test_compiles_without_graph_break():
    from exact_attention_fa_amd.torch_op import attention
    from exact_attention_fa_amd.inputs import Shape, make_inputs
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    q, k, v, _ = (t.cuda() for t in make_inputs(Shape(1, 4, 4, 200, 64, "fp16", True), 37))

    def f(q, k, v):
        return attention(q, k, v, causal=True)

    compiled = torch.compile(f, fullgraph=True, backend="aot_eager")
    o1 = compiled(q, k, v)
    o2 = f(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
