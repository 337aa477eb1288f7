"""The HuggingFace attention hook: registration and refusals without a GPU; on the GPU, a small
randomly initialised Llama-style model (grouped-query heads, built in-process, no download)
whose layers run through the fused kernels, with one layer's attention output compared with
the oracle on that layer's own q, k, v."""
import pytest
import torch

transformers = pytest.importorskip("transformers")


def small_llama(attn):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(vocab_size=512, hidden_size=512, intermediate_size=1024, num_hidden_layers=2,
                      num_attention_heads=8, num_key_value_heads=2, max_position_embeddings=1024,
                      attn_implementation=attn)
    torch.manual_seed(0)
    return LlamaForCausalLM(cfg)


def test_register_and_refusals():
    from exact_attention_fa_amd import hf_attention as hf
    from transformers import AttentionInterface
    name = hf.register()
    assert name in AttentionInterface._global_mapping
    ones = torch.ones(2, 16, dtype=torch.bool)
    assert hf.mask_for_fused(2, 16, 16, attention_mask=ones) is None
    pad = ones.clone()
    pad[0, :3] = False
    assert hf.mask_for_fused(2, 16, 16, attention_mask=pad) is not None
    q = torch.zeros(1, 4, 16, 64, dtype=torch.bfloat16)
    mod = torch.nn.Module()
    with pytest.raises(NotImplementedError, match="mask"):
        hf.attention_forward(mod, q, q, q, pad)
    with pytest.raises(NotImplementedError, match="decoding"):
        hf.attention_forward(mod, q[:, :, :1], q, q, None)
    with pytest.raises(NotImplementedError, match="sliding_window"):
        hf.attention_forward(mod, q, q, q, None, sliding_window=8)


def test_model_on_host_memory_raises():
    """No silent fallback: the fused path refuses host tensors."""
    from exact_attention_fa_amd import hf_attention as hf
    model = small_llama(hf.register())
    ids = torch.randint(0, 512, (1, 32))
    with pytest.raises(RuntimeError, match="GPU"):
        model(ids)


@pytest.mark.gpu
def test_llama_layer_matches_oracle():
    import numpy as np
    from exact_attention_fa_amd import hf_attention as hf
    from oracle import attention_forward as oracle_forward
    from parity_util import TOL_O, f64
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    seen = []

    def recording(module, query, key, value, attention_mask, **kw):
        out, w = hf.attention_forward(module, query, key, value, attention_mask, **kw)
        seen.append((module.layer_idx, query.detach().clone(), key.detach().clone(), value.detach().clone(),
                     out.detach().clone(), kw.get("scaling")))
        return out, w

    name = hf.register("fa_mi355x_recording", recording)
    model = small_llama(name).to(device="cuda", dtype=torch.bfloat16)
    ids = torch.randint(0, 512, (2, 200), generator=torch.Generator().manual_seed(3)).cuda()
    logits = model(ids).logits
    logits.float().logsumexp(-1).mean().backward()   # autograd through the fused op
    torch.cuda.synchronize()
    assert torch.isfinite(logits.float()).all()
    assert all(p.grad is None or torch.isfinite(p.grad.float()).all() for p in model.parameters())
    assert sorted({s[0] for s in seen}) == [0, 1]
    layer, q, k, v, out, scaling = next(s for s in seen if s[0] == 1)
    assert q.shape == (2, 8, 200, 64) and k.shape == (2, 2, 200, 64)
    o_ref, _ = oracle_forward(f64(q), f64(k), f64(v), scaling, True)
    err = float(np.abs(f64(out.transpose(1, 2)) - o_ref).max())
    assert err <= TOL_O, f"layer {layer}: attention output max-abs error {err:.3e}"
