"""HuggingFace ``transformers`` integration: routes a model's attention through the fused
kernels.

    from exact_attention_fa_amd.hf_attention import register
    register()                                   # adds the "fa_mi355x" implementation
    model = AutoModelForCausalLM.from_config(cfg, attn_implementation="fa_mi355x")

One call switches a model's attention modules to the fused kernel ("FlashAttention for Tesla
P100", sections "Quick start" and "Driving a real model"); the op is the registered
``torch.ops.fa_mi355x`` custom operator, so autograd and ``torch.compile`` see one node
("FlashNystrom", section "PyTorch compatibility").

What the kernels do not offer is refused, never approximated ("FlashAttention for Tesla
P100", section "What it supports"): padding or arbitrary masks, attention dropout while
training, sliding windows, soft-capping, and query/key lengths that differ (KV-cache
decoding).  Only argument checks and layout changes happen here; the attention itself runs in
the HIP kernels.
"""
from __future__ import annotations

NAME = "fa_mi355x"


def mask_for_fused(batch_size, q_length, kv_length, q_offset=0, kv_offset=0, mask_function=None,
                   attention_mask=None, **kwargs):
    """The model-side mask for this implementation: None when every token is visible apart from
    the causal structure (the kernel applies that itself), else the 2-D padding mask, which
    the attention call then refuses."""
    if attention_mask is None:
        return None
    am = attention_mask[:, -kv_length:]
    if am.shape[1] == kv_length and bool(am.all()):
        return None
    return am


def attention_forward(module, query, key, value, attention_mask, dropout: float = 0.0, scaling=None,
                      is_causal=None, **kwargs):
    """The attention function transformers calls per layer: query (B, Hq, N, D), key and value
    (B, Hkv, N, D); returns (output (B, N, Hq, D), None)."""
    from .torch_op import attention

    if attention_mask is not None:
        raise NotImplementedError(f"{NAME}: padding or arbitrary attention masks are not supported")
    if dropout and getattr(module, "training", False):
        raise NotImplementedError(f"{NAME}: attention dropout is not supported")
    for unsupported in ("sliding_window", "softcap", "s_aux"):
        if kwargs.get(unsupported) is not None:
            raise NotImplementedError(f"{NAME}: {unsupported} is not supported")
    if kwargs.get("output_attentions"):
        raise NotImplementedError(f"{NAME}: attention weights are never materialised")
    if query.shape[2] != key.shape[2]:
        raise NotImplementedError(f"{NAME}: query and key lengths differ (KV-cache decoding is not supported)")
    causal = getattr(module, "is_causal", True) if is_causal is None else bool(is_causal)
    causal = causal and query.shape[2] > 1
    out = attention(query.contiguous(), key.contiguous(), value.contiguous(), causal=causal,
                    softmax_scale=scaling)
    return out.transpose(1, 2).contiguous(), None


def register(name: str = NAME, fn=None) -> str:
    """Registers the attention function (or `fn`, a wrapper of it) and its mask function with
    transformers under `name`; returns the name to pass as ``attn_implementation``."""
    from transformers import AttentionInterface
    from transformers.masking_utils import AttentionMaskInterface

    AttentionInterface.register(name, fn or attention_forward)
    AttentionMaskInterface.register(name, mask_for_fused)
    return name
