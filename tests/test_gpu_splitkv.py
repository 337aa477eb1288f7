"""GPU parity of the small-grid paths against the CPU oracle, through the C ABI: the
split-key-range forward (fa_fwd_splitkv), the merge of partial results (fa_merge_partials),
and the backward's query- and key-range pieces on the per-GPU share of a head-sharded
long-context problem.

The merge is checked on partials the oracle computes itself (attention over disjoint slices
of the keys, plus an empty part), so it is pinned to the oracle's full result independently
of the forward kernels.
"""
import sys
import zlib

import numpy as np
import pytest

from exact_attention_fa_amd.inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu


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


SPLIT = [
    # (B, Hq, Hkv, N, D, dtype, causal, n_split); 0 = the library's choice
    (1, 2, 1, 1500, 128, "bf16", False, 3),
    (1, 2, 2, 1000, 64, "fp16", True, 5),
    (1, 1, 1, 4096, 128, "bf16", True, 0),
    (2, 3, 1, 333, 128, "fp16", True, 7),     # many pieces hold no key of the short rows
    (1, 1, 1, 64, 64, "bf16", False, 2),      # one tile: the first piece is empty
    (1, 4, 2, 2049, 64, "bf16", False, 64),   # the most pieces, ragged
]


@pytest.mark.parametrize("dims", SPLIT, ids=[f"B{b}H{hq}/{hk}N{n}D{d}{t}{'c' if cz else ''}S{s}"
                                              for b, hq, hk, n, d, t, cz, s in SPLIT])
def test_splitkv_full(dims):
    import torch
    import exact_attention_fa_amd as fa
    from parity_util import assert_fwd_close, attention_forward, f64
    B, Hq, Hkv, N, D, dtype, causal, n_split = dims
    shape = Shape(B, Hq, Hkv, N, D, dtype, causal)
    log("splitkv", shape, "n_split", n_split, "resolved", n_split or fa.fa_fwd_splitkv_parts(B, Hq, Hkv, N, D, causal))
    q, k, v, _ = make_inputs(shape, seed=zlib.crc32(repr(dims).encode()) % (1 << 31), with_grad=False)
    dev = torch.device("cuda", 0)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o, lse = fa.fa_fwd_splitkv(qd, kd, vd, causal=causal, n_split=n_split)
    o2, lse2 = fa.fa_fwd_splitkv(qd, kd, vd, causal=causal, n_split=n_split)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "split forward is not deterministic"
    o_ref, lse_ref = attention_forward(f64(q), f64(k), f64(v), shape.scale, causal)
    log("  errors", assert_fwd_close(f64(o), f64(lse), o_ref, lse_ref, str(shape)))


def test_splitkv_auto_on_one_head_long_sequence():
    """The per-GPU share of a head-sharded long-context problem (one head, N = 16384, causal):
    the library splits it, and sampled rows match the oracle."""
    import torch
    import exact_attention_fa_amd as fa
    from parity_util import assert_fwd_close, attention_forward, f64
    shape = Shape(1, 1, 1, 16384, 128, "bf16", True, 0.5)
    n = fa.fa_fwd_splitkv_parts(1, 1, 1, 16384, 128, True)
    assert n > 1
    q, k, v, _ = make_inputs(shape, seed=4242, with_grad=False)
    dev = torch.device("cuda", 0)
    o, lse = fa.fa_fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 63, 64, 8191, 16383], rng.choice(16384, 60, replace=False)]))
    o_ref, lse_ref = attention_forward(f64(q), f64(k), f64(v), shape.scale, True, rows=rows)
    log("  n", n, "errors", assert_fwd_close(f64(o)[:, :, rows], f64(lse)[:, :, rows], o_ref, lse_ref, str(shape)))


def test_backward_pieces_on_one_head_long_sequence():
    """One head, N = 16384, causal: the backward cuts the dK/dV pass's query ranges and the dQ
    pass's key ranges into pieces; sampled rows and keys match the oracle."""
    import exact_attention_fa_amd as fa
    from parity_util import sampled_check
    shape = Shape(1, 1, 1, 16384, 128, "bf16", True, 0.5)
    ws = fa.fa_bwd_workspace_size(1, 1, 1, 16384, 128)
    rows = 16384
    assert ws > 2 * rows * 4 + 3 * rows * 128 * 4, "expected partial buffers for the pieces"
    errs, _ = sampled_check(shape, 4343, units=[(0, 0)], n_rows=48, backward=True)
    log("  errors", errs)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp16", 64)])
def test_merge_partials_against_oracle(dtype, D):
    import torch
    import exact_attention_fa_amd as fa
    from oracle import softmax_probs
    from parity_util import assert_fwd_close, attention_forward, f64
    shape = Shape(2, 3, 3, 700, D, dtype, False)
    q, k, v, _ = make_inputs(shape, seed=99, with_grad=False)
    qs, ks, vs = f64(q), f64(k), f64(v)
    cuts = [0, 100, 101, 450, 700]                     # key slices 100, 1, 349, 250 long
    rows = np.arange(shape.N)
    o_parts, l_parts = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        # the oracle's softmax over the slice's keys alone, then P V of the slice
        o_s = np.zeros_like(qs)
        l_s = np.zeros(qs.shape[:3])
        for bi in range(shape.B):
            for h in range(shape.Hq):
                _, P, L = softmax_probs(qs[bi, h], ks[bi, h, a:b], shape.scale, rows, False)
                o_s[bi, h] = P @ vs[bi, h, a:b]
                l_s[bi, h] = L
        o_parts.append(o_s)
        l_parts.append(l_s)
    o_parts.insert(2, np.zeros_like(o_parts[0]))      # a part with no key at all
    l_parts.insert(2, np.full_like(l_parts[0], -np.inf))
    dev = torch.device("cuda", 0)
    op = torch.tensor(np.stack(o_parts), dtype=torch.float32, device=dev)
    lp = torch.tensor(np.stack(l_parts), dtype=torch.float32, device=dev)
    out = torch.empty(q.shape, dtype=q.dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    fa.fa_merge_partials(op, lp, out, lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_forward(qs, ks, vs, shape.scale, False)
    log("  errors", assert_fwd_close(f64(out), f64(lse), o_ref, lse_ref, "merge"))
    # every part empty: o = 0, lse = -inf
    lp.fill_(float("-inf"))
    fa.fa_merge_partials(op, lp, out, lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
