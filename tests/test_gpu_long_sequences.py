"""Sequences far longer than the benchmarked ones (N = 131072 and 65536): head offsets, tile
counts and grid sizes well away from the small cases.

The forward, and the backward's dQ, are compared with the oracle on sampled rows (a row's O,
LSE and dQ need only that row's scores).  dK and dV need every row's statistics, too slow for
the oracle at this length, so they are checked through properties that hold at any size:
  * every row of dS sums to zero, so sum_j dK_j = 0;
  * every row of P sums to one, so sum_j dV_j = sum over the group's query heads of sum_i dO_i;
  * causal: only the last query sees the last key, so dV_{N-1} and dK_{N-1} are single terms,
    built from the oracle's O and LSE of row N-1.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LONG = [
    # (B, Hq, Hkv, N, D, dtype, causal)
    (1, 2, 1, 131072, 128, "bf16", False),
    (1, 4, 1, 65536, 64, "fp16", True),
]


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


@pytest.mark.parametrize("dims", LONG, ids=[f"H{h}/{hk}N{n}D{d}{t}{'c' if cz else ''}" for _, h, hk, n, d, t, cz in LONG])
def test_long_sequence(dims):
    import torch
    import exact_attention_fa_amd as fa
    from exact_attention_fa_amd.inputs import Shape, make_inputs
    from parity_util import TOL_GRAD, assert_fwd_close, f64
    from oracle import attention_dq_rows, attention_forward

    B, Hq, Hkv, N, D, dtype, causal = dims
    shape = Shape(B, Hq, Hkv, N, D, dtype, causal)
    log("long sequence", shape)
    q, k, v, do = (t.cuda() for t in make_inputs(shape, 4242 + N // 1024))
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    scale = shape.scale
    grp = Hq // Hkv

    # forward: sampled rows of every query head against the oracle
    rng = np.random.default_rng(N)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, N // 2, N - 65, N - 64, N - 1],
                                     rng.choice(N, size=24, replace=False)]))
    qh, kh, vh = f64(q), f64(k), f64(v)
    o_ref, lse_ref = attention_forward(qh, kh, vh, scale, causal, rows=rows)
    eo, el = assert_fwd_close(f64(o)[:, :, rows], f64(lse)[:, :, rows], o_ref, lse_ref, str(shape))
    log("  forward sampled rows: O err %.2e, LSE err %.2e" % (eo, el))

    # backward, dQ of the sampled rows: a row's gradient needs only that row's statistics
    dq_ref = attention_dq_rows(qh, kh, vh, f64(do), scale, causal, rows)
    e_dq = float(np.abs(f64(dq)[:, :, rows] - dq_ref).max() / max(np.abs(dq_ref).max(), 1e-2))
    log("  dQ sampled rows relative error %.2e" % e_dq)
    assert e_dq <= TOL_GRAD, f"{shape}: sampled dQ rows relative error {e_dq:.3e}"

    # backward: sum_j dK_j = 0 and sum_j dV_j = sum_group sum_i dO_i, per KV head and column
    dk64, dv64, do64 = dk.double(), dv.double(), do.double()
    resid = dk64.sum(dim=2).abs()
    mass = dk64.abs().sum(dim=2)
    r_dk = float((resid / mass).max())
    tot = do64.reshape(B, Hkv, grp, N, D).sum(dim=(2, 3))
    e_dv = float((dv64.sum(dim=2) - tot).abs().max()) / float(tot.abs().max())
    log("  sum_j dK_j / sum_j |dK_j| %.2e; sum_j dV_j error %.2e" % (r_dk, e_dv))
    assert r_dk < 2e-2 and e_dv < 2e-2
    assert bool(torch.isfinite(dq).all()) and bool(torch.isfinite(dk).all()) and bool(torch.isfinite(dv).all())

    if causal:
        # the last key: one term per query head, from row N-1's oracle statistics
        last = np.array([N - 1])
        o_l, lse_l = attention_forward(qh, kh, vh, scale, causal, rows=last)
        dh = f64(do)[:, :, N - 1]
        dv_ref = np.zeros((B, Hkv, D))
        dk_ref = np.zeros((B, Hkv, D))
        for hq in range(Hq):
            kv = hq // grp
            qv, kvv, vv = qh[:, hq, N - 1], kh[:, kv, N - 1], vh[:, kv, N - 1]
            p = np.exp(scale * np.sum(qv * kvv, axis=-1) - lse_l[:, hq, 0])          # P_{N-1,N-1}
            dp = np.sum(dh[:, hq] * vv, axis=-1)
            delta = np.sum(dh[:, hq] * o_l[:, hq, 0], axis=-1)
            dv_ref[:, kv] += p[:, None] * dh[:, hq]
            dk_ref[:, kv] += scale * (p * (dp - delta))[:, None] * qv
        for name, g, r in (("dV", f64(dv)[:, :, N - 1], dv_ref), ("dK", f64(dk)[:, :, N - 1], dk_ref)):
            e = float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-30))
            log("  last key %s relative error %.2e" % (name, e))
            assert e <= TOL_GRAD, f"{shape}: last key {name} relative error {e:.3e}"
