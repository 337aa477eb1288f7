"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI, run the
oracle on the same seeded inputs, compare with the stated tolerances.

Tolerances (float; inputs bf16/fp16, fp32 accumulation):
  O    max |O_gpu - O_ref|                    <= 1e-2
  LSE  max |LSE_gpu - LSE_ref|                <= 1e-3
  dQ, dK, dV  max |g - g_ref| / max(max |g_ref|, 1e-2)   <= 2e-2   (per tensor)
The 1e-2 floor only matters when the exact gradient vanishes (e.g. N = 1, where
dS = P (dP - D) = 0): the check then becomes an absolute bound of 2e-4.
"""
from __future__ import annotations

import numpy as np
import torch

import exact_attention_fa_amd as fa
from exact_attention_fa_amd.inputs import Shape, make_inputs
from oracle import attention_backward, attention_forward

TOL_O = 1e-2
TOL_LSE = 1e-3
TOL_GRAD = 2e-2
GRAD_FLOOR = 1e-2


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_forward(q, k, v, causal, scale):
    dev = torch.device("cuda", 0)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return o, lse


def gpu_backward(q, k, v, o, do, lse, causal, scale):
    dev = torch.device("cuda", 0)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, dod, lse, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def rel_err(g, ref):
    return float(np.abs(g - ref).max() / max(np.abs(ref).max(), GRAD_FLOOR))


def derived_o_tol(v, dtype: str) -> float:
    """Bound on |O_gpu - O_ref| from the arithmetic, for scales other than 1/sqrt(D).

    P is rounded to the input type as an MFMA operand (relative error <= u/2 per weight, so
    |dO| <= (u/2) max|V|) and O is rounded once on output (<= u |O| <= u max|V|), with u the
    unit roundoff step 2^-8 (bf16) or 2^-11 (fp16).  Peaked softmax rows (large scales) push
    |O| towards max|V|, where the fixed 1e-2 bound of the configured workloads no longer
    leaves room for the output rounding alone.
    """
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    return max(TOL_O, 1.5 * u * float(np.abs(v).max()))


def assert_fwd_close(o_gpu, lse_gpu, o_ref, lse_ref, what="", tol_o=TOL_O):
    eo = float(np.abs(o_gpu - o_ref).max())
    el = float(np.abs(lse_gpu - lse_ref).max())
    assert np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all(), what
    assert eo <= tol_o, f"{what}: O max-abs error {eo:.3e} > {tol_o:.3e}"
    assert el <= TOL_LSE, f"{what}: LSE max-abs error {el:.3e} > {TOL_LSE}"
    return eo, el


def assert_grad_close(g, ref, name, what=""):
    assert np.isfinite(g).all(), f"{what}: {name} has non-finite values"
    e = rel_err(g, ref)
    assert e <= TOL_GRAD, f"{what}: {name} relative max error {e:.3e} > {TOL_GRAD}"
    return e


def full_check(shape: Shape, seed: int, backward: bool = True, scale=None):
    """Element-by-element comparison of every output against the oracle.

    At the workloads' scale 1/sqrt(D) the O bound is the fixed 1e-2; for other scales it is
    the bound derived from the arithmetic (``derived_o_tol``).
    """
    default_scale = scale is None
    scale = shape.scale if scale is None else scale
    q, k, v, do = make_inputs(shape, seed)
    o, lse = gpu_forward(q, k, v, shape.causal, scale)
    o_ref, lse_ref = attention_forward(f64(q), f64(k), f64(v), scale, shape.causal)
    tol_o = TOL_O if default_scale else derived_o_tol(f64(v), shape.dtype)
    errs = dict(zip(("o", "lse"), assert_fwd_close(f64(o), f64(lse), o_ref, lse_ref, str(shape), tol_o)))
    if backward:
        dq, dk, dv = gpu_backward(q, k, v, o, do, lse, shape.causal, scale)
        dq_r, dk_r, dv_r = attention_backward(f64(q), f64(k), f64(v), f64(do), scale, shape.causal)
        for name, g, r in (("dq", dq, dq_r), ("dk", dk, dk_r), ("dv", dv, dv_r)):
            errs[name] = assert_grad_close(f64(g), r, name, str(shape))
    return errs


def sampled_check(shape: Shape, seed: int, units, n_rows: int, backward: bool, rng_seed: int = 0):
    """Full-size GPU run; the oracle recomputes sampled outputs of some (batch, kv-group) units.

    ``units`` lists (b, kv) pairs; each unit is the sub-problem of KV head kv of batch b and
    its Hq/Hkv query heads, which the oracle solves exactly (heads are independent).  Within
    a unit, ``n_rows`` query rows (for O, LSE, dQ) and ``n_rows`` keys (for dK, dV) are
    compared, always including the first and last index and the start of the last tile.
    """
    q, k, v, do = make_inputs(shape, seed, with_grad=backward)
    o, lse = gpu_forward(q, k, v, shape.causal, shape.scale)
    grads = gpu_backward(q, k, v, o, do, lse, shape.causal, shape.scale) if backward else None
    o_h, lse_h = f64(o), f64(lse)
    if backward:
        dq_h, dk_h, dv_h = (f64(t) for t in grads)
    rng = np.random.default_rng(rng_seed)
    N, grp = shape.N, shape.Hq // shape.Hkv
    errs = {"o": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b, kv in units:
        hs = slice(kv * grp, (kv + 1) * grp)
        must = [0, N - 1, max(0, (N - 1) // 64 * 64), N // 2]
        idx = np.unique(np.concatenate([must, rng.choice(N, size=min(n_rows, N), replace=False)]))
        qs, ks, vs = f64(q[b:b + 1, hs]), f64(k[b:b + 1, kv:kv + 1]), f64(v[b:b + 1, kv:kv + 1])
        o_ref, lse_ref = attention_forward(qs, ks, vs, shape.scale, shape.causal, rows=idx)
        eo, el = assert_fwd_close(o_h[b:b + 1, hs][:, :, idx], lse_h[b:b + 1, hs][:, :, idx], o_ref, lse_ref,
                                  f"{shape} unit {(b, kv)}")
        errs["o"], errs["lse"] = max(errs["o"], eo), max(errs["lse"], el)
        if backward:
            dos = f64(do[b:b + 1, hs])
            dq_r, dk_r, dv_r = attention_backward(qs, ks, vs, dos, shape.scale, shape.causal, rows=idx, keys=idx)
            # relative errors are normalised by the largest reference value of the sample
            for name, g, r in (("dq", dq_h[b:b + 1, hs][:, :, idx], dq_r),
                               ("dk", dk_h[b:b + 1, kv:kv + 1][:, :, idx], dk_r),
                               ("dv", dv_h[b:b + 1, kv:kv + 1][:, :, idx], dv_r)):
                errs[name] = max(errs[name], assert_grad_close(g, r, name, f"{shape} unit {(b, kv)}"))
    return errs, (o, lse, grads)


def bench_path_run(shape: Shape, seed: int, scale=None):
    """The launch configuration bench.py times: fa_fwd_splitkv with the library's choice of
    key-range pieces, then the four backward stages on one workspace.  Returns the CPU inputs
    and the GPU outputs."""
    dev = torch.device("cuda", 0)
    scale = shape.scale if scale is None else scale
    q, k, v, do = make_inputs(shape, seed)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    B, Hq, Hkv, N, D = shape.B, shape.Hq, shape.Hkv, shape.N, shape.D
    n = fa.fa_fwd_splitkv_parts(B, Hq, Hkv, N, D, shape.causal)
    o, lse = fa.fa_fwd_splitkv(qd, kd, vd, causal=shape.causal, softmax_scale=scale, n_split=n)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    fa.fa_bwd_preprocess(o, dod, lse, ws, Hkv)
    fa.fa_bwd_dkdv(qd, kd, vd, dod, dk, dv, ws, causal=shape.causal, softmax_scale=scale)
    fa.fa_bwd_dq(qd, kd, vd, dod, dq, ws, causal=shape.causal, softmax_scale=scale)
    fa.fa_bwd_postprocess(dk, dv, ws, Hq)
    torch.cuda.synchronize()
    return (q, k, v, do), (o, lse, dq, dk, dv)


def unit_full_check(shape: Shape, inputs, outputs, units, backward=True, scale=None):
    """Every row of O, LSE (and dQ) of the query heads of each (batch, kv-group) unit, and every
    key of its dK, dV, against the oracle solving that unit alone (heads are independent)."""
    scale = shape.scale if scale is None else scale
    q, k, v, do = inputs
    o, lse, dq, dk, dv = (f64(t) for t in outputs)
    grp = shape.Hq // shape.Hkv
    errs = {"o": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b, kv in units:
        hs = slice(kv * grp, (kv + 1) * grp)
        what = f"{shape} unit {(b, kv)}"
        qs, ks, vs = f64(q[b:b + 1, hs]), f64(k[b:b + 1, kv:kv + 1]), f64(v[b:b + 1, kv:kv + 1])
        o_r, l_r = attention_forward(qs, ks, vs, scale, shape.causal)
        eo, el = assert_fwd_close(o[b:b + 1, hs], lse[b:b + 1, hs], o_r, l_r, what)
        errs["o"], errs["lse"] = max(errs["o"], eo), max(errs["lse"], el)
        if backward:
            dq_r, dk_r, dv_r = attention_backward(qs, ks, vs, f64(do[b:b + 1, hs]), scale, shape.causal)
            for name, g, r in (("dq", dq[b:b + 1, hs], dq_r), ("dk", dk[b:b + 1, kv:kv + 1], dk_r),
                               ("dv", dv[b:b + 1, kv:kv + 1], dv_r)):
                errs[name] = max(errs[name], assert_grad_close(g, r, name, what))
    return errs



def unit_roundoff(dtype: str) -> float:
    """Relative rounding bound of round-to-nearest-even into the 16-bit type."""
    return 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11


def grad_error_bound(q, k, v, do, o_gpu, lse_gpu, scale, causal, dtype):
    """Elementwise bound on |g_gpu - g_exact| for dQ, dK, dV (float64 arrays of their shapes),
    derived from the arithmetic of the backward, for inputs where the fixed relative tolerance
    does not apply (nearly one-hot rows make the exact gradients a cancellation).

    With P, dP, D the exact values (float64, from the definition), u the 16-bit unit roundoff
    and e = 2^-24 the fp32 one, the kernels form
      P^    = exp2(S^ c2 - LSE^ log2 e): relative error eta <= |LSE^ - LSE| + the fp32 error of
              the score products (D e sum_d |Q K|, scaled) and of the exponent's FMA and exp2;
      dP^   = dO V^T in fp32: |dP^ - dP| <= D e sum_d |dO V|;
      D^    = dO . O^ from the stored 16-bit O^: |D^ - D| = |dO . (O^ - O)| (measured from the
              GPU's own O) + D e sum_d |dO O^|;
      dS^   = P^ (dP^ - D^), rounded to the 16-bit type as an MFMA operand (relative u; fp16
              adds 2^-25 absolute for subnormals);
      dQ    = scale dS^ K, dK = scale dS^T Q, dV = P^T dO (P rounded like dS), summed in fp32
              (n e of the absolute sum) and rounded once on output (relative u).
    Each first-order term is bounded by its absolute value; the bound is returned without
    safety factor (callers add one for second-order terms)."""
    q, k, v, do, o_gpu, lse_gpu = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do, o_gpu, lse_gpu))
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    u, e = unit_roundoff(dtype), 2.0 ** -24
    sub = 2.0 ** -25 if dtype == "fp16" else 0.0
    o_ref, lse_ref = attention_forward(q, k, v, scale, causal)
    bdq = np.zeros_like(q)
    bdk = np.zeros_like(k)
    bdv = np.zeros_like(v)
    idx = np.arange(N)
    vis = (idx[None, :] <= idx[:, None]) if causal else np.ones((N, N), dtype=bool)
    for b in range(B):
        for hq in range(Hq):
            kv = hq // grp
            Q, K, V, dO = q[b, hq], k[b, kv], v[b, kv], do[b, hq]
            S = scale * (Q @ K.T)
            P = np.where(vis, np.exp(np.where(vis, S, 0.0) - lse_ref[b, hq][:, None]), 0.0)
            dP = dO @ V.T
            Dex = np.einsum("nd,nd->n", dO, o_ref[b, hq])
            absS = abs(scale) * (np.abs(Q) @ np.abs(K).T)
            eta = (np.abs(lse_gpu[b, hq] - lse_ref[b, hq])[:, None] + D * e * absS
                   + 4 * e * (np.abs(S) + np.abs(lse_ref[b, hq])[:, None]) * 1.4427 + 4 * e)
            g_dp = D * e * (np.abs(dO) @ np.abs(V).T)
            dD = (np.abs(np.einsum("nd,nd->n", dO, o_gpu[b, hq] - o_ref[b, hq]))
                  + D * e * np.einsum("nd,nd->n", np.abs(dO), np.abs(o_gpu[b, hq])) + 2 * e * np.abs(Dex))
            dS = P * (dP - Dex[:, None])
            E = (P * (eta * np.abs(dP - Dex[:, None]) + (1 + eta) * (g_dp + dD[:, None]))) * (1 + u) \
                + u * np.abs(dS) + sub
            E = np.where(vis, E, 0.0)
            absdS = np.abs(dS) + E
            bdq[b, hq] += abs(scale) * (E @ np.abs(K) + N * e * (absdS @ np.abs(K)))
            bdk[b, kv] += abs(scale) * (E.T @ np.abs(Q) + N * e * (absdS.T @ np.abs(Q)))
            EP = np.where(vis, P * (eta + u + eta * u) + sub, 0.0)
            bdv[b, kv] += EP.T @ np.abs(dO) + N * e * (P.T @ np.abs(dO))
    dq_r, dk_r, dv_r = attention_backward(q, k, v, do, scale, causal)
    # the fp32 sums of the group's partials, then one rounding of each output
    bdk += grp * e * np.abs(dk_r)
    bdv += grp * e * np.abs(dv_r)
    bounds = [bd + u * (np.abs(r) + bd) for bd, r in ((bdq, dq_r), (bdk, dk_r), (bdv, dv_r))]
    return bounds, (dq_r, dk_r, dv_r)


def assert_within_bound(g, ref, bound, name, what="", safety=1.25):
    """|g - ref| <= safety * bound elementwise (plus 1e-9 of the largest reference value)."""
    g = np.asarray(g, dtype=np.float64)
    assert np.isfinite(g).all(), f"{what}: {name} has non-finite values"
    err = np.abs(g - ref)
    lim = safety * bound + 1e-9 * max(float(np.abs(ref).max()), 1e-30)
    worst = float((err / lim).max())
    assert worst <= 1.0, f"{what}: {name} exceeds its derived bound (worst error / bound = {worst:.3f})"
    return worst
