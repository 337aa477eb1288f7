"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on seeded inputs.

Small shapes are compared element by element on every output; the full-size workloads
are run exactly as the benchmark launches them and compared on sampled outputs that the
oracle recomputes one (batch, kv-group) unit at a time.
"""
import sys
import zlib

import pytest

from exact_attention_fa_amd.inputs import WORKLOADS, Shape, workload_seed

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


# ------------------------------------------------------------ tiny workload (full oracle)

@pytest.mark.parametrize("variant", [0, 1], ids=["noncausal", "causal"])
def test_tiny_fp16_full(variant):
    from parity_util import full_check
    shape = WORKLOADS["tiny_fp16"][variant]
    log("tiny", shape)
    errs = full_check(shape, workload_seed("tiny_fp16", variant))
    log("  errors", errs)


# ------------------------------------------------ small shapes spanning tiles and tails

SMALL = [
    # (B, Hq, Hkv, N, D)
    (1, 2, 2, 1, 64),        # single token
    (1, 2, 1, 7, 128),       # shorter than one MFMA block
    (2, 4, 1, 129, 64),      # MQA, one row past a tile
    (1, 6, 2, 333, 128),     # GQA 3:1, ragged
    (1, 2, 2, 640, 64),      # several whole tiles
    (2, 4, 4, 517, 128),     # MHA, ragged, B=2
    (1, 16, 1, 300, 128),    # MQA, sixteen query heads summed into one K/V gradient
]


@pytest.mark.parametrize("dims", SMALL, ids=[f"B{b}H{hq}/{hk}N{n}D{d}" for b, hq, hk, n, d in SMALL])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True], ids=["nc", "causal"])
def test_small_full(dims, dtype, causal):
    from parity_util import full_check
    B, Hq, Hkv, N, D = dims
    shape = Shape(B, Hq, Hkv, N, D, dtype, causal)
    log("small", shape)
    full_check(shape, seed=zlib.crc32(repr((dims, dtype, causal)).encode()) % (1 << 31))


# Grids large enough for the 256-query workgroups (B*Hq*ceil(N/256) >= 512), and non-causal
# grids of 128-query tiles that fill every CU with two 4-wave workgroups
# (B*Hq*ceil(N/128) >= 512); everything smaller, and every other causal grid, takes the
# workgroups that split the key range over two wave groups (the small shapes above).  Ragged
# sequence ends, compared element by element.
LARGE_GRID = [
    (4, 32, 8, 1000, 128, "bf16", False),
    (4, 32, 32, 777, 64, "fp16", True),
    (2, 64, 16, 1030, 128, "fp16", True),
    (2, 64, 16, 1030, 128, "bf16", True),   # bf16 causal on the 256-query forward workgroups
    (2, 32, 8, 1000, 64, "fp16", False),
    (1, 64, 64, 900, 128, "bf16", False),
    # split key range over many tiles per group, GQA, ragged; these grids are also small
    # enough for the backward to cut query and key ranges into pieces (2-3 here)
    (1, 8, 2, 2000, 128, "bf16", False),
    (1, 8, 8, 1500, 64, "fp16", True),
    # tiny grids: many backward pieces (dK/dV 5 and dQ 11; dK/dV 4 and dQ 4)
    (1, 1, 1, 3000, 128, "bf16", True),
    (1, 2, 1, 4100, 64, "fp16", False),
]


@pytest.mark.parametrize("dims", LARGE_GRID, ids=[f"B{b}H{hq}/{hk}N{n}D{d}{t}{'c' if cz else ''}"
                                                  for b, hq, hk, n, d, t, cz in LARGE_GRID])
def test_large_grid_full(dims):
    from parity_util import full_check
    B, Hq, Hkv, N, D, dtype, causal = dims
    shape = Shape(B, Hq, Hkv, N, D, dtype, causal)
    log("large grid", shape)
    full_check(shape, seed=zlib.crc32(repr(dims).encode()) % (1 << 31))


# Scores that rise along the key axis, so that later key tiles far exceed the running maximum
# set by the first tile: the forward must move its reference and rescale (including scores
# large enough to overflow exp2 against the old reference).  The grids are large enough for
# the 256-query workgroups.  Inputs: the seeded draw with key row j multiplied by
# 1 + (R - 1) j / (N - 1).
RISING = [
    (4, 32, 8, 1000, 128, "bf16", False, 4.0),
    (4, 32, 8, 1000, 128, "bf16", False, 40.0),
    (2, 64, 16, 1030, 128, "fp16", True, 6.0),
    (4, 32, 32, 777, 64, "fp16", False, 30.0),
]


@pytest.mark.parametrize("dims", RISING, ids=[f"B{b}H{hq}/{hk}N{n}D{d}{t}{'c' if cz else ''}R{r:g}"
                                              for b, hq, hk, n, d, t, cz, r in RISING])
def test_rising_scores_full(dims):
    import numpy as np
    import torch
    from parity_util import (assert_fwd_close, assert_grad_close, attention_backward, attention_forward,
                             derived_o_tol, f64, gpu_backward, gpu_forward)
    from exact_attention_fa_amd.inputs import make_inputs
    B, Hq, Hkv, N, D, dtype, causal, R = dims
    shape = Shape(B, Hq, Hkv, N, D, dtype, causal)
    log("rising scores", shape, "ramp", R)
    q, k, v, do = make_inputs(shape, seed=zlib.crc32(repr(dims).encode()) % (1 << 31))
    ramp = 1.0 + (R - 1.0) * torch.arange(N, dtype=torch.float32) / max(N - 1, 1)
    k = (k.float() * ramp[None, None, :, None]).to(k.dtype)
    o, lse = gpu_forward(q, k, v, causal, shape.scale)
    o_ref, lse_ref = attention_forward(f64(q), f64(k), f64(v), shape.scale, causal)
    errs = assert_fwd_close(f64(o), f64(lse), o_ref, lse_ref, str(shape), derived_o_tol(f64(v), dtype))
    log("  fwd errors", errs)
    assert np.isfinite(f64(o)).all()
    dq, dk, dv = gpu_backward(q, k, v, o, do, lse, causal, shape.scale)
    if R > 8.0:
        # Nearly one-hot rows: dS = P (dP - D) is a cancellation, and D is formed from the stored
        # 16-bit O, so a gradient's error is set by O's rounding, not by its own magnitude.  Each
        # element is held to the bound derived from the arithmetic (parity_util.grad_error_bound).
        from parity_util import assert_within_bound, grad_error_bound
        bounds, refs = grad_error_bound(f64(q), f64(k), f64(v), f64(do), f64(o), f64(lse), shape.scale, causal,
                                        dtype)
        worst = {name: assert_within_bound(f64(g), r, bd, name, str(shape))
                 for name, g, r, bd in zip(("dq", "dk", "dv"), (dq, dk, dv), refs, bounds)}
        log("  backward: worst error / derived bound", worst)
        return
    dq_r, dk_r, dv_r = attention_backward(f64(q), f64(k), f64(v), f64(do), shape.scale, causal)
    for name, g, r in (("dq", dq, dq_r), ("dk", dk, dk_r), ("dv", dv, dv_r)):
        assert_grad_close(f64(g), r, name, str(shape))


def test_nondefault_scale_full():
    from parity_util import full_check
    for scale in (0.0, 0.05, 0.4):
        shape = Shape(1, 4, 2, 300, 64, "bf16", True)
        log("scale", scale)
        full_check(shape, seed=77, scale=scale)


# Negative softmax scales (S = scale Q K^T with scale < 0): the kernels run |scale| on the
# negated stationary operand.  Small grids (split key range, key- and query-range pieces) and
# a grid large enough for the 256-query forward workgroups and the 8-wave dQ pass.
NEGATIVE = [
    (1, 4, 2, 300, 64, "bf16", True, -0.1),
    (2, 4, 4, 517, 128, "fp16", False, -0.3),
    (1, 1, 1, 3000, 128, "bf16", True, -0.08),
    (4, 32, 8, 1000, 128, "bf16", False, -0.1),
]


@pytest.mark.parametrize("dims", NEGATIVE, ids=[f"B{b}H{hq}/{hk}N{n}D{d}{t}{'c' if cz else ''}s{sc:g}"
                                                for b, hq, hk, n, d, t, cz, sc in NEGATIVE])
def test_negative_scale_full(dims):
    from parity_util import full_check
    B, Hq, Hkv, N, D, dtype, causal, scale = dims
    shape = Shape(B, Hq, Hkv, N, D, dtype, causal)
    log("negative scale", shape, scale)
    errs = full_check(shape, seed=zlib.crc32(repr(dims).encode()) % (1 << 31), scale=scale)
    log("  errors", errs)


# --------------------------------------------------- the full-size workloads (sampled)

def test_fwd_bf16_n4096_full():
    """The default benchmark workload (B=4, H=16, N=4096, D=128, bf16) in full: every element of
    O, LSE, dQ, dK and dV against the oracle."""
    from parity_util import full_check
    shape = WORKLOADS["fwd_bf16_n4096"][0]
    log("workload", shape)
    errs = full_check(shape, workload_seed("fwd_bf16_n4096", 0))
    log("  errors", errs)


def test_fwd_bf16_n8192_full():
    """B=1, H=16, N=8192, D=128, bf16 in full: every element of O, LSE, dQ, dK and dV."""
    from parity_util import full_check
    shape = WORKLOADS["fwd_bf16_long"][0]
    assert shape.N == 8192
    log("workload", shape)
    errs = full_check(shape, workload_seed("fwd_bf16_long", 0))
    log("  errors", errs)


def test_fwd_bf16_n16384_unit_full():
    """B=1, H=16, N=16384, D=128, bf16, run exactly as bench.py launches it: every row of O, LSE
    and dQ of head 11, and every key of its dK and dV, against the oracle; sampled rows of the
    forward of head 0."""
    from parity_util import assert_fwd_close, attention_forward, bench_path_run, f64, unit_full_check
    import numpy as np
    shape = WORKLOADS["fwd_bf16_long"][1]
    assert shape.N == 16384
    log("workload", shape)
    inputs, outputs = bench_path_run(shape, workload_seed("fwd_bf16_long", 1))
    errs = unit_full_check(shape, inputs, outputs, units=[(0, 11)])
    log("  unit (0, 11) errors", errs)
    q, k, v, _ = inputs
    rows = np.unique(np.concatenate([[0, 1, 8191, 8192, 16320, 16383],
                                     np.random.default_rng(5).choice(16384, 64, replace=False)]))
    o_r, l_r = attention_forward(f64(q[:, :1]), f64(k[:, :1]), f64(v[:, :1]), shape.scale, False, rows=rows)
    eo, el = assert_fwd_close(f64(outputs[0][:, :1])[:, :, rows], f64(outputs[1][:, :1])[:, :, rows], o_r, l_r,
                              "head 0 sampled rows")
    log("  head 0 sampled rows", eo, el)


@pytest.mark.parametrize("variant", range(6), ids=[f"N{s.N}D{s.D}" for s in WORKLOADS["gqa_causal_fp16"]])
def test_gqa_causal_fp16_full(variant):
    """The grouped-query causal workloads at full size (N = 2048, 4096 and the ragged 4000; D =
    64 and 128), every element of O, LSE, dQ, dK and dV against the oracle."""
    from parity_util import full_check
    shape = WORKLOADS["gqa_causal_fp16"][variant]
    log("workload", shape)
    errs = full_check(shape, workload_seed("gqa_causal_fp16", variant))
    log("  errors", errs)


def test_causal_long_bf16_unit_full():
    """B=1, H=8, N=16384, D=128, causal, bf16, inputs x0.5, run exactly as bench.py launches it
    (the 256-query forward workgroups and the 8-wave dQ pass): every row of O, LSE and dQ of
    head 5 and every key of its dK and dV against the oracle."""
    from parity_util import bench_path_run, unit_full_check
    shape = WORKLOADS["causal_long_bf16"][0]
    log("workload", shape)
    inputs, outputs = bench_path_run(shape, workload_seed("causal_long_bf16", 0))
    errs = unit_full_check(shape, inputs, outputs, units=[(0, 5)])
    log("  unit (0, 5) errors", errs)


def test_shard_causal_bf16_full():
    """One GPU's share of the long causal workload (one head, N = 16384) in the launch
    configuration bench.py times: fa_fwd_splitkv with the library's choice of key-range pieces,
    then fa_bwd with its query- and key-range pieces; every element of O, LSE, dQ, dK and dV
    against the oracle."""
    import torch
    import exact_attention_fa_amd as fa
    from parity_util import assert_fwd_close, assert_grad_close, attention_backward, attention_forward, f64
    from exact_attention_fa_amd.inputs import make_inputs
    shape = WORKLOADS["shard_causal_bf16"][0]
    log("workload", shape)
    B, Hq, Hkv, N, D = shape.B, shape.Hq, shape.Hkv, shape.N, shape.D
    assert fa.fa_fwd_splitkv_parts(B, Hq, Hkv, N, D, True) > 1
    q, k, v, do = (t.cuda() for t in make_inputs(shape, workload_seed("shard_causal_bf16", 0)))
    o, lse = fa.fa_fwd_splitkv(q, k, v, causal=True)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    qs, ks, vs, dos = f64(q), f64(k), f64(v), f64(do)
    o_r, l_r = attention_forward(qs, ks, vs, shape.scale, True)
    errs = dict(zip(("o", "lse"), assert_fwd_close(f64(o), f64(lse), o_r, l_r, str(shape))))
    dq_r, dk_r, dv_r = attention_backward(qs, ks, vs, dos, shape.scale, True)
    for name, g, r in (("dq", dq, dq_r), ("dk", dk, dk_r), ("dv", dv, dv_r)):
        errs[name] = assert_grad_close(f64(g), r, name, str(shape))
    log("  errors", errs)


def _random_cases(n, seed, n_max=1500, cap=4e7):
    """Seeded shapes across the supported space: batch, MQA/GQA/MHA head ratios, ragged N
    (log-uniform up to n_max, including 1), both head dims and dtypes, causal or not, and the
    default, zero, small, large or negative softmax scales.  Each case's oracle work is capped
    (B * Hq * N^2 <= cap) so the whole sweep runs in well under a minute."""
    import numpy as np
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        B = int(rng.integers(1, 4))
        Hkv = int(rng.choice([1, 1, 2, 3]))
        grp = int(rng.choice([1, 1, 2, 3, 4, 8]))
        N = int(np.clip(round(float(np.exp(rng.uniform(0.0, np.log(n_max))))), 1, n_max))
        D = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["bf16", "fp16"]))
        causal = bool(rng.integers(0, 2))
        kind = int(rng.integers(0, 5))
        scale = None if kind < 2 else (0.0 if kind == 2 else float(np.round(rng.uniform(-0.25, 0.25), 4)))
        if B * Hkv * grp * N * N > cap:
            continue
        cases.append((B, Hkv * grp, Hkv, N, D, dtype, causal, scale))
    return cases


RANDOM = _random_cases(64, 2026) + _random_cases(16, 2027, n_max=4000, cap=2e8)


@pytest.mark.parametrize("dims", RANDOM, ids=[f"B{b}H{hq}/{hk}N{n}D{d}{t}{'c' if cz else ''}s{sc}"
                                              for b, hq, hk, n, d, t, cz, sc in RANDOM])
def test_random_shapes_full(dims):
    """A seeded sweep of shapes, each compared element by element with the oracle (forward and
    backward)."""
    from parity_util import full_check
    B, Hq, Hkv, N, D, dtype, causal, scale = dims
    shape = Shape(B, Hq, Hkv, N, D, dtype, causal)
    log("random shape", shape, "scale", scale)
    errs = full_check(shape, zlib.crc32(repr(dims).encode()) % (1 << 31), scale=scale)
    log("  errors", errs)
