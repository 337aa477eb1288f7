#!/usr/bin/env python3
"""Benchmark of the fused exact-attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: the forward
(fa_fwd_splitkv with the library's choice of key-range pieces, which is exactly fa_fwd
except on grids too small to fill the GPU) and the backward (fa_bwd, in the stage order
fa_bwd_plan names: the dQ pass forming the row values, then the dK/dV pass; or the
preprocess, the dK/dV pass, the dQ pass and the postprocess) on the same stream.
Inputs, outputs and workspace are allocated and resident in HBM before timing starts.

Prints ONE JSON line on stdout:
  value           whole-step attention TFLOP/s (fwd+bwd algorithmic FLOPs / step time)
  fwd_tflops ...  the forward and backward alone, and both as % of the bf16 dense MFMA peak
  roofline        the dominant kernel (largest share of step time), timed with HIP events
                  on the stream it is launched on, against the MFMA peak; `traffic` is its HBM
                  bytes per launch from the committed hardware-counter summary under profiles/,
                  or null when the kernel source has changed since the counters were taken
  hbm             the memory-bound stage, the backward preprocess (fa_bwd_preprocess), timed
                  on its own after the steps: an event pair around each of 10 launches over
                  rotated copies of O and dO (at least 1 GiB in all, more than the Infinity
                  Cache holds); algorithmic bytes per launch over the median, against the HBM
                  peak (where fa_bwd forms these values inside its dQ pass, the stage is not
                  part of the step)
  cpu_baseline    the CPU oracle timed on a bounded sample of the same workload
  kernel_*_ms     per-kernel average, median, minimum and maximum over the timed steps (steps
                  under a millisecond: over K further steps timed kernel by kernel)
  mfma_util       MFMA (and VALU) busy fraction and sustained shader clock of the dominant
                  kernel, from the committed hardware-counter summary under profiles/ (null
                  when the kernel source has changed since the counters were taken)
  measured_gemm   an 8192^3 library GEMM in the workload's dtype, run after the timed steps:
                  the measured MFMA ceiling, with fwd and fwd+bwd as % of it
  gpu_power_w     board power (sysfs hwmon, read in-process) before the warmup and after the
                  timed steps
  gpu_clock       the shader clock level the driver reports (sysfs, read in-process) before
                  the warmup and after the timed steps

`value` and `ms_per_step` use the median of the per-step HIP-event durations (the pages'
protocol: warmups, then the median of the timed repetitions); `wall_ms_per_step` is the
host wall time of the whole timed region divided by the steps.  Steps of a millisecond or
more run the backward's stages (in fa_bwd's order, the same launches) with an event between
every two kernels, which also gives the per-kernel figures; shorter steps (the tiny and grouped-query workloads) instead time one
fa_fwd_splitkv and one fa_bwd call per step (one event pair) and take their per-kernel
figures from K further steps.  The default workload is the
long non-causal bf16 sequence (B=1, H=16, N=16384, D=128).  The tiny fp16 workloads
(`--workload tiny_fp16_nc` / `tiny_fp16_causal`, B=1, H=2, N=256, D=64) are latency-bound:
their line adds microseconds per kernel and the step's algorithmic HBM bytes per second.

The script starts no child process: under a profiler every child would inherit the
profiler's preloaded library.

FLOP convention: forward 4*B*H*N^2*D, backward 10*B*H*N^2*D (five N x N x D products,
including the recompute of S), halved when causal.

`--copy-calibration BYTES` instead runs a plain device-to-device copy of BYTES bytes five
times (the reference kernel for scaling the FETCH_SIZE / WRITE_SIZE counters) and exits.
`--ceilings` instead measures what the GPU sustains on plain library work (8192^3 bf16 and
fp16 GEMMs, 2 GiB HBM read and copy), and the backward preprocess at the default size and at
8x its rows, context for the roofline fractions, and exits.
`--summarize KIND DIR...` reads rocprofv3 CSV output (no GPU) and prints the summary lines that
the files under profiles/ hold (see summarize()).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (fwd; fwd+bwd) and % of MI355X bf16 MFMA peak"
PEAK_MFMA_TFLOPS = 2516.6   # 256 CU x 4096 dense bf16/fp16 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0

WORKLOAD_KEYS = {
    "tiny_fp16_nc": ("tiny_fp16", 0),
    "tiny_fp16_causal": ("tiny_fp16", 1),
    "fwd_bf16_n4096": ("fwd_bf16_n4096", 0),
    "fwd_bf16_n8192": ("fwd_bf16_long", 0),
    "fwd_bf16_n16384": ("fwd_bf16_long", 1),
    "causal_long_bf16": ("causal_long_bf16", 0),
    "shard_causal_bf16_h1": ("shard_causal_bf16", 0),
}
for _i, (_n, _d) in enumerate([(2048, 64), (2048, 128), (4096, 64), (4096, 128), (4000, 64), (4000, 128)]):
    WORKLOAD_KEYS[f"gqa_causal_fp16_n{_n}_d{_d}"] = ("gqa_causal_fp16", _i)


# Which sources (and build options) each timed kernel is built from, for matching a counter
# summary to the code.
_DEV = ["exact_attention_fa_amd/csrc/fa_device.h", "exact_attention_fa_amd/_build.py"]
KERNEL_SOURCES = {
    "fwd": ["exact_attention_fa_amd/csrc/fa_fwd.hip", *_DEV],
    "bwd_preprocess": ["exact_attention_fa_amd/csrc/fa_bwd.hip", *_DEV],
    "bwd_dkdv": ["exact_attention_fa_amd/csrc/fa_bwd.hip", *_DEV],
    "bwd_dq": ["exact_attention_fa_amd/csrc/fa_bwd.hip", *_DEV],
    "bwd_postprocess": ["exact_attention_fa_amd/csrc/fa_bwd.hip", *_DEV],
}


def _code_only(rel, text):
    """The source without comments and blank lines: editing a comment leaves the kernel, and
    so the counters taken on it, unchanged."""
    if rel.endswith(".py"):
        text = re.sub(r"#[^\n]*", "", text)
    else:
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_hash(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(rel, f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from profiles/traffic_<kernel>_<workload>.txt (key = value lines),
    if that summary was taken on the current source of the kernel; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_sha256_16") != source_hash(kernel) or "hbm_bytes_per_launch" not in kv:
        return None
    return int(float(kv["hbm_bytes_per_launch"]))


def machine_ceilings():
    """What this GPU sustains on plain library work, as context for the roofline fractions:
    a large bf16 and fp16 GEMM (torch.matmul, i.e. hipBLASLt) and HBM streaming (a reduction
    that reads 2 GiB, and a 2 GiB device copy).  One JSON line."""
    import torch

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    out = {"clock_before": gpu_clock()}
    n = 8192
    for name, dt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        a = torch.randn(n, n, device="cuda").to(dt)
        b = torch.randn(n, n, device="cuda").to(dt).contiguous()
        t = timed(lambda: torch.matmul(a, b), 40)
        out[f"gemm_{name}_{n}_tflops"] = round(2 * n ** 3 / t / 1e12, 1)
        out[f"gemm_{name}_pct_of_spec"] = round(100 * 2 * n ** 3 / t / 1e12 / PEAK_MFMA_TFLOPS, 1)
        del a, b
    x = torch.ones(1 << 30, dtype=torch.bfloat16, device="cuda")  # 2 GiB
    t = timed(lambda: x.sum(dtype=torch.float32), 20)
    out["hbm_read_gbs"] = round(x.numel() * 2 / t / 1e9, 1)
    y = torch.empty_like(x)
    t = timed(lambda: y.copy_(x), 20)
    out["hbm_copy_read_plus_write_gbs"] = round(2 * x.numel() * 2 / t / 1e9, 1)
    del x, y
    # The backward preprocess (a pure stream: O and dO read, two fp32 values per row written) at
    # the default workload's size and at 8x its rows: how much of its rate the size sets.
    import exact_attention_fa_amd as fa
    from exact_attention_fa_amd.inputs import Shape
    fa.load_library()
    for B in (1, 8):
        H, N, D = 16, 16384, 128
        o = torch.randn((B, H, N, D), device="cuda").to(torch.bfloat16)
        do = torch.randn((B, H, N, D), device="cuda").to(torch.bfloat16)
        lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
        ws = torch.empty(fa.fa_bwd_workspace_size(B, H, H, N, D), dtype=torch.uint8, device="cuda")
        t = timed(lambda: fa.fa_bwd_preprocess(o, do, lse, ws, H), 20)
        nbytes = algorithmic_bytes(Shape(B, H, H, N, D, "bf16", False))["bwd_preprocess"]
        out[f"bwd_preprocess_B{B}_H16_N16384_MiB"] = round(nbytes / 2 ** 20, 1)
        out[f"bwd_preprocess_B{B}_H16_N16384_gbs"] = round(nbytes / t / 1e9, 1)
        del o, do, lse, ws
    out["clock_after"] = gpu_clock()
    print(json.dumps(out), flush=True)


def gpu_clock():
    """The shader clock levels the amdgpu driver lists in sysfs (the current one is marked
    with '*'), read as plain files in this process, or None where they cannot be read.  Each
    card visible in sysfs is reported by its PCI address."""
    out = {}
    try:
        for card in sorted(os.listdir("/sys/class/drm")):
            path = os.path.join("/sys/class/drm", card, "device", "pp_dpm_sclk")
            if not card.startswith("card") or "-" in card or not os.path.exists(path):
                continue
            with open(path) as f:
                cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
            pci = os.path.basename(os.path.realpath(os.path.join("/sys/class/drm", card, "device")))
            if cur:
                out[pci] = cur[0].rstrip(" *")
    except OSError:  # the clock is context for the numbers, never a reason to fail the run
        return None
    return out or None


def gpu_power():
    """Board power in watts from the amdgpu driver's hwmon files (power1_average, else
    power1_input, in microwatts), read in this process, per card by PCI address; None where
    they cannot be read."""
    out = {}
    try:
        for card in sorted(os.listdir("/sys/class/drm")):
            dev = os.path.join("/sys/class/drm", card, "device")
            hw = os.path.join(dev, "hwmon")
            if not card.startswith("card") or "-" in card or not os.path.isdir(hw):
                continue
            for h in sorted(os.listdir(hw)):
                for name in ("power1_average", "power1_input"):
                    path = os.path.join(hw, h, name)
                    if os.path.exists(path):
                        with open(path) as f:
                            out[os.path.basename(os.path.realpath(dev))] = round(int(f.read().strip()) / 1e6, 1)
                        break
    except (OSError, ValueError):  # context only, never a reason to fail the run
        return None
    return out or None


def measured_gemm_tflops(dtype_name):
    """What a plain library GEMM sustains on this GPU right now, in the workload's dtype: an
    8192^3 torch.matmul (hipBLASLt), 10 products after 3 warmups, timed with HIP events.  The
    measured MFMA ceiling beside the spec peak."""
    import torch
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype_name]
    n = 8192
    a = torch.randn(n, n, device="cuda").to(dt)
    b = torch.randn(n, n, device="cuda").to(dt)
    for _ in range(3):
        torch.matmul(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.matmul(a, b)
    e1.record()
    e1.synchronize()
    return 2 * n ** 3 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12


def copy_calibration(nbytes):
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 5
    print(json.dumps({"copy_bytes": n * 4, "launches": 5, "ms_per_copy": round(dt * 1e3, 4),
                      "read_plus_write_GBs": round(2 * n * 4 / dt / 1e9, 1)}), flush=True)


def flops(shape, fwd=True, bwd=True):
    f = 4.0 * shape.B * shape.Hq * shape.N * shape.N * shape.D
    if shape.causal:
        f /= 2
    return (f if fwd else 0.0) + (2.5 * f if bwd else 0.0)


def cpu_baseline(shape, seed, budget_s):
    """Time the float64 oracle's fwd+bwd on whole (batch, kv-group) units until ~budget_s."""
    import numpy as np
    from exact_attention_fa_amd.inputs import make_inputs
    from oracle import attention_backward, attention_forward
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    q, k, v, do = make_inputs(shape, seed)
    grp = shape.Hq // shape.Hkv
    f = lambda t: t.double().numpy()
    units = [(b, kv) for b in range(shape.B) for kv in range(shape.Hkv)]
    done, t0 = 0, time.perf_counter()
    for b, kv in units:
        hs = slice(kv * grp, (kv + 1) * grp)
        qs, ks, vs, dos = f(q[b:b + 1, hs]), f(k[b:b + 1, kv:kv + 1]), f(v[b:b + 1, kv:kv + 1]), f(do[b:b + 1, hs])
        attention_forward(qs, ks, vs, shape.scale, shape.causal)
        attention_backward(qs, ks, vs, dos, shape.scale, shape.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    unit_flops = flops(shape) / len(units)
    return {
        "value": round(done * unit_flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{done} of {len(units)} (batch, kv-group) units of the workload, fwd+bwd in float64 "
                   f"(NumPy, {threads} BLAS threads), {dt:.1f} s; the oracle computes the full N^2 work even "
                   f"when causal, rated with the same algorithmic FLOP convention"),
        "host_cpu": platform.processor() or platform.machine(),
    }


def algorithmic_bytes(shape, rows_first=False):
    """Algorithmic HBM bytes of each timed stage: every input read once and every output
    written once (K/V re-reads across query tiles and Q/dO re-reads across key blocks are
    implementation traffic, not counted).  rows_first: the dQ pass forms the row values
    (fa_bwd_dq_rows) and the preprocess stage is not run."""
    es = 2 if shape.dtype in ("bf16", "fp16") else 4
    q = shape.B * shape.Hq * shape.N * shape.D * es
    kv = shape.B * shape.Hkv * shape.N * shape.D * es
    rows = shape.B * shape.Hq * shape.N
    out = {
        "fwd": 2 * q + 2 * kv + 4 * rows,                    # Q, K, V read; O, LSE written
        "bwd_preprocess": 2 * q + 4 * rows + 8 * rows,       # O, dO, LSE read; -D, LSE*log2 e written
        "bwd_dkdv": 2 * q + 2 * kv + 8 * rows + 2 * kv,      # Q, dO, K, V, LSE, D read; dK, dV written
        "bwd_dq": 2 * q + 2 * kv + 8 * rows + q,             # Q, dO, K, V, LSE, D read; dQ written
        "bwd_postprocess": 0,                                # partials only (none for MHA grids)
    }
    if rows_first:
        # Q, dO, O, K, V, LSE read; -D, LSE*log2 e and dQ written
        out["bwd_dq"] = 3 * q + 2 * kv + 4 * rows + 8 * rows + q
        del out["bwd_preprocess"], out["bwd_postprocess"]
    return out


def standalone_preprocess(fa, torch, o, do, lse, ws, Hkv, launches=10):
    """Median time (ms) of one fa_bwd_preprocess launch, timed with an event pair around each of
    `launches` launches over rotated copies of O and dO: enough copies for 1 GiB of inputs
    (at least two), so that no launch finds its inputs in the 256 MB Infinity Cache."""
    import statistics
    copies = max(2, min(16, -(-(1 << 30) // max(1, 2 * o.numel() * o.element_size()))))
    pairs = [(o.clone(), do.clone()) for _ in range(copies)]
    stream = torch.cuda.current_stream()
    for oc, dc in pairs:
        fa.fa_bwd_preprocess(oc, dc, lse, ws, Hkv)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for i, (a, b) in enumerate(ev):
        oc, dc = pairs[i % copies]
        a.record(stream)
        fa.fa_bwd_preprocess(oc, dc, lse, ws, Hkv)
        b.record(stream)
    torch.cuda.synchronize()
    ms = statistics.median(a.elapsed_time(b) for a, b in ev)
    del pairs
    return ms, copies


def counter_summary(kernel, workload):
    """MFMA busy fraction and sustained shader clock from profiles/busy_<kernel>_<workload>.txt,
    if that summary was taken on the current source of the kernel; else None."""
    path = os.path.join(ROOT, "profiles", f"busy_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.split("#", 1)[0].strip()
    if kv.get("source_sha256_16") != source_hash(kernel):
        return None
    try:
        out = {"kernel": kernel, "mfma_busy_frac": float(kv["mfma_busy_frac"]),
               "sclk_mhz_sustained": float(kv["sclk_mhz_sustained"]),
               "source": f"profiles/busy_{kernel}_{workload}.txt"}
        if "valu_busy_frac" in kv:
            out["valu_busy_frac"] = float(kv["valu_busy_frac"])
        return out
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ rocprofv3 summaries

def _csv_rows(directory, suffix):
    import csv
    rows = []
    for base, _, files in os.walk(directory):
        for name in sorted(files):
            if name.endswith(suffix):
                with open(os.path.join(base, name), newline="") as f:
                    rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no *{suffix} under {directory}")
    return rows


def _short(name):
    """Kernel name without namespaces, return type and argument list."""
    name = name.replace("(anonymous namespace)::", "").replace("fa::", "")
    name = re.sub(r"^void ", "", name)
    depth = 0
    for i, ch in enumerate(name):  # cut at the argument list: the first '(' outside <...>
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            return name[:i]
    return name


_STAGE_OF = {"fwd_kernel": "fwd", "bwd_pre_kernel": "bwd_preprocess", "bwd_dkdv_kernel": "bwd_dkdv",
             "bwd_dq_kernel": "bwd_dq"}


def _counter_avg(directory, counter):
    from collections import defaultdict
    vals = defaultdict(list)
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] == counter:
            vals[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: statistics.fmean(v) for k, v in vals.items()}


def rows_first_plan(shape):
    """True where fa_bwd runs the dQ pass first and forms the row values there
    (fa_bwd_plan == FA_BWD_PLAN_ROWS); asks the library, which needs no GPU for it."""
    import exact_attention_fa_amd as fa
    code = {"fp16": fa.FA_FP16, "bf16": fa.FA_BF16}[shape.dtype]
    return fa.fa_bwd_plan(shape.B, shape.Hq, shape.Hkv, shape.N, shape.D, code) == fa.FA_BWD_PLAN_ROWS


def _traffic(dirs, copy_bytes, workload):
    """The blocks that profiles/traffic_<stage>_<workload>.txt hold (see summarize).  The
    preprocess's launches in these runs are the standalone ones after the steps."""
    from exact_attention_fa_amd.inputs import WORKLOADS
    name, variant = WORKLOAD_KEYS[workload]
    shape = WORKLOADS[name][variant]
    alg = {**algorithmic_bytes(shape), **algorithmic_bytes(shape, rows_first_plan(shape))}
    fetch, write = _counter_avg(dirs[0], "FETCH_SIZE"), _counter_avg(dirs[1], "WRITE_SIZE")
    cfetch, cwrite = _counter_avg(dirs[2], "FETCH_SIZE"), _counter_avg(dirs[3], "WRITE_SIZE")
    copy = [k for k in cfetch if "copy" in k.lower()]
    if len(copy) != 1 or copy[0] not in cwrite:
        raise SystemExit(f"expected one copy kernel in the calibration runs, found {sorted(cfetch)}")
    fscale = copy_bytes / (cfetch[copy[0]] * 1024.0)
    wscale = copy_bytes / (cwrite[copy[0]] * 1024.0)
    for k in sorted(fetch):
        stage = _STAGE_OF.get(k.split("<", 1)[0])
        if stage is None or k not in write:
            continue
        rd, wr = fetch[k] * 1024.0 * fscale, write[k] * 1024.0 * wscale
        print(f"# {stage}: {k}")
        for key, val in (("kernel", stage), ("workload", workload),
                         ("fetch_size_kib", f"{fetch[k]:.1f}"), ("write_size_kib", f"{write[k]:.1f}"),
                         ("fetch_scale", f"{fscale:.5f}"), ("write_scale", f"{wscale:.5f}"),
                         ("hbm_read_bytes", f"{rd:.0f}"), ("hbm_write_bytes", f"{wr:.0f}"),
                         ("hbm_bytes_per_launch", f"{rd + wr:.0f}"),
                         ("algorithmic_bytes_per_launch", alg[stage]),
                         ("source_sha256_16", source_hash(stage))):
            print(f"{key} = {val}")


def summarize(kind, dirs, skip=0, copy_bytes=0, workload=None):
    """Summary lines from rocprofv3 CSV output, per kernel (the template name shortened):
      trace DIR       average dispatch duration (us) over the dispatches after the first `skip`
      counters DIR..  per-dispatch averages of every collected counter (one or more runs)
      busy DIR..      from SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE and the dispatches' own
                      timestamps: MFMA busy fraction per SIMD (busy cycles / 1024 SIMDs / the
                      kernel's cycles) and the sustained shader clock (GRBM_GUI_ACTIVE / 8 XCDs /
                      duration); with SQ_ACTIVE_INST_VALU also the VALU busy fraction (its
                      4-cycle units summed over waves, per SIMD and kernel cycle)
      traffic F W CF CW   HBM bytes per launch from a FETCH_SIZE run (F) and a WRITE_SIZE run (W)
                      of the workload, each scaled by what the same counter reads for a plain copy
                      of `copy_bytes` bytes (runs CF and CW), next to the stage's algorithmic bytes
    Prints `kernel: key = value` lines (traffic: a block of `key = value` lines per kernel); no
    GPU is needed."""
    from collections import defaultdict
    if kind == "traffic":
        if len(dirs) != 4 or not copy_bytes or workload is None:
            raise SystemExit("--summarize traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR "
                             "needs --workload and --copy-calibration BYTES")
        _traffic(dirs, copy_bytes, workload)
        return
    if kind == "trace":
        rows = _csv_rows(dirs[0], "kernel_trace.csv")
        dur = defaultdict(list)
        for r in rows:
            dur[_short(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        for k, v in dur.items():
            v = v[skip:] or v
            print(f"{k}: dispatches = {len(v)}; avg_us = {statistics.fmean(v):.1f}; "
                  f"median_us = {statistics.median(v):.1f}; min_us = {min(v):.1f}; max_us = {max(v):.1f}")
        return
    vals = defaultdict(lambda: defaultdict(list))
    durs = defaultdict(dict)
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            k = _short(r["Kernel_Name"])
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if "Start_Timestamp" in r and "End_Timestamp" in r:
                durs[k][(d, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    for k, cs in vals.items():
        avg = {c: statistics.fmean(v) for c, v in cs.items()}
        dur_us = statistics.fmean(durs[k].values()) if durs[k] else None
        if kind == "counters":
            print(f"{k}: " + "; ".join(f"{c} = {v:.4g}" for c, v in sorted(avg.items())))
            continue
        gui = avg.get("GRBM_GUI_ACTIVE")
        mfma = avg.get("SQ_VALU_MFMA_BUSY_CYCLES")
        if gui is None or mfma is None:
            continue
        cycles = gui / 8.0                       # per XCD: the kernel's duration in shader cycles
        busy = mfma / 1024.0 / cycles            # 1024 SIMDs (256 CUs x 4)
        line = f"{k}: mfma_busy_frac = {busy:.4f}"
        if "SQ_ACTIVE_INST_VALU" in avg:         # counted in units of 4 cycles, summed over waves
            line += f"; valu_busy_frac = {avg['SQ_ACTIVE_INST_VALU'] * 4.0 / 1024.0 / cycles:.4f}"
        line += f"; gui_cycles_per_xcd = {cycles:.4g}"
        if dur_us:
            line += f"; dur_us = {dur_us:.1f}; sclk_mhz_sustained = {cycles / dur_us:.0f}"
        print(line)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fwd_bf16_n16384", choices=sorted(WORKLOAD_KEYS))
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-ceiling", action="store_true", help="skip the library GEMM measured after the timed steps")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--ceilings", action="store_true", help="measure library GEMM and HBM rates and exit")
    ap.add_argument("--summarize", nargs="+", metavar=("KIND", "DIR"),
                    help="summarise rocprofv3 CSV output: trace DIR | counters DIR... | busy DIR... | "
                         "traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR")
    ap.add_argument("--skip", type=int, default=0, help="with --summarize trace: dispatches to skip")
    args = ap.parse_args()

    if args.summarize:
        summarize(args.summarize[0], args.summarize[1:], args.skip, args.copy_calibration,
                  args.workload if args.summarize[0] == "traffic" else None)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (attention heads and "
              "batches shard with no communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.ceilings:
        machine_ceilings()
        return

    import torch
    import exact_attention_fa_amd as fa
    from exact_attention_fa_amd.inputs import WORKLOADS, make_inputs, workload_seed

    name, variant = WORKLOAD_KEYS[args.workload]
    shape = WORKLOADS[name][variant]
    seed = workload_seed(name, variant)
    fa.load_library()
    dev = torch.device("cuda", 0)
    q, k, v, do = (t.to(dev) for t in make_inputs(shape, seed))
    B, Hq, Hkv, N, D = shape.B, shape.Hq, shape.Hkv, shape.N, shape.D
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, Hq, Hkv, N, D), dtype=torch.uint8, device=dev)
    causal, scale = shape.causal, shape.scale
    # the forward takes key-range pieces only where the grid is too small to fill the GPU
    n_split = fa.fa_fwd_splitkv_parts(B, Hq, Hkv, N, D, causal)
    fws = torch.empty(max(fa.fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, D, n_split), 256), dtype=torch.uint8,
                      device=dev)
    stream = torch.cuda.current_stream(dev)

    # fa_bwd's stages in its own order: the dQ pass forming the row values, then the dK/dV pass
    # (FA_BWD_PLAN_ROWS), or the preprocess, dK/dV pass, dQ pass and postprocess
    rows_first = rows_first_plan(shape)
    if rows_first:
        kernels = ["fwd", "bwd_dq", "bwd_dkdv"]
    else:
        kernels = ["fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq", "bwd_postprocess"]

    def fwd_call():
        fa.fa_fwd_splitkv(q, k, v, causal=causal, softmax_scale=scale, n_split=n_split, workspace=fws, out=o, lse=lse)

    calls = {
        "fwd": fwd_call,
        "bwd_preprocess": lambda: fa.fa_bwd_preprocess(o, do, lse, ws, Hkv),
        "bwd_dkdv": lambda: fa.fa_bwd_dkdv(q, k, v, do, dk, dv, ws, causal=causal, softmax_scale=scale),
        "bwd_dq": ((lambda: fa.fa_bwd_dq_rows(q, k, v, o, do, lse, dq, ws, causal=causal, softmax_scale=scale))
                   if rows_first else
                   (lambda: fa.fa_bwd_dq(q, k, v, do, dq, ws, causal=causal, softmax_scale=scale))),
        "bwd_postprocess": lambda: fa.fa_bwd_postprocess(dk, dv, ws, Hq),
    }

    def step(ev=None):
        if ev is None:  # as a caller runs it: one forward call and one fa_bwd call
            fwd_call()
            fa.fa_bwd(q, k, v, o, do, lse, causal=causal, softmax_scale=scale, workspace=ws, dq=dq, dk=dk, dv=dv)
            return
        # kernel by kernel: fa_bwd's stages (the same launches) with an event between every two
        for i, kname in enumerate(kernels):
            ev[i].record(stream)
            calls[kname]()
        ev[len(kernels)].record(stream)

    clock_before, power_before = gpu_clock(), gpu_power()
    for _ in range(args.warmup):
        step()
    # the step's length, from three more (untimed) steps after the warmup
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(3):
        step()
    w1.record(stream)
    torch.cuda.synchronize()
    short_step = w0.elapsed_time(w1) / 3 < 1.0  # milliseconds

    # Timed region: exactly K steps, bracketed by device synchronisation.  Steps of a millisecond
    # or more run kernel by kernel with an event between every two kernels (microseconds of
    # events against milliseconds of work), so the per-kernel figures come from the same steps
    # as the step time.  Shorter steps run as a caller runs them (one forward and one fa_bwd
    # call, one event pair), since events and host calls between their kernels would be a
    # visible part of their time; their per-kernel breakdown comes from K further steps.
    latency_bound = name == "tiny_fp16"
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if short_step:
            evs[s][0].record(stream)
            step()
            evs[s][len(kernels)].record(stream)
        else:
            step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock_after, power_after = gpu_clock(), gpu_power()
    ms_per_step = statistics.median([ev[0].elapsed_time(ev[len(kernels)]) for ev in evs])
    if short_step:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
        for s in range(args.steps):
            step(evs[s])
        torch.cuda.synchronize()
    per_kernel = {kname: [] for kname in kernels}
    for ev in evs:
        for i, kname in enumerate(kernels):
            per_kernel[kname].append(ev[i].elapsed_time(ev[i + 1]))
    avg = {kname: statistics.fmean(vals) for kname, vals in per_kernel.items()}
    med = {kname: statistics.median(vals) for kname, vals in per_kernel.items()}

    f_fwd, f_bwd = flops(shape, True, False), flops(shape, False, True)
    fwd_ms = med["fwd"]
    bwd_ms = statistics.median([sum(per_kernel[kname][s] for kname in kernels if kname != "fwd")
                                for s in range(args.steps)])
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    dominant = max(kernels, key=lambda kname: avg[kname])
    # Algorithmic FLOPs per launch: the dK/dV pass does four of the backward's five N x N x D
    # products (S, dP, dV, dK); the dQ pass adds the fifth (dQ).  Its recompute of S and dP
    # (another 0.4 of the backward's FLOPs) is work this design adds, so it is not credited.
    kflops = {"fwd": f_fwd, "bwd_dkdv": 0.8 * f_bwd, "bwd_dq": 0.2 * f_bwd,
              "bwd_preprocess": 0.0, "bwd_postprocess": 0.0}
    kbytes = algorithmic_bytes(shape, rows_first)
    if latency_bound:
        # A few hundred kilobytes per launch: every kernel is bound by launch and memory latency,
        # and the HBM rate of its algorithmic bytes is reported against the HBM peak.
        gbs = kbytes[dominant] / (avg[dominant] * 1e-3) / 1e9
        roofline = {"kernel": dominant, "bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 5), "traffic": None,
                    "avg_ms": round(avg[dominant], 4), "note": "latency-bound launch"}
    else:
        achieved = kflops[dominant] / (avg[dominant] * 1e-3) / 1e12
        roofline = {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2),
                    "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                    "traffic": measured_traffic(dominant, args.workload), "avg_ms": round(avg[dominant], 4)}
    # The memory-bound stage: the preprocess reads O and dO (input dtype) and the LSE, and
    # writes -D and LSE*log2(e), all fp32 per row.
    pre_bytes = algorithmic_bytes(shape)["bwd_preprocess"]
    pre_ms, pre_copies = standalone_preprocess(fa, torch, o, do, lse, ws, Hkv)
    pre_gbs = pre_bytes / (pre_ms * 1e-3) / 1e9
    hbm = {"kernel": "bwd_preprocess", "bound": "hbm", "achieved": round(pre_gbs, 1), "peak": PEAK_HBM_GBS,
           "unit": "GB/s", "frac": round(pre_gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": pre_bytes,
           "median_ms": round(pre_ms, 4), "timed": f"alone after the steps, {pre_copies} rotated copies of O and dO",
           "in_step": not rows_first}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "D": D,
                   "causal": causal, "softmax_scale": scale, "inputs": "N(0,1) seeded, cast RNE"
                   + (f", x{shape.mult}" if shape.mult != 1.0 else ""), "fwd_key_pieces": n_split},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2),
        "fwd_pct_peak": round(100 * f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 2),
        "fwd_bwd_pct_peak": round(100 * value / PEAK_MFMA_TFLOPS, 2),
        "kernel_avg_ms": {kname: round(val, 4) for kname, val in avg.items()},
        "kernel_median_ms": {kname: round(val, 4) for kname, val in med.items()},
        "kernel_min_ms": {kname: round(min(vals), 4) for kname, vals in per_kernel.items()},
        "kernel_max_ms": {kname: round(max(vals), 4) for kname, vals in per_kernel.items()},
        "gpu_clock": {"before": clock_before, "after": clock_after},
        "gpu_power_w": {"before": power_before, "after": power_after},
        "mfma_util": None if latency_bound else counter_summary(dominant, args.workload),
        "roofline": roofline,
        "hbm": hbm,
        "cpu_baseline": None,
    }
    if latency_bound:
        step_bytes = sum(kbytes.values())
        out["latency"] = {
            "step_us": round(ms_per_step * 1e3, 2),
            "kernel_median_us": {kname: round(val * 1e3, 2) for kname, val in med.items()},
            "step_algorithmic_bytes": step_bytes,
            "step_gbs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
            "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 5),
        }
    if not latency_bound and not args.no_gemm_ceiling:
        g = measured_gemm_tflops(shape.dtype)
        out["measured_gemm"] = {"tflops": round(g, 1), "what": f"8192^3 {shape.dtype} torch.matmul (hipBLASLt), after the timed steps",
                                "fwd_pct": round(100 * out["fwd_tflops"] / g, 1),
                                "fwd_bwd_pct": round(100 * value / g, 1)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shape, seed, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
