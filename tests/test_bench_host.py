"""Host-side parts of bench.py, without a GPU: it starts no child process (under a profiler a
child inherits the profiler's preloaded library), its rocprofv3 CSV summaries, its workload
table and its algorithmic byte counts."""
import ast
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_no_child_process_api_in_source():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            names.add(node.module)
        elif isinstance(node, ast.Attribute) and isinstance(node.value, ast.Name) and node.value.id == "os":
            names.add("os." + node.attr)
    banned = {"subprocess", "multiprocessing", "os.system", "os.popen", "os.fork", "os.spawnv", "os.execv",
              "os.execvp", "os.execve", "os.posix_spawn"}
    assert not names & banned, names & banned


def test_clock_query_spawns_nothing(monkeypatch):
    def refuse(*a, **k):
        raise AssertionError("bench.py started a child process")
    monkeypatch.setattr(subprocess, "Popen", refuse)
    monkeypatch.setattr(os, "system", refuse)
    monkeypatch.setattr(os, "posix_spawn", refuse, raising=False)
    clk = bench.gpu_clock()  # None here (no GPU), or the sysfs levels
    assert clk is None or isinstance(clk, dict)
    pw = bench.gpu_power()
    assert pw is None or isinstance(pw, dict)


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(f'"{x}"' for x in r) + "\n")


def test_summaries_from_rocprof_csv(tmp_path, capsys):
    name = "void fa::(anonymous namespace)::bwd_dkdv_kernel<fa::Bf16, 128, false, false>(unsigned short const*, int)"
    _write(str(tmp_path / "t" / "host" / "1" / "run_kernel_trace.csv"),
           ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [["KERNEL_DISPATCH", name, 1000, 1000 + 3_000_000], ["KERNEL_DISPATCH", name, 5000, 5000 + 4_000_000]])
    bench.summarize("trace", [str(tmp_path / "t")], skip=1)
    out = capsys.readouterr().out
    assert "bwd_dkdv_kernel<Bf16, 128, false, false>: dispatches = 1; avg_us = 4000.0" in out
    rows = [[name, "GRBM_GUI_ACTIVE", 8 * 2.0e6], [name, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1.2e6],
            [name, "GRBM_GUI_ACTIVE", 8 * 2.0e6], [name, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1.0e6]]
    _write(str(tmp_path / "c" / "host" / "1" / "run_counter_collection.csv"),
           ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    bench.summarize("busy", [str(tmp_path / "c")])
    out = capsys.readouterr().out
    assert "mfma_busy_frac = 0.5500" in out and "gui_cycles_per_xcd = 2e+06" in out
    _write(str(tmp_path / "v" / "host" / "1" / "run_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
           rows[:2] + [[name, "SQ_ACTIVE_INST_VALU", 1024 * 2.0e6 / 4 * 0.3]])
    bench.summarize("busy", [str(tmp_path / "v")])
    out = capsys.readouterr().out
    assert "valu_busy_frac = 0.3000" in out


def test_workloads_and_bytes():
    from exact_attention_fa_amd.inputs import WORKLOADS
    for key, (name, variant) in bench.WORKLOAD_KEYS.items():
        WORKLOADS[name][variant]
    assert bench.WORKLOAD_KEYS["tiny_fp16_causal"] == ("tiny_fp16", 1)
    s = WORKLOADS["fwd_bf16_long"][1]
    b = bench.algorithmic_bytes(s)
    q = 16 * 16384 * 128 * 2
    assert b["fwd"] == 4 * q + 4 * 16 * 16384
    assert b["bwd_dkdv"] == 6 * q + 8 * 16 * 16384
    # fa_bwd's plan for this workload: the dQ pass forms the row values (it also reads O and the
    # LSE and writes -D and LSE*log2 e), and there is no preprocess launch
    assert bench.rows_first_plan(s)
    r = bench.algorithmic_bytes(s, rows_first=True)
    assert r["bwd_dq"] == 6 * q + 12 * 16 * 16384 and "bwd_preprocess" not in r
    assert not bench.rows_first_plan(WORKLOADS["gqa_causal_fp16"][0])
    assert bench.flops(s) == pytest.approx(7696.58e9, rel=1e-5)


def test_busy_summary_needs_matching_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    for rel in bench.KERNEL_SOURCES["fwd"]:
        os.makedirs(os.path.dirname(tmp_path / rel), exist_ok=True)
        with open(tmp_path / rel, "w") as f:
            f.write("int x;\n")
    h = bench.source_hash("fwd")
    with open(tmp_path / "profiles" / "busy_fwd_w.txt", "w") as f:
        f.write(f"mfma_busy_frac = 0.61\nsclk_mhz_sustained = 1900  # note\nsource_sha256_16 = {h}\n")
    assert bench.counter_summary("fwd", "w")["mfma_busy_frac"] == 0.61
    with open(tmp_path / rel, "w") as f:
        f.write("int y;\n")
    assert bench.counter_summary("fwd", "w") is None


def test_traffic_summary_scales_by_copy(tmp_path, capsys):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled so that the copy reads and writes its size."""
    name = "void fa::(anonymous namespace)::bwd_dkdv_kernel<fa::Bf16, 128, false, false>(unsigned short const*, int)"
    copy = "__amd_rocclr_copyBuffer"
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(str(tmp_path / "f" / "h" / "run_counter_collection.csv"), hdr, [[name, "FETCH_SIZE", 1000.0]])
    _write(str(tmp_path / "w" / "h" / "run_counter_collection.csv"), hdr, [[name, "WRITE_SIZE", 300.0]])
    _write(str(tmp_path / "cf" / "h" / "run_counter_collection.csv"), hdr, [[copy, "FETCH_SIZE", 512.0]])
    _write(str(tmp_path / "cw" / "h" / "run_counter_collection.csv"), hdr, [[copy, "WRITE_SIZE", 1024.0]])
    dirs = [str(tmp_path / d) for d in ("f", "w", "cf", "cw")]
    bench.summarize("traffic", dirs, copy_bytes=1024 * 1024, workload="fwd_bf16_n16384")
    out = capsys.readouterr().out
    assert "kernel = bwd_dkdv" in out and "fetch_scale = 2.00000" in out and "write_scale = 1.00000" in out
    assert f"hbm_bytes_per_launch = {2000 * 1024 + 300 * 1024}" in out
    from exact_attention_fa_amd.inputs import WORKLOADS
    alg = bench.algorithmic_bytes(WORKLOADS["fwd_bf16_long"][1])["bwd_dkdv"]
    assert f"algorithmic_bytes_per_launch = {alg}" in out
    assert f"source_sha256_16 = {bench.source_hash('bwd_dkdv')}" in out


@pytest.mark.parametrize("env, argv", [({}, ["--gpus", "2"]), ({"WORLD_SIZE": "4"}, [])])
def test_more_than_one_gpu_is_refused(env, argv):
    """More than one GPU (a flag, or a launcher's WORLD_SIZE) exits with status 2 and says why,
    before touching torch's device state."""
    e = dict(os.environ, **env)
    p = subprocess.run([sys.executable, bench.__file__, *argv], capture_output=True, text=True, env=e, timeout=120)
    assert p.returncode == 2, p.stderr[-500:]
    assert "measures one GPU" in p.stderr and p.stdout == ""
