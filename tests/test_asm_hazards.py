"""Data hazards around the written-out MFMAs (host-side check of the gfx950 assembly).

The forward kernel for waves of 64 query rows and the dK/dV pass issue MFMAs as inline assembly
(accumulators and stationary operands in AGPRs, scores in VGPRs).  The compiler inserts no
wait states for them, so the kernels place their own.  This test compiles the sources to
assembly with the library's flags and walks every control-flow path from each written-out
MFMA:

  * no instruction other than an MFMA chaining on exactly the same accumulator may read or
    write the MFMA's destination within 19 wait states (an 8-pass XDL result needs at most 19
    before a VALU, v_accvgpr or memory access; the CDNA3/CDNA4 dependency tables);
  * no VALU instruction (v_accvgpr writes included) may write one of the MFMA's source
    registers within the 2 wait states before it.

Wait states are counted as the compiler's hazard recognizer does: one per instruction and N + 1
per s_nop N.  The kernels must also be free of scratch spills.
"""
import collections
import os
import re
import shutil
import subprocess

import pytest

from exact_attention_fa_amd import _build

WINDOW_AFTER = 19
WINDOW_BEFORE = 2


def _regs(tok):
    tok = tok.strip()
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _functions(asm, pattern):
    out = {}
    for m in re.finditer(r"^(_Z\S+):", asm, re.M):
        if re.search(pattern, m.group(1)):
            end = asm.index(".Lfunc_end", m.start())
            out[m.group(1)] = asm[m.start():end]
    return out


def _instructions(body):
    """[(label, op, operands, in_asm)]: labels as (name, None, [], False)."""
    ins, in_asm = [], False
    for line in body.splitlines()[1:]:
        raw = line.strip()
        if raw.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if raw.startswith(";;#ASMEND"):
            in_asm = False
            continue
        t = raw.split(";")[0].strip()
        if not t or (t.startswith(".") and not t.endswith(":")):
            continue
        if t.endswith(":"):
            ins.append((t[:-1], None, [], False))
            continue
        parts = t.split(None, 1)
        ops = [x.strip() for x in parts[1].split(",")] if len(parts) > 1 else []
        ins.append((None, parts[0], ops, in_asm))
    return ins


def _defs_uses(op, ops):
    regs = [_regs(o) for o in ops]
    every = set().union(*regs) if regs else set()
    if op.startswith(("s_", "global_store", "buffer_store", "ds_write", "scratch_store", "flat_store",
                      "v_cmp")) or (op.startswith("buffer_load") and "lds" in ops):
        return set(), every
    if not regs:
        return set(), set()
    d, u = regs[0], set().union(*regs[1:]) if len(regs) > 1 else set()
    if op.startswith("v_mfma"):
        d = _regs(ops[0])
        u = _regs(ops[1]) | _regs(ops[2]) | (_regs(ops[3]) if len(ops) > 3 else set())
    elif "fmac" in op or "dot2c" in op or "mac_" in op:
        u |= d
    return d, u


def _check(body):
    ins = _instructions(body)
    at = {lab: i for i, (lab, op, _, _) in enumerate(ins) if lab}

    def succ(i):
        op, ops = ins[i][1], ins[i][2]
        nxt = [i + 1] if i + 1 < len(ins) else []
        if op is None:
            return nxt
        if op == "s_endpgm":
            return []
        if op == "s_branch":
            return [at[ops[0]]]
        if op.startswith("s_cbranch"):
            return ([at[ops[0]]] if ops and ops[0] in at else []) + nxt
        return nxt

    preds = collections.defaultdict(list)
    for i in range(len(ins)):
        for j in succ(i):
            preds[j].append(i)

    def cost(i):
        op, ops = ins[i][1], ins[i][2]
        if op is None:
            return 0
        return int(ops[0], 0) + 1 if op == "s_nop" else 1

    problems, n_asm = [], 0
    for i, (_, op, ops, in_asm) in enumerate(ins):
        if not (op and op.startswith("v_mfma") and in_asm):
            continue
        n_asm += 1
        vdst = _regs(ops[0])
        srcs = _regs(ops[1]) | _regs(ops[2]) | (_regs(ops[3]) if len(ops) > 3 else set())
        seen, stack = {}, [(j, 0) for j in succ(i)]
        while stack:
            j, ws = stack.pop()
            if ws >= WINDOW_AFTER or seen.get(j, 1 << 30) <= ws:
                continue
            seen[j] = ws
            op2, ops2 = ins[j][1], ins[j][2]
            if op2:
                d2, u2 = _defs_uses(op2, ops2)
                chain = (op2.startswith("v_mfma") and len(ops2) > 3 and _regs(ops2[0]) == vdst
                         and _regs(ops2[3]) == vdst and not (_regs(ops2[1]) | _regs(ops2[2])) & vdst)
                if (d2 | u2) & vdst and not chain:
                    problems.append(f"{op} {ops[0]} -> {ws} wait states -> {op2} {', '.join(ops2)}")
                    continue
            stack.extend((k, ws + cost(j)) for k in succ(j))
        seen, stack = {}, [(p, 0) for p in preds[i]]
        while stack:
            j, ws = stack.pop()
            if ws >= WINDOW_BEFORE or seen.get(j, 1 << 30) <= ws:
                continue
            seen[j] = ws
            op2, ops2 = ins[j][1], ins[j][2]
            if op2 and op2.startswith("v_") and not op2.startswith("v_mfma"):
                if _defs_uses(op2, ops2)[0] & srcs:
                    problems.append(f"{op2} {ops2[0]} -> {ws} wait states -> {op} {', '.join(ops)}")
            stack.extend((k, ws + cost(j)) for k in preds[j])
    return problems, n_asm


def _compile(tmp_path_factory, src):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / (src + ".s")
    cmd = [hipcc, *_build.common_flags(), *_build.DEVICE_FLAGS.get(src, []), "--cuda-device-only",
           "-S", os.path.join(_build.CSRC, src), "-o", str(out)]
    cmd = [c for c in cmd if c != "-fPIC"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-2000:]
    return out.read_text()


# (source, kernels that use written-out MFMAs, kernels that must not spill)
SOURCES = [("fa_fwd.hip", r"fwd_kernel"), ("fa_bwd.hip", r"bwd_dkdv_kernel")]


@pytest.fixture(scope="module", params=SOURCES, ids=[s for s, _ in SOURCES])
def compiled(request, tmp_path_factory):
    src, pattern = request.param
    return _compile(tmp_path_factory, src), pattern


def test_written_out_mfmas_have_their_wait_states(compiled):
    asm, pattern = compiled
    kernels = _functions(asm, pattern)
    assert kernels, "no kernels in the assembly"
    total_asm = 0
    for name, body in kernels.items():
        problems, n_asm = _check(body)
        total_asm += n_asm
        assert not problems, f"{name}: " + "; ".join(problems[:5])
    assert total_asm > 0


def test_kernels_do_not_spill(compiled):
    asm, pattern = compiled
    for name, body in _functions(asm, pattern).items():
        assert "scratch_store" not in body and "scratch_load" not in body, f"{name} spills to scratch"


def test_checker_sees_a_missing_wait():
    """The walk flags a VALU read of a written-out MFMA's result 2 instructions later, and
    accepts it after three s_nop 7 or through a chained MFMA."""
    head = "_Zfake:\n"
    bad = head + ";;#ASMSTART\n\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]\n;;#ASMEND\n" \
        "\tv_add_f32_e32 v8, v9, v9\n\tv_accvgpr_read_b32 v10, a3\n\ts_endpgm\n.Lfunc_end0:\n"
    ok = head + ";;#ASMSTART\n\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]\n" \
        "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n;;#ASMEND\n\tv_accvgpr_read_b32 v10, a3\n\ts_endpgm\n.Lfunc_end0:\n"
    chain = head + ";;#ASMSTART\n\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]\n;;#ASMEND\n" \
        ";;#ASMSTART\n\tv_mfma_f32_32x32x16_bf16 a[0:15], v[8:11], v[4:7], a[0:15]\n" \
        "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n;;#ASMEND\n\ts_endpgm\n.Lfunc_end0:\n"
    before = head + "\tv_mov_b32_e32 v5, 0\n;;#ASMSTART\n\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], " \
        "a[0:15]\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n;;#ASMEND\n\ts_endpgm\n.Lfunc_end0:\n"
    assert _check(_functions(bad, "fake")["_Zfake"])[0]
    assert not _check(_functions(ok, "fake")["_Zfake"])[0]
    assert not _check(_functions(chain, "fake")["_Zfake"])[0]
    assert _check(_functions(before, "fake")["_Zfake"])[0]
