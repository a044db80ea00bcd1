"""The built gfx950 code of the mat-vec kernels, read back on the CPU.

Kernels that stage x with loads writing LDS directly (global_load_lds) wait
for them before the workgroup barrier with ``s_waitcnt vmcnt(N)``, where N
is the number of load instructions the wave issued after its last staging
load (the first items' weights, left in flight; loads complete in issue
order).  N is written in the source from the per-piece load counts, so this
test reads every such kernel out of the built objects and checks that
exactly N loads stand between the last staging load and the barrier, on
every path: fewer would let the barrier pass before x is in LDS.
"""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
LLVM = "/opt/rocm/llvm/bin"
TYPES = ["f16", "q8_0", "q4_k", "q6_k", "q5_0", "f32", "bf16"]

LOAD = re.compile(r"^\s*(global_load|buffer_load|flat_load)\w*")
DMA = re.compile(r"^\s*global_load_lds_dword")
WAIT = re.compile(r"^\s*s_waitcnt\b.*\bvmcnt\((\d+)\)")
BRANCH = re.compile(r"^\s*s_cbranch_\w+\s+(\S+)")
LABEL = re.compile(r"^(L\d+):$")


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        pytest.skip(f"{path} not available")
    return path


def _disassemble(obj):
    with tempfile.TemporaryDirectory() as d:
        fat, co = os.path.join(d, "fatbin"), os.path.join(d, "co")
        subprocess.run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", obj], check=True)
        subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o", f"--input={fat}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"], check=True)
        out = subprocess.run([_tool("llvm-objdump"), "-d", "--no-show-raw-insn", "--symbolize-operands", co],
                             check=True, capture_output=True, text=True).stdout
    # per kernel: instruction lines and label lines ("L12:"; branches name them)
    kernels, name = {}, None
    for line in out.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m and not LABEL.match(m.group(1) + ":"):
            name = m.group(1)
            kernels[name] = []
        elif m and name:
            kernels[name].append(m.group(1) + ":")
        elif name and line.strip():
            kernels[name].append(line.split("//")[0].strip())
    return kernels


def _labels(lines):
    """Line index of each label."""
    return {m.group(1): i for i, ln in enumerate(lines) for m in [LABEL.match(ln)] if m}


@pytest.fixture(scope="module")
def code():
    out = {}
    for t in TYPES:
        obj = os.path.join(BUILD, f"re_mv_{t}.o")
        if not os.path.exists(obj):
            pytest.fail(f"{obj} missing: build the library first (__graft_entry__.build())")
        out.update(_disassemble(obj))
    return out


def test_staging_waits_match_the_loads_in_flight(code):
    """Correct: the barrier's vmcnt(N) has N no larger than the loads issued
    after the staging (then the staging loads, issued before them, are
    done).  Exact, for instances that do not spill registers: N equals that
    count and no wait in between waits for a weight load (instances that
    spill, only reachable with a pinned schedule, may wait earlier)."""
    checked = 0
    for name, ins in code.items():
        dma = [i for i, s in enumerate(ins) if DMA.match(s)]
        if not dma:
            continue
        last = dma[-1]
        bar = next(i for i in range(last, len(ins)) if ins[i].startswith("s_barrier"))
        waits = [(i, int(WAIT.match(ins[i]).group(1))) for i in range(last + 1, bar) if WAIT.match(ins[i])]
        assert waits, f"{name}: no vmcnt wait between the staging loads and the barrier"
        wi, n = waits[-1]
        assert all(not LOAD.match(ins[i]) for i in range(wi + 1, bar)), name
        loads = [i for i in range(last + 1, wi) if LOAD.match(ins[i]) and not DMA.match(ins[i])]
        # every load is on every path: no branch in the range skips one
        addr = _labels(ins)
        for i in range(last + 1, wi):
            m = BRANCH.match(ins[i])
            if m:
                j = addr.get(m.group(1))
                assert j is not None and j > i, f"{name}: branch to {m.group(1)} in the staging range"
                assert not any(i < q < j for q in loads), f"{name}: a branch skips a weight load"
        drained = any(v == 0 for _, v in waits[:-1])
        assert n <= len(loads) or drained, \
            f"{name}: vmcnt({n}) before the barrier with only {len(loads)} loads after the staging"
        if not any("scratch_" in s for s in ins):
            assert n == len(loads), f"{name}: vmcnt({n}) before the barrier, {len(loads)} loads in flight"
            for i, v in waits[:-1]:
                issued = sum(1 for j in loads if j < i)
                assert v >= issued, f"{name}: vmcnt({v}) waits for weight loads ({issued} issued)"
        checked += 1
    assert checked > 0, "no kernel stages x with LDS loads"
