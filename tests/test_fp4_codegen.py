"""The FP4 prefill kernel's generated code keeps its loads in flight.

Each step of `ffn_fp4` issues the next chunk's activation copy (global-to-LDS)
and weight loads, then runs the current chunk's MFMAs. A wait for every
outstanding vector-memory operation between those loads and the MFMAs would
make each step wait for the loads it has just issued, so no weight load would
overlap any arithmetic. The compiler inserts exactly that wait when it is left
to place the wait for the current chunk's registers (with a global-to-LDS copy
outstanding it waits for all loads); the kernel therefore waits explicitly at
the top of the step. The same holds for the LDS operand reads of each MFMA
step: they are issued a step ahead, behind the previous step's first MFMA.
These tests compile the kernel for gfx950 (no GPU needed) and check the
instruction order in every step of both GEMMs.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "expert_weight_residency_amd", "csrc", "ffn_fp4.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("fp4") / "ffn_fp4.s"
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "--offload-arch=gfx950", "-O3",
           "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"), "--cuda-device-only", "-S", "-o", str(out), SRC]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    return out.read_text()


def kernel_body(asm, gate_up):
    name = re.search(r"^(_Z\w*ffn_fp4ILb%dE\w*):" % (1 if gate_up else 0), asm, re.M)
    assert name, "ffn_fp4 kernel not found in the assembly"
    start = name.end()
    return asm[start:asm.index("s_endpgm", start)]


def steps(body):
    """Instruction streams between consecutive barriers."""
    ops = []
    for line in body.splitlines():
        t = line.strip()
        if t.startswith("s_barrier"):
            ops.append("BAR")
        elif t.startswith("global_load_lds"):
            ops.append("COPY")
        elif t.startswith("global_load_dwordx4"):
            ops.append("W")
        elif t.startswith("v_mfma"):
            ops.append("MFMA")
        elif t.startswith("s_waitcnt"):
            m = re.search(r"vmcnt\((\d+)\)", t)
            if m:
                ops.append("VM%s" % m.group(1))
    out, cur = [], []
    for o in ops:
        if o == "BAR":
            out.append(cur)
            cur = []
        else:
            cur.append(o)
    out.append(cur)
    return out


@pytest.mark.parametrize("gate_up", [True, False], ids=["gate_up", "down"])
def test_no_full_wait_between_weight_loads_and_mfma(asm, gate_up):
    checked = 0
    for seg in steps(kernel_body(asm, gate_up)):
        if "MFMA" not in seg or "W" not in seg or "COPY" not in seg:
            continue
        first_w = seg.index("W")
        first_mfma = seg.index("MFMA")
        if first_mfma < first_w:
            continue
        checked += 1
        between = seg[first_w:first_mfma]
        assert "VM0" not in between, (
            "a wait for every outstanding load sits between the next chunk's weight loads "
            "and this chunk's MFMAs: " + " ".join(seg[:first_mfma + 1]))
    assert checked >= 4, "no steady-state step found in the assembly"


def lds_streams(body):
    """Per segment between barriers: LDS operand reads, MFMAs and LDS waits."""
    out, cur = [], []
    for line in body.splitlines():
        t = line.strip()
        if t.startswith("s_barrier"):
            out.append(cur)
            cur = []
        elif t.startswith("ds_read_b128"):
            cur.append("DS")
        elif t.startswith("v_mfma"):
            cur.append("MFMA")
        elif t.startswith("s_waitcnt") and "lgkmcnt" in t:
            cur.append("LGKM")
    out.append(cur)
    return out


@pytest.mark.parametrize("gate_up", [True, False], ids=["gate_up", "down"])
def test_operand_reads_issued_a_step_ahead(asm, gate_up):
    """Each step's B-operand reads from LDS go out right after the previous
    step's first MFMA, so that step's other 7 MFMAs run before the wait for
    them (the wait counts every outstanding LDS read). A schedule that issues
    them late, after most of the MFMAs, leaves each step waiting for an LDS
    round trip."""
    covers = []
    for seg in lds_streams(kernel_body(asm, gate_up)):
        if "MFMA" not in seg:
            continue
        first_mfma = seg.index("MFMA")
        for i in range(first_mfma, len(seg)):
            if seg[i] != "DS":
                continue
            n = 0
            for o in seg[i + 1:]:
                if o == "LGKM":
                    break
                n += o == "MFMA"
            covers.append(n)
    assert len(covers) >= 16, "no steady-state operand reads found in the assembly"
    assert min(covers) >= 7, (
        "an LDS operand read is followed by fewer than 7 MFMAs before the wait for it: "
        "min %d over %d reads" % (min(covers), len(covers)))
