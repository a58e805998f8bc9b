"""Barrier ordering in the generated code (CPU only: compiles for gfx950 and reads the
AMD assembly of this build).

Kernels that keep copies in flight across their barriers (the MXFP4 GEMM's
global_load_lds ring) use a bare s_barrier with explicit s_waitcnt instead of a
workgroup fence.  Their correctness then rests on every barrier being reached
with the wave's LDS reads complete (lgkmcnt 0): a read still in flight at a
barrier can be overtaken by another wave's copy into the buffer it reads.  The
compiler decides where those waits land, so the property is checked on the
code it produces: for the MXFP4 GEMM, and for the int4 GEMM and the fused
kernels, whose fenced barriers must keep it too.  (k1 is left out: the linear
scan cannot follow a loop whose waiting block the compiler lays out elsewhere,
and its barriers are all fenced.)
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "bit_diffusion_model_svdq_amd"))
import build  # noqa: E402  (the package's build script: flags and sources)

SOURCES = ["k2_mxfp4_gemm.hip", "k2_w4a4_gemm.hip", "k12_fused_smallk.hip"]
assert all(src in build.HIP_SOURCES for src in SOURCES)


def barriers_with_reads_in_flight(asm: str):
    """(kernel, barriers, barriers reached after an LDS read not yet waited for), by a
    linear scan of each kernel body in program order."""
    out = []
    for m in re.finditer(r"^(_Z\w+):[^\n]*\n(.*?)\bs_endpgm\b", asm, flags=re.S | re.M):
        pending, bad, total = False, 0, 0
        for line in m.group(2).split("\n"):
            if re.search(r"\bds_(read|bpermute|swizzle)", line):
                pending = True
            if "s_waitcnt" in line and "lgkmcnt(0)" in line:
                pending = False
            if re.search(r"\bs_barrier\b", line):
                total += 1
                bad += pending
        out.append((m.group(1), total, bad))
    return out


def test_scan_flags_a_read_left_in_flight():
    """The scan itself: a read waited for before the barrier passes, one waited for
    after it does not."""
    ok = "_Zk:  ; @_Zk\n ds_read_b128 v[0:3], v4\n s_waitcnt vmcnt(4) lgkmcnt(0)\n s_barrier\n s_endpgm\n"
    late = "_Zk:\n ds_read_u8 v0, v4\n s_waitcnt vmcnt(4)\n s_barrier\n s_waitcnt lgkmcnt(0)\n s_endpgm\n"
    assert barriers_with_reads_in_flight(ok) == [("_Zk", 1, 0)]
    assert barriers_with_reads_in_flight(late) == [("_Zk", 1, 1)]


@pytest.mark.parametrize("src", SOURCES)
def test_every_barrier_follows_the_waves_lds_reads(src, tmp_path):
    if not os.path.exists(build.HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    cmd = [build.HIPCC] + build.HIP_FLAGS + ["-S", "--cuda-device-only",
                                             os.path.join(build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    res = barriers_with_reads_in_flight(asm)
    assert len(res) == asm.count(".amdhsa_kernel "), f"{src}: kernel bodies not all found"
    bad = [(k, t, b) for k, t, b in res if b]
    assert not bad, f"{src}: barriers reached with LDS reads in flight: {bad}"
