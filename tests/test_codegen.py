"""Generated-code checks of the streaming kernels (host only: hipcc compiles
them to gfx950 assembly with the library's own flags).

Every weight and x load of the small- and mid-M kernels and of the GEMM is
meant to be in flight together with the others, each use waiting only for its
own data.  A code generator that instead waits for every load right after
issuing it (`s_waitcnt vmcnt(0)` directly behind each load) serialises the
memory round trips; a harmless-looking source edit once did that to the
small-M MFMA kernel (1.8x slower launches).  At most two such pairs per
kernel are expected: a final bias read and the GEMM's prologue wait."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from weight_only_int4_rtn_amd import build as libbuild  # noqa: E402

CSRC = os.path.join(ROOT, "weight_only_int4_rtn_amd", "csrc")
SOURCES = ("gemv.hip", "mgemv.hip", "skinny.hip", "gemm.hip", "gemm8_rows256.hip", "gemm8_rows128.hip")


def _assembly(src, tmp_path):
    out = tmp_path / (src + ".s")
    flags = [f for f in libbuild.FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [libbuild.HIPCC, *flags, "--cuda-device-only", "-S", "-I" + CSRC, os.path.join(CSRC, src), "-o", str(out)]
    proc = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert proc.returncode == 0, proc.stderr[-2000:]
    return out.read_text()


def _serialised_loads(asm):
    """{kernel: number of vector loads directly followed by a full wait}"""
    counts = {}
    for name in re.findall(r"^(_ZN5w4a16\w+):", asm, re.M):
        body = asm[asm.index(name + ":"):asm.index(".Lfunc_end", asm.index(name + ":"))]
        lines = [ln.strip() for ln in body.splitlines() if ln.strip() and not ln.strip().startswith(";")]
        counts[name] = sum(1 for a, b in zip(lines, lines[1:])
                           if a.startswith(("global_load", "buffer_load")) and b.startswith("s_waitcnt vmcnt(0)"))
    return counts


@pytest.mark.skipif(not shutil.which(libbuild.HIPCC) and not os.path.exists(libbuild.HIPCC), reason="hipcc not found")
@pytest.mark.parametrize("src", SOURCES)
def test_loads_stay_in_flight(src, tmp_path):
    counts = _serialised_loads(_assembly(src, tmp_path))
    assert counts, f"no kernels found in {src}"
    bad = {k: v for k, v in counts.items() if v > 2}
    assert not bad, f"{src}: kernels that wait for each load before the next: {bad}"


def _lds_read_runs(asm):
    """{kernel: [(address register, [(first, last) destination registers])]}
    for every run of consecutive ds_read_b128 (an asm block of reads that
    are all issued before one wait)."""
    runs = {}
    for name in re.findall(r"^(_ZN5w4a16\w+):", asm, re.M):
        body = asm[asm.index(name + ":"):asm.index(".Lfunc_end", asm.index(name + ":"))].splitlines()
        cur = []
        out = []
        for ln in body:
            m = re.match(r"\s*ds_read_b128 v\[(\d+):(\d+)\], v(\d+)", ln)
            if m:
                cur.append((int(m.group(3)), int(m.group(1)), int(m.group(2))))
            elif ln.strip() and not ln.strip().startswith(";"):
                if len(cur) > 1:
                    out.append(cur)
                cur = []
        runs[name] = out
    return runs


@pytest.mark.skipif(not shutil.which(libbuild.HIPCC) and not os.path.exists(libbuild.HIPCC), reason="hipcc not found")
def test_lds_read_runs_keep_their_address(tmp_path):
    """In a run of LDS reads issued back to back, no read may write the
    address register of a later one: its returning data would change that
    read's address (the mid-M kernel reads a pair of groups' x fragments in one
    asm block; its outputs are early-clobber for this reason)."""
    runs = _lds_read_runs(_assembly("skinny.hip", tmp_path))
    assert any(runs.values()), "no runs of LDS reads found"
    bad = {k: [r for r in v if _clobbers_later_address(r)] for k, v in runs.items()}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, f"LDS read runs that overwrite a later read's address register: {bad}"


def _clobbers_later_address(run):
    """True if a read's destination holds the address register of a read
    after it in the run (the last read may overwrite its own address: it has
    been read at issue)."""
    return any(lo <= run[j][0] <= hi for i, (_, lo, hi) in enumerate(run) for j in range(i + 1, len(run)))
