"""Build the HIP library ``libw4a16.so`` in-tree for gfx950 with hipcc.

Each source compiles to its own object in parallel (no cross-file device
references, so no relocatable device code is needed), then one link step
makes the shared library.

    python -m weight_only_int4_rtn_amd.build
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4a16.so")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMPILE_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # gfx950: no packed-FP32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE behaviour the quantizer relies on: correctly rounded FP32
    # division and gradual underflow
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]
# kept for callers that read the single-command flag list
FLAGS = COMPILE_FLAGS + ["-shared"]

# hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
_NOISE = "is not a recognized feature for this target"


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in proc.stderr.splitlines() if _NOISE not in ln)
    return proc.returncode, err


def build(verbose: bool = False, extra_flags=(), jobs: int | None = None) -> str:
    """Compile every source into the in-tree shared library (always rebuilds)."""
    srcs = sources()
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with tempfile.TemporaryDirectory(prefix="w4a16_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]
        cmds = [[HIPCC, *COMPILE_FLAGS, *extra_flags, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for cmd, (rc, err) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-3]}:\n{err}")
            if err.strip() and verbose:
                print(err, file=sys.stderr)
        tmp = LIB + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        rc, err = _run(link)
        if rc != 0:
            raise RuntimeError(f"hipcc link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
