"""Build the HIP library libmoments.so for gfx950 (in-tree, under _build/).

Three translation units: moments.hip (the C ABI, the dispatcher and every
kernel but the lane-pair forward), and fwd4.hip twice, for the lane-pair
forward's instances that do not save carries (with the ILP machine-scheduling
strategy) and for those that do (default strategy). They are compiled in
parallel and linked with no undefined symbols allowed."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libmoments.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# object -> (source, extra compiler flags)
UNITS = {
    "moments.o": ("moments.hip", []),
    "fwd4.o": ("fwd4.hip", ["-DMOM_FWD4_SAVE=0", "-mllvm", "-amdgpu-sched-strategy=max-ilp"]),
    "fwd4_save.o": ("fwd4.hip", ["-DMOM_FWD4_SAVE=1"]),
}


def _clean(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops' is not a recognized" not in l)


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    procs = []
    for name, (unit, extra) in UNITS.items():
        obj = os.path.join(OUT_DIR, name)
        cmd = [HIPCC, *FLAGS, *extra, *inc, "-c", os.path.join(CSRC, unit), "-o", obj]
        procs.append((name, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    errs = []
    for unit, obj, p in procs:
        _, err = p.communicate()
        err = _clean(err)
        if p.returncode != 0:
            errs.append(f"hipcc failed on {unit} ({p.returncode}):\n{err}")
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if errs:
        raise RuntimeError("\n".join(errs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined",
           *[obj for _, obj, _ in procs], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{_clean(res.stderr)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
