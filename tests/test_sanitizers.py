"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

A separate gcc build of oracle/moments_oracle.c with -fsanitize=address,undefined
is loaded in a child process (gcc's libasan preloaded, MOMENTS_ORACLE_LIB
pointing at it). The child runs the forward and the checkpointed backward over
every rotation mode, ragged valid lengths, chain subsets, row groups and several
threads, and checks the results against the numpy block form. Any out-of-bounds
access, use after free or undefined behaviour aborts the child.
"""
import os
import subprocess
import sys

import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import numpy as np
import workloads as W
from oracle import oracle_fwd, oracle_bwd, ROT_NONE, ROT_PAIRWISE, ROT_HALF, ROT_QUAT
from oracle import chunk_form as cf

def rel(x, y):
    return np.abs(x - y).max() / max(np.abs(y).max(), 1e-300)

cases = [(ROT_PAIRWISE, 8, 0, 40, 37), (ROT_HALF, 8, 0, 40, 40), (ROT_QUAT, 0, 2, 40, 33),
         (ROT_NONE, 0, 0, 40, 0), (ROT_QUAT, 0, 3, 600, 577), (ROT_PAIRWISE, 12, 0, 520, 300)]
for rot_kind, rope_dim, qb, s, V in cases:
    w = W.small("san", b=2, s=s, c=2, h=2, p=5, r=12, chunk_len=8, valid_len=V, rot_kind=rot_kind,
                rope_dim=rope_dim, quat_blocks=qb, seed=5)
    a = {k: (None if v is None else v.double().numpy().copy()) for k, v in W.generate(w).items()}
    args = (a["xhat"], a["bhat"], a["da"], a["rot"], a["h0"])
    for nt, npg, chains in ((1, None, None), (4, 2, None), (3, 5, [1, 2])):
        m2, m1 = oracle_fwd(*args, V, rot_kind, rope_dim, chains=chains, nthreads=nt, npg=npg)
        g = oracle_bwd(*args, a["d_m2"], a["d_m1"], V, rot_kind, rope_dim, chains=chains, nthreads=nt, npg=npg)
    q2, q1 = cf.moments_fwd_chunked(*args, V, rot_kind, rope_dim, 8)
    gp = cf.moments_bwd_chunked(*args, a["d_m2"], a["d_m1"], V, rot_kind, rope_dim, 8)
    m2, m1 = oracle_fwd(*args, V, rot_kind, rope_dim, nthreads=4)
    g = oracle_bwd(*args, a["d_m2"], a["d_m1"], V, rot_kind, rope_dim, nthreads=4)
    assert rel(m2, q2) < 1e-11 and rel(m1, q1) < 1e-11, (rot_kind, s, V)
    for k, v in g.items():
        if v is not None and np.abs(gp[k]).max() > 0:
            assert rel(v, gp[k]) < 1e-10, (k, rot_kind, s, V)
print("SANITIZED-OK", flush=True)
"""


def _libasan():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_asan_and_ubsan():
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's libasan is not installed")
    lib = O.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=asan, MOMENTS_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    res = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=600)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0 and "SANITIZED-OK" in res.stdout, tail
    assert "runtime error" not in res.stderr, tail
