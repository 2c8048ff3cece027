"""ctypes front end of the C oracle (test infrastructure; see package docstring)."""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

ROT_NONE, ROT_PAIRWISE, ROT_HALF, ROT_QUAT = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moments_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")
_LIB_SAN = os.path.join(_HERE, "_build", "liboracle_san.so")
_lock = threading.Lock()
_lib = None


class _Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("b", "s", "c", "h", "p", "r", "valid_len", "rot_kind", "rope_dim", "quat_blocks")]


def library_path() -> str:
    return _LIB


def build(sanitize: bool = False) -> str:
    """Compile the oracle with gcc (always recompiles). With ``sanitize``, a
    separate AddressSanitizer + UndefinedBehaviorSanitizer build
    (liboracle_san.so), which a process loads through MOMENTS_ORACLE_LIB with
    gcc's libasan preloaded."""
    out = _LIB_SAN if sanitize else _LIB
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    opt = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=undefined"] if sanitize else ["-O3", "-march=x86-64-v3"])
    subprocess.run(["gcc", *opt, "-fPIC", "-shared", "-std=c11", "-pthread", _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("MOMENTS_ORACLE_LIB") or _LIB
            if path == _LIB and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                build()
            lib = ctypes.CDLL(path)
            dp = ctypes.POINTER(ctypes.c_double)
            ip = ctypes.POINTER(ctypes.c_int64)
            lib.oracle_fwd.argtypes = [ctypes.POINTER(_Desc)] + [dp] * 7 + [ip, ctypes.c_int64, ctypes.c_int64,
                                                               ctypes.c_int]
            lib.oracle_bwd.argtypes = [ctypes.POINTER(_Desc)] + [dp] * 12 + [ip, ctypes.c_int64, ctypes.c_int64,
                                                                ctypes.c_int]
            lib.oracle_fwd.restype = ctypes.c_int
            lib.oracle_bwd.restype = ctypes.c_int
            _lib = lib
    return _lib


def _desc(b, s, c, h, p, r, valid_len, rot_kind, rope_dim, quat_blocks):
    return _Desc(b, s, c, h, p, r, valid_len, rot_kind, rope_dim, quat_blocks)


def _f64(a):
    if a is None:
        return None
    a = np.asarray(a, dtype=np.float64)
    return np.ascontiguousarray(a)


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shapes(xhat, bhat):
    b, s, c, h, p = xhat.shape
    r = bhat.shape[-1]
    return b, s, c, h, p, r


def _rot_meta(rot_kind, rope_dim, rot):
    if rot_kind == ROT_QUAT:
        return 0, int(rot.shape[3])
    if rot_kind in (ROT_PAIRWISE, ROT_HALF):
        return int(rope_dim), 0
    return 0, 0


def _chains(chains):
    if chains is None:
        return None, ctypes.POINTER(ctypes.c_int64)(), 0
    arr = np.ascontiguousarray(np.asarray(chains, dtype=np.int64))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(arr.size)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _npg(nchains, p, nthreads, npg):
    if npg:
        return int(npg)
    return max(1, min(p, -(-nthreads // max(1, nchains))))


def oracle_fwd(xhat, bhat, da, rot, h0, valid_len, rot_kind, rope_dim=0, chains=None, nthreads=None,
               npg=None):
    """Returns (m2[b,h,r,r], m1[b,h,p,r]) in fp64. ``chains`` restricts the work
    to the listed flat (b*h + h) chain ids; other chains' outputs stay zero."""
    xhat, bhat, da, rot, h0 = map(_f64, (xhat, bhat, da, rot, h0))
    b, s, c, h, p, r = _shapes(xhat, bhat)
    rd, qb = _rot_meta(rot_kind, rope_dim, rot)
    d = _desc(b, s, c, h, p, r, int(valid_len), rot_kind, rd, qb)
    m2 = np.zeros((b, h, r, r))
    m1 = np.zeros((b, h, p, r))
    keep, cp, nc = _chains(chains)
    nt = int(nthreads or default_threads())
    g = _npg(nc or b * h, p, nt, npg)
    rc = _load().oracle_fwd(ctypes.byref(d), _ptr(xhat), _ptr(bhat), _ptr(da), _ptr(rot), _ptr(h0),
                            _ptr(m2), _ptr(m1), cp, nc, g, nt)
    if rc != 0:
        raise ValueError("oracle_fwd rejected the descriptor")
    return m2, m1


def oracle_bwd(xhat, bhat, da, rot, h0, dm2, dm1, valid_len, rot_kind, rope_dim=0, chains=None,
               nthreads=None, npg=None):
    """Returns dict of fp64 gradients d_xhat, d_bhat, d_da, d_rot (None if no
    rotation), d_h0 — the VJP of (m2, m1[b,h,p,r]) with cotangents (dm2, dm1)."""
    xhat, bhat, da, rot, h0, dm2, dm1 = map(_f64, (xhat, bhat, da, rot, h0, dm2, dm1))
    b, s, c, h, p, r = _shapes(xhat, bhat)
    rd, qb = _rot_meta(rot_kind, rope_dim, rot)
    d = _desc(b, s, c, h, p, r, int(valid_len), rot_kind, rd, qb)
    out = {
        "d_xhat": np.zeros_like(xhat), "d_bhat": np.zeros_like(bhat), "d_da": np.zeros_like(da),
        "d_rot": np.zeros_like(rot) if (rot is not None and rot_kind != ROT_NONE) else None,
        "d_h0": np.zeros((b, h, p, r)),
    }
    keep, cp, nc = _chains(chains)
    nt = int(nthreads or default_threads())
    g = _npg(nc or b * h, p, nt, npg)
    rc = _load().oracle_bwd(ctypes.byref(d), _ptr(xhat), _ptr(bhat), _ptr(da), _ptr(rot), _ptr(h0),
                            _ptr(dm2), _ptr(dm1), _ptr(out["d_xhat"]), _ptr(out["d_bhat"]),
                            _ptr(out["d_da"]), _ptr(out["d_rot"]), _ptr(out["d_h0"]), cp, nc, g, nt)
    if rc != 0:
        raise ValueError("oracle_bwd rejected the descriptor")
    return out
