"""MI355X-native physical-frame state moments (Mamba-3): fwd + recompute bwd.

Python entry points with the C ABI's names. They marshal torch tensors into the
HIP library (libmoments.so) and run on torch's current HIP stream; no
computation happens in Python. See include/moments.h for the operation.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (BF16, F32, ROT_HALF, ROT_NONE, ROT_PAIRWISE, ROT_QUAT, Desc,  # noqa: F401
                   MomentsError)

__all__ = ["make_desc", "moments_validate", "moments_workspace_size", "moments_fwd", "moments_bwd",
           "Desc", "MomentsError", "ROT_NONE", "ROT_PAIRWISE", "ROT_HALF", "ROT_QUAT"]


def make_desc(xhat, bhat, chunk_len, valid_len, rot_kind, rope_dim=0, quat_blocks=0, dtype=None):
    b, s, c, h, p = xhat.shape
    r = bhat.shape[-1]
    if dtype is None:
        dtype = BF16 if xhat.dtype == torch.bfloat16 else F32
    return Desc(b, s, c, h, p, r, int(chunk_len), int(valid_len), int(dtype), int(rot_kind),
                int(rope_dim), int(quat_blocks))


def moments_validate(desc: Desc) -> int:
    return _lib.load().moments_validate(ctypes.byref(desc))


def moments_workspace_size(desc: Desc, is_bwd: bool) -> int:
    n = _lib.load().moments_workspace_size(ctypes.byref(desc), int(bool(is_bwd)))
    if n < 0:
        _lib.check(int(n))
    return int(n)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors must be contiguous device tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(desc, is_bwd, device, workspace):
    n = moments_workspace_size(desc, is_bwd)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    return workspace


def moments_fwd(desc: Desc, xhat, bhat, da, rot, h0, m2=None, m1=None, workspace=None):
    """Returns (m2 [b,h,r,r], m1 [b,h,p,r]) float32."""
    dev = xhat.device
    if m2 is None:
        m2 = torch.empty(desc.b, desc.h, desc.r, desc.r, dtype=torch.float32, device=dev)
    if m1 is None:
        m1 = torch.empty(desc.b, desc.h, desc.p, desc.r, dtype=torch.float32, device=dev)
    ws = _workspace(desc, False, dev, workspace)
    rc = _lib.load().moments_fwd(ctypes.byref(desc), _ptr(xhat), _ptr(bhat), _ptr(da), _ptr(rot),
                                 _ptr(h0), _ptr(m2), _ptr(m1), _ptr(ws), ws.numel(), _stream(dev))
    _lib.check(rc)
    return m2, m1


def moments_bwd(desc: Desc, xhat, bhat, da, rot, h0, d_m2, d_m1, want=("xhat", "bhat", "da", "rot", "h0"),
                out=None, workspace=None):
    """Returns dict d_xhat, d_bhat, d_da, d_rot, d_h0 (input dtype; None when
    not wanted or not defined)."""
    dev = xhat.device
    dt = xhat.dtype
    out = dict(out or {})
    shapes = {"xhat": xhat.shape, "bhat": bhat.shape, "da": da.shape,
              "rot": None if rot is None else rot.shape,
              "h0": (desc.b, desc.h, desc.p, desc.r)}
    for k in ("xhat", "bhat", "da", "rot", "h0"):
        key = "d_" + k
        if k in want and shapes[k] is not None and not (k == "rot" and desc.rot_kind == ROT_NONE):
            if out.get(key) is None:
                out[key] = torch.empty(shapes[k], dtype=dt, device=dev)
        else:
            out[key] = None
    ws = _workspace(desc, True, dev, workspace)
    rc = _lib.load().moments_bwd(ctypes.byref(desc), _ptr(xhat), _ptr(bhat), _ptr(da), _ptr(rot),
                                 _ptr(h0), _ptr(d_m2), _ptr(d_m1), _ptr(out["d_xhat"]),
                                 _ptr(out["d_bhat"]), _ptr(out["d_da"]), _ptr(out["d_rot"]),
                                 _ptr(out["d_h0"]), _ptr(ws), ws.numel(), _stream(dev))
    _lib.check(rc)
    return out


def profile_enable(on: bool) -> bool:
    """Turn per-kernel HIP-event timing on or off; returns the previous state."""
    return bool(_lib.load().moments_profile_enable(int(bool(on))))


def profile_reset() -> None:
    _lib.load().moments_profile_reset()


def profile_read() -> dict:
    """{kernel name: (timed launches, summed ms)} of the launches timed so far."""
    lib = _lib.load()
    out = {}
    name = ctypes.c_char_p()
    n = ctypes.c_int64()
    ms = ctypes.c_double()
    count = lib.moments_profile_read(0, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms))
    _lib.check(min(count, 0))
    for i in range(count):
        lib.moments_profile_read(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms))
        out[name.value.decode()] = (int(n.value), float(ms.value))
    return out
