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

__all__ = ["make_desc", "set_valid_lens", "moments_validate", "moments_workspace_size", "moments_fwd", "moments_fwd_static",
           "moments_bwd", "moments_saved_size", "moments_fwd_save", "moments_bwd_saved", "rot_desc", "moments_rot_workspace_size", "moments_rot_fwd", "moments_rot_bwd",
           "kernel_chunk_len",
           "Desc", "MomentsError", "ROT_NONE", "ROT_PAIRWISE", "ROT_HALF", "ROT_QUAT"]


def make_desc(xhat, bhat, chunk_len, valid_len, rot_kind, rope_dim=0, quat_blocks=0, dtype=None,
              valid_lens=None):
    b, s, c, h, p = xhat.shape
    r = bhat.shape[-1]
    if dtype is None:
        dtype = BF16 if xhat.dtype == torch.bfloat16 else F32
    d = Desc(b, s, c, h, p, r, int(chunk_len), int(valid_len), int(dtype), int(rot_kind),
             int(rope_dim), int(quat_blocks))
    return set_valid_lens(d, valid_lens)


def set_valid_lens(desc: Desc, valid_lens):
    """Per-sequence valid lengths: ``valid_lens`` is an int32 GPU tensor of shape
    [b] (or None for one length, desc.valid_len, for the whole batch). Sequence
    bi then uses min(max(valid_lens[bi], 0), desc.valid_len, s). The descriptor
    keeps a reference to the tensor, whose contents the kernels read."""
    if valid_lens is None:
        desc.valid_lens = None
        desc._valid_lens_ref = None
        return desc
    if not isinstance(valid_lens, torch.Tensor):
        raise ValueError("valid_lens must be a torch.Tensor")
    if tuple(valid_lens.shape) != (int(desc.b),) or valid_lens.dtype != torch.int32:
        raise ValueError(f"valid_lens must be int32 of shape ({desc.b},), got {valid_lens.dtype} "
                         f"{tuple(valid_lens.shape)}")
    if valid_lens.device.type != "cuda" or not valid_lens.is_contiguous():
        raise ValueError("valid_lens must be a contiguous GPU tensor")
    desc.valid_lens = valid_lens.data_ptr()
    desc._valid_lens_ref = valid_lens
    return desc


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
    return ctypes.c_void_p(t.data_ptr())


def _expect(name, t, shape, dtype, device, optional=False):
    """Raises ValueError unless t is a contiguous tensor of exactly this shape and
    dtype on this device (the kernels index every buffer from the descriptor)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, the descriptor needs {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, the descriptor needs {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _input_specs(desc: Desc):
    """Expected shapes and dtype of the five inputs (rot: None when there is no rotation)."""
    b, s, c, h, p, r = desc.b, desc.s, desc.c, desc.h, desc.p, desc.r
    if desc.rot_kind in (ROT_PAIRWISE, ROT_HALF):
        rot = (b, s, h, desc.rope_dim // 2)
    elif desc.rot_kind == ROT_QUAT:
        rot = (b, s, h, desc.quat_blocks, 4)
    else:
        rot = None
    dt = torch.bfloat16 if desc.dtype == BF16 else torch.float32
    return {"xhat": (b, s, c, h, p), "bhat": (b, s, c, h, r), "da": (b, s, h), "rot": rot,
            "h0": (b, h, p, r)}, dt


def _check_inputs(desc: Desc, xhat, bhat, da, rot, h0):
    """Shapes, dtypes and devices of the inputs against the descriptor (all on
    xhat's device, which must be a GPU)."""
    if not isinstance(xhat, torch.Tensor):
        raise ValueError("xhat must be a torch.Tensor")
    dev = xhat.device
    if desc.valid_lens:
        ref = getattr(desc, "_valid_lens_ref", None)
        if ref is None or ref.data_ptr() != desc.valid_lens:
            raise ValueError("set per-sequence lengths with set_valid_lens (the descriptor keeps the tensor)")
        if ref.device != dev:
            raise ValueError(f"valid_lens is on {ref.device}, the inputs on {dev}")
    specs, dt = _input_specs(desc)
    _expect("xhat", xhat, specs["xhat"], dt, dev)
    _expect("bhat", bhat, specs["bhat"], dt, dev)
    _expect("da", da, specs["da"], dt, dev)
    if specs["rot"] is None:
        if rot is not None:
            raise ValueError("rot must be None when the descriptor has no rotation")
    else:
        _expect("rot", rot, specs["rot"], dt, dev)
    _expect("h0", h0, specs["h0"], dt, dev, optional=True)
    return dev, specs, dt


def _require_gpu(dev):
    if dev.type != "cuda":
        raise ValueError(f"the inputs are on {dev}; the kernels need GPU tensors")
    _lib.load()


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(desc, is_bwd, device, workspace):
    n = moments_workspace_size(desc, is_bwd)
    if workspace is None:
        return torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if workspace.numel() * workspace.element_size() < n:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"the descriptor needs {n}")
    return workspace


def moments_fwd(desc: Desc, xhat, bhat, da, rot, h0, m2=None, m1=None, workspace=None):
    """Returns (m2 [b,h,r,r], m1 [b,h,p,r]) float32."""
    dev, _, _ = _check_inputs(desc, xhat, bhat, da, rot, h0)
    _expect("m2", m2, (desc.b, desc.h, desc.r, desc.r), torch.float32, dev, optional=True)
    _expect("m1", m1, (desc.b, desc.h, desc.p, desc.r), torch.float32, dev, optional=True)
    _require_gpu(dev)
    if m2 is None:
        m2 = torch.empty(desc.b, desc.h, desc.r, desc.r, dtype=torch.float32, device=dev)
    if m1 is None:
        m1 = torch.empty(desc.b, desc.h, desc.p, desc.r, dtype=torch.float32, device=dev)
    ws = _workspace(desc, False, dev, workspace)
    rc = _lib.load().moments_fwd(ctypes.byref(desc), _ptr(xhat), _ptr(bhat), _ptr(da), _ptr(rot),
                                 _ptr(h0), _ptr(m2), _ptr(m1), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(dev))
    _lib.check(rc)
    return m2, m1


def moments_fwd_static(desc: Desc, xhat, bhat, da, rot, h0, m2, m1):
    """moments_fwd without a workspace: the library's static device scratch
    (64 MiB per GPU) holds the kernels' intermediates. m2 and m1 are the
    caller's float32 output tensors; nothing is allocated here."""
    dev, _, _ = _check_inputs(desc, xhat, bhat, da, rot, h0)
    _expect("m2", m2, (desc.b, desc.h, desc.r, desc.r), torch.float32, dev)
    _expect("m1", m1, (desc.b, desc.h, desc.p, desc.r), torch.float32, dev)
    _require_gpu(dev)
    rc = _lib.load().moments_fwd_static(ctypes.byref(desc), _ptr(xhat), _ptr(bhat), _ptr(da), _ptr(rot),
                                        _ptr(h0), _ptr(m2), _ptr(m1), _stream(dev))
    _lib.check(rc)
    return m2, m1


def moments_saved_size(desc: Desc) -> int:
    """Bytes of the saved-carry buffer of moments_fwd_save / moments_bwd_saved."""
    n = _lib.load().moments_saved_size(ctypes.byref(desc))
    if n < 0:
        _lib.check(int(n))
    return int(n)


def _saved_buffer(desc, device, saved):
    n = moments_saved_size(desc)
    if saved is None:
        return torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    if not isinstance(saved, torch.Tensor) or saved.device != device or not saved.is_contiguous():
        raise ValueError(f"saved must be a contiguous tensor on {device}")
    if saved.numel() * saved.element_size() < n:
        raise ValueError(f"saved holds {saved.numel() * saved.element_size()} bytes, the descriptor needs {n}")
    return saved


def moments_fwd_save(desc: Desc, xhat, bhat, da, rot, h0, m2=None, m1=None, saved=None, workspace=None):
    """moments_fwd that also keeps the chunk-boundary states for the backward.
    Returns (m2, m1, saved); saved is an opaque uint8 device tensor to pass to
    moments_bwd_saved with the same descriptor and inputs."""
    dev, _, _ = _check_inputs(desc, xhat, bhat, da, rot, h0)
    _expect("m2", m2, (desc.b, desc.h, desc.r, desc.r), torch.float32, dev, optional=True)
    _expect("m1", m1, (desc.b, desc.h, desc.p, desc.r), torch.float32, dev, optional=True)
    _require_gpu(dev)
    if m2 is None:
        m2 = torch.empty(desc.b, desc.h, desc.r, desc.r, dtype=torch.float32, device=dev)
    if m1 is None:
        m1 = torch.empty(desc.b, desc.h, desc.p, desc.r, dtype=torch.float32, device=dev)
    sv = _saved_buffer(desc, dev, saved)
    ws = _workspace(desc, False, dev, workspace)
    rc = _lib.load().moments_fwd_save(ctypes.byref(desc), _ptr(xhat), _ptr(bhat), _ptr(da), _ptr(rot),
                                      _ptr(h0), _ptr(m2), _ptr(m1), _ptr(sv), sv.numel(), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(dev))
    _lib.check(rc)
    return m2, m1, sv


def moments_bwd_saved(desc: Desc, xhat, bhat, da, rot, h0, saved, d_m2, d_m1,
                      want=("xhat", "bhat", "da", "rot", "h0"), out=None, workspace=None):
    """moments_bwd reading the chunk-boundary states moments_fwd_save kept
    (no carry pass). Same returns as moments_bwd."""
    return moments_bwd(desc, xhat, bhat, da, rot, h0, d_m2, d_m1, want=want, out=out, workspace=workspace,
                       _saved=saved)


def moments_bwd(desc: Desc, xhat, bhat, da, rot, h0, d_m2, d_m1, want=("xhat", "bhat", "da", "rot", "h0"),
                out=None, workspace=None, _saved=None):
    """Returns dict d_xhat, d_bhat, d_da, d_rot, d_h0 (input dtype; None when
    not wanted or not defined)."""
    dev, specs, dt = _check_inputs(desc, xhat, bhat, da, rot, h0)
    _expect("d_m2", d_m2, (desc.b, desc.h, desc.r, desc.r), torch.float32, dev)
    _expect("d_m1", d_m1, (desc.b, desc.h, desc.p, desc.r), torch.float32, dev)
    out = dict(out or {})
    for k in ("xhat", "bhat", "da", "rot", "h0"):
        key = "d_" + k
        if k in want and specs[k] is not None:
            _expect(key, out.get(key), specs[k], dt, dev, optional=True)
        else:
            out[key] = None
    _require_gpu(dev)
    for k in ("xhat", "bhat", "da", "rot", "h0"):
        key = "d_" + k
        if k in want and specs[k] is not None and out.get(key) is None:
            out[key] = torch.empty(specs[k], dtype=dt, device=dev)
    ws = _workspace(desc, True, dev, workspace)
    grads = (_ptr(d_m2), _ptr(d_m1), _ptr(out["d_xhat"]), _ptr(out["d_bhat"]), _ptr(out["d_da"]),
             _ptr(out["d_rot"]), _ptr(out["d_h0"]), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    if _saved is None:
        rc = _lib.load().moments_bwd(ctypes.byref(desc), _ptr(xhat), _ptr(bhat), _ptr(da), _ptr(rot),
                                     _ptr(h0), *grads)
    else:
        sv = _saved_buffer(desc, dev, _saved)
        rc = _lib.load().moments_bwd_saved(ctypes.byref(desc), _ptr(xhat), _ptr(bhat), _ptr(da), _ptr(rot),
                                           _ptr(h0), _ptr(sv), sv.numel() * sv.element_size(), *grads)
    _lib.check(rc)
    return out


def rot_desc(inc, rot_kind, rope_dim=0, quat_blocks=0):
    """Descriptor of the rotation-sequence producer for increments ``inc``
    ([b,s,h,a] angles with rope_dim = 2a, or [b,s,h,J,4] quaternions). Only b,
    s, h, dtype, rot_kind and rope_dim / quat_blocks are read by the library."""
    if not isinstance(inc, torch.Tensor):
        raise ValueError("inc must be a torch.Tensor")
    b, s, h = (int(x) for x in inc.shape[:3])
    if rot_kind == ROT_QUAT and quat_blocks == 0 and inc.dim() == 5:
        quat_blocks = int(inc.shape[3])
    if rot_kind in (ROT_PAIRWISE, ROT_HALF) and rope_dim == 0 and inc.dim() == 4:
        rope_dim = 2 * int(inc.shape[3])
    dtype = BF16 if inc.dtype == torch.bfloat16 else F32
    return Desc(b, s, 1, h, 1, 1, 1, s, int(dtype), int(rot_kind), int(rope_dim), int(quat_blocks))


def _rot_shape(desc: Desc):
    if desc.rot_kind == ROT_QUAT:
        return (desc.b, desc.s, desc.h, desc.quat_blocks, 4)
    if desc.rot_kind in (ROT_PAIRWISE, ROT_HALF):
        return (desc.b, desc.s, desc.h, desc.rope_dim // 2)
    raise ValueError("the producer needs a rotation (rot_kind must not be ROT_NONE)")


def moments_rot_workspace_size(desc: Desc, is_bwd: bool) -> int:
    n = _lib.load().moments_rot_workspace_size(ctypes.byref(desc), int(bool(is_bwd)))
    if n < 0:
        _lib.check(int(n))
    return int(n)


def _rot_call(desc, is_bwd, inc, d_rot, out):
    if not isinstance(inc, torch.Tensor):
        raise ValueError("inc must be a torch.Tensor")
    dev = inc.device
    shape = _rot_shape(desc)
    dt = torch.bfloat16 if desc.dtype == BF16 else torch.float32
    _expect("inc", inc, shape, dt, dev)
    if is_bwd:
        _expect("d_rot", d_rot, shape, dt, dev)
    _expect("out", out, shape, dt, dev, optional=True)
    _require_gpu(dev)
    if out is None:
        out = torch.empty(shape, dtype=dt, device=dev)
    n = moments_rot_workspace_size(desc, is_bwd)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    lib = _lib.load()
    if is_bwd:
        rc = lib.moments_rot_bwd(ctypes.byref(desc), _ptr(inc), _ptr(d_rot), _ptr(out), _ptr(ws), n, _stream(dev))
    else:
        rc = lib.moments_rot_fwd(ctypes.byref(desc), _ptr(inc), _ptr(out), _ptr(ws), n, _stream(dev))
    _lib.check(rc)
    return out


def moments_rot_fwd(desc: Desc, inc, rot=None):
    """Cumulative rotation (the moments path's ``rot``) from per-token increments."""
    return _rot_call(desc, False, inc, None, rot)


def moments_rot_bwd(desc: Desc, inc, d_rot, d_inc=None):
    """Cotangent of the increments from the cotangent of the cumulative rotation."""
    return _rot_call(desc, True, inc, d_rot, d_inc)


def kernel_chunk_len() -> int:
    """Tokens per kernel chunk (the kernels' own chunking, whatever chunk_len is)."""
    return int(_lib.load().moments_kernel_chunk_len())


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
