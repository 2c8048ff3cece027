"""The C-ABI library loads, exports every declared symbol, and validates
descriptors on the host (no GPU needed for any of this)."""
import ctypes
import os
import re

import pytest

import mamba_ssm_chunkwise_amd as M
from mamba_ssm_chunkwise_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moments.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moments_\w+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.moments_strerror(0) == b"ok"


def _desc(**kw):
    d = dict(b=2, s=64, c=2, h=3, p=8, r=16, chunk_len=16, valid_len=50, dtype=M.F32,
             rot_kind=M.ROT_PAIRWISE, rope_dim=8, quat_blocks=0)
    d.update(kw)
    return M.Desc(**d)


@pytest.mark.parametrize("kw,code", [
    ({}, 0),
    (dict(dtype=M.BF16), 0),
    (dict(rot_kind=M.ROT_QUAT, rope_dim=0, quat_blocks=4), 0),
    (dict(rot_kind=M.ROT_HALF, rope_dim=16), 0),
    (dict(rot_kind=M.ROT_NONE, rope_dim=0), 0),
    (dict(valid_len=0), 0),
    (dict(valid_len=10 ** 6), 0),
    (dict(s=60), -1),                      # s % chunk_len != 0
    (dict(chunk_len=0), -1),
    (dict(p=0), -1),
    (dict(valid_len=-1), -1),
    (dict(rope_dim=7), -1),                # odd rope_dim
    (dict(rope_dim=18), -1),               # rope_dim > r
    (dict(rot_kind=M.ROT_HALF, r=15, rope_dim=4), -1),   # half-split needs even r
    (dict(rot_kind=M.ROT_QUAT, quat_blocks=5), -1),      # 4J > r
    (dict(rot_kind=9), -1),
    (dict(dtype=7), -1),
    (dict(r=129), -2),                     # beyond the compiled kernels
    (dict(c=5), -2),
])
def test_validate(kw, code):
    assert M.moments_validate(_desc(**kw)) == code


def test_workspace_sizes_are_positive_and_grow():
    small = M.moments_workspace_size(_desc(), False)
    big = M.moments_workspace_size(_desc(s=640, valid_len=640), False)
    assert 0 < small < big
    assert M.moments_workspace_size(_desc(), True) > 0
    with pytest.raises(M.MomentsError):
        M.moments_workspace_size(_desc(p=0), True)


def test_null_and_workspace_errors_without_gpu():
    """Argument errors are caught before anything touches a device."""
    lib = _lib.load()
    d = _desc()
    null = ctypes.c_void_p()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    rc = lib.moments_fwd(ctypes.byref(d), null, fake, fake, fake, null, fake, fake, fake, 1 << 40, null)
    assert rc == _lib.EINVAL
    rc = lib.moments_fwd(ctypes.byref(d), fake, fake, fake, fake, null, fake, fake, fake, 16, null)
    assert rc == _lib.EWORKSPACE
    misaligned = ctypes.c_void_p((1 << 20) + 4)
    rc = lib.moments_fwd(ctypes.byref(d), misaligned, fake, fake, fake, null, fake, fake, fake, 1 << 40, null)
    assert rc == _lib.EINVAL
    dn = _desc(rot_kind=M.ROT_NONE, rope_dim=0)
    rc = lib.moments_bwd(ctypes.byref(dn), fake, fake, fake, null, null, fake, fake, fake, fake, fake,
                         fake, fake, fake, 1 << 40, null)
    assert rc == _lib.EINVAL  # d_rot given without a rotation


# ---------------------------------------------------------------- binding argument checks
def _tensors(d, dtype=None):
    import torch
    dt = dtype or (torch.bfloat16 if d.dtype == M.BF16 else torch.float32)
    t = {"xhat": torch.zeros(d.b, d.s, d.c, d.h, d.p, dtype=dt),
         "bhat": torch.zeros(d.b, d.s, d.c, d.h, d.r, dtype=dt),
         "da": torch.zeros(d.b, d.s, d.h, dtype=dt),
         "rot": torch.zeros(d.b, d.s, d.h, d.rope_dim // 2, dtype=dt),
         "h0": torch.zeros(d.b, d.h, d.p, d.r, dtype=dt),
         "d_m2": torch.zeros(d.b, d.h, d.r, d.r), "d_m1": torch.zeros(d.b, d.h, d.p, d.r)}
    return t


def _call(kind, d, t):
    if kind == "fwd":
        return M.moments_fwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"])
    return M.moments_bwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], t["d_m2"], t["d_m1"])


@pytest.mark.parametrize("kind", ["fwd", "bwd"])
@pytest.mark.parametrize("bad,match", [
    (dict(xhat=(2, 64, 2, 3, 9)), "xhat has shape"),
    (dict(bhat=(2, 64, 2, 3, 8)), "bhat has shape"),
    (dict(da=(2, 64, 1)), "da has shape"),
    (dict(rot=(2, 64, 3, 3)), "rot has shape"),
    (dict(h0=(2, 3, 8)), "h0 has shape"),
])
def test_binding_rejects_mismatched_shapes(kind, bad, match):
    """Every tensor is checked against the descriptor before the C ABI is called:
    a mismatched buffer would make the kernels read or write out of bounds."""
    import torch
    d = _desc()
    t = _tensors(d)
    for k, shape in bad.items():
        t[k] = torch.zeros(shape, dtype=t[k].dtype)
    with pytest.raises(ValueError, match=match):
        _call(kind, d, t)


def test_binding_rejects_dtypes_devices_and_pooled_cotangent():
    import torch
    d = _desc(dtype=M.BF16)
    t = _tensors(d, dtype=torch.float32)          # fp32 tensors with a bf16 descriptor
    with pytest.raises(ValueError, match="dtype"):
        _call("fwd", d, t)
    t = _tensors(d)
    t["d_m1"] = torch.zeros(d.b, d.h, d.r)        # the pages' pooled [b,h,r] cotangent
    with pytest.raises(ValueError, match="d_m1 has shape"):
        _call("bwd", d, t)
    t = _tensors(d)
    t["d_m2"] = t["d_m2"].to(torch.float64)
    with pytest.raises(ValueError, match="d_m2 has dtype"):
        _call("bwd", d, t)
    t = _tensors(d)
    t["rot"] = t["rot"].transpose(0, 1).contiguous().transpose(0, 1)   # right shape, not contiguous
    with pytest.raises(ValueError, match="contiguous"):
        _call("fwd", d, t)
    dn = _desc(rot_kind=M.ROT_NONE, rope_dim=0)
    t = _tensors(dn)
    t["rot"] = torch.zeros(2, 64, 3, 1)
    with pytest.raises(ValueError, match="no rotation"):
        _call("fwd", dn, t)
    t = _tensors(d)                                # everything right, but on the host
    with pytest.raises(ValueError, match="GPU"):
        _call("bwd", d, t)


# ---------------------------------------------------------------- rotation-sequence producer
@pytest.mark.parametrize("kw,code", [
    (dict(rot_kind=M.ROT_PAIRWISE, rope_dim=8), 0),
    (dict(rot_kind=M.ROT_HALF, rope_dim=8), 0),
    (dict(rot_kind=M.ROT_QUAT, rope_dim=0, quat_blocks=3), 0),
    (dict(rot_kind=M.ROT_NONE, rope_dim=0), -1),
    (dict(rot_kind=M.ROT_PAIRWISE, rope_dim=7), -1),
    (dict(rot_kind=M.ROT_PAIRWISE, rope_dim=0), -1),
    (dict(rot_kind=M.ROT_QUAT, rope_dim=0, quat_blocks=0), -1),
    (dict(dtype=5), -1),
    (dict(s=-1), -1),
    (dict(b=70000), -2),
    (dict(r=4096, rope_dim=2000, p=0, c=99, chunk_len=0), 0),   # fields the producer does not read
])
def test_rot_workspace_and_validation(kw, code):
    n = _lib.load().moments_rot_workspace_size(ctypes.byref(_desc(**kw)), 1)
    if code == 0:
        assert n > 0
    else:
        assert n == code


def test_rot_workspace_sizes():
    lib = _lib.load()
    q = _desc(rot_kind=M.ROT_QUAT, rope_dim=0, quat_blocks=3)
    fwd = lib.moments_rot_workspace_size(ctypes.byref(q), 0)
    bwd = lib.moments_rot_workspace_size(ctypes.byref(q), 1)
    assert 0 < fwd < bwd   # the quaternion VJP keeps a second per-segment array
    a = _desc()
    assert lib.moments_rot_workspace_size(ctypes.byref(a), 0) == lib.moments_rot_workspace_size(ctypes.byref(a), 1)
    assert lib.moments_rot_workspace_size(ctypes.byref(_desc(s=0)), 1) == 0


def test_rot_errors_without_gpu():
    lib = _lib.load()
    d = _desc()
    null = ctypes.c_void_p()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    assert lib.moments_rot_fwd(ctypes.byref(d), null, fake, fake, 1 << 40, null) == _lib.EINVAL
    assert lib.moments_rot_bwd(ctypes.byref(d), fake, null, fake, fake, 1 << 40, null) == _lib.EINVAL
    assert lib.moments_rot_fwd(ctypes.byref(d), fake, fake, fake, 16, null) == _lib.EWORKSPACE
    misaligned = ctypes.c_void_p((1 << 20) + 8)
    assert lib.moments_rot_fwd(ctypes.byref(d), misaligned, fake, fake, 1 << 40, null) == _lib.EINVAL
    # empty shapes launch nothing and accept NULL pointers
    assert lib.moments_rot_fwd(ctypes.byref(_desc(s=0)), null, null, null, 0, null) == 0
    assert lib.moments_rot_bwd(ctypes.byref(_desc(b=0)), null, null, null, null, 0, null) == 0


def test_rot_binding_rejects_shapes():
    import torch
    inc = torch.zeros(2, 16, 3, 4)
    d = M.rot_desc(inc, M.ROT_PAIRWISE)
    assert (d.b, d.s, d.h, d.rope_dim) == (2, 16, 3, 8)
    with pytest.raises(ValueError, match="inc has shape"):
        M.moments_rot_fwd(d, torch.zeros(2, 16, 3, 5))
    with pytest.raises(ValueError, match="d_rot has shape"):
        M.moments_rot_bwd(d, inc, torch.zeros(2, 16, 3))
    with pytest.raises(ValueError, match="GPU"):
        M.moments_rot_fwd(d, inc)


# ---------------------------------------------------------------- saved-carry variant
def test_saved_size_and_errors_without_gpu():
    lib = _lib.load()
    d = _desc()
    n = M.moments_saved_size(d)
    # fp32 states entering each 32-token kernel chunk, then the chunk decays
    ell = M.kernel_chunk_len()
    nk = -(-min(d.valid_len, d.s) // ell)
    states = d.b * d.h * nk * d.p * d.r * 4
    assert n == (states + 255) // 256 * 256 + (d.b * d.h * nk * 4 + 255) // 256 * 256
    assert M.moments_saved_size(_desc(valid_len=0)) == 0
    with pytest.raises(M.MomentsError):
        M.moments_saved_size(_desc(p=0))
    null = ctypes.c_void_p()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    big = 1 << 40
    rc = lib.moments_fwd_save(ctypes.byref(d), fake, fake, fake, fake, null, fake, fake, null, big, fake, big, null)
    assert rc == _lib.EINVAL           # NULL saved buffer
    rc = lib.moments_fwd_save(ctypes.byref(d), fake, fake, fake, fake, null, fake, fake, fake, 16, fake, big, null)
    assert rc == _lib.EWORKSPACE       # saved buffer too small
    args = [fake] * 5 + [null, big] + [fake] * 7 + [fake, big, null]
    rc = lib.moments_bwd_saved(ctypes.byref(d), *args)
    assert rc == _lib.EINVAL
    args = [fake] * 5 + [fake, 16] + [fake] * 7 + [fake, big, null]
    rc = lib.moments_bwd_saved(ctypes.byref(d), *args)
    assert rc == _lib.EWORKSPACE
