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
