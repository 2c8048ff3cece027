"""ctypes binding of libmoments.so (argument marshalling only).

Every step of the computation runs in the HIP kernels; this module only builds
the descriptor, allocates the workspace with torch and passes device pointers
and torch's current HIP stream. It fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_build", "libmoments.so")

OK, EINVAL, ENOTSUP, EWORKSPACE, EHIP, ESCRATCH, ENONFINITE = 0, -1, -2, -3, -4, -5, -6
STATIC_SCRATCH_BYTES = 64 << 20
F32, BF16 = 0, 1
ROT_NONE, ROT_PAIRWISE, ROT_HALF, ROT_QUAT = 0, 1, 2, 3

EXPORTS = ("moments_validate", "moments_workspace_size", "moments_fwd", "moments_fwd_static", "moments_bwd",
           "moments_strerror", "moments_last_hip_error", "moments_kernel_chunk_len",
           "moments_profile_enable", "moments_profile_read", "moments_profile_reset",
           "moments_rot_workspace_size", "moments_rot_fwd", "moments_rot_bwd",
           "moments_saved_size", "moments_fwd_save", "moments_bwd_saved")


class Desc(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("s", ctypes.c_int64), ("c", ctypes.c_int64),
                ("h", ctypes.c_int64), ("p", ctypes.c_int64), ("r", ctypes.c_int64),
                ("chunk_len", ctypes.c_int64), ("valid_len", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("rot_kind", ctypes.c_int32),
                ("rope_dim", ctypes.c_int64), ("quat_blocks", ctypes.c_int64),
                ("valid_lens", ctypes.c_void_p)]


class MomentsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_lib = None


def load():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mamba_ssm_chunkwise_amd.build` (no CPU fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        dp = ctypes.POINTER(Desc)
        lib.moments_validate.argtypes = [dp]
        lib.moments_validate.restype = ctypes.c_int
        lib.moments_workspace_size.argtypes = [dp, ctypes.c_int]
        lib.moments_workspace_size.restype = ctypes.c_int64
        lib.moments_fwd.argtypes = [dp] + [vp] * 7 + [vp, ctypes.c_size_t, vp]
        lib.moments_fwd.restype = ctypes.c_int
        lib.moments_fwd_static.argtypes = [dp] + [vp] * 7 + [vp]
        lib.moments_fwd_static.restype = ctypes.c_int
        lib.moments_bwd.argtypes = [dp] + [vp] * 12 + [vp, ctypes.c_size_t, vp]
        lib.moments_bwd.restype = ctypes.c_int
        lib.moments_saved_size.argtypes = [dp]
        lib.moments_saved_size.restype = ctypes.c_int64
        lib.moments_fwd_save.argtypes = [dp] + [vp] * 7 + [vp, ctypes.c_size_t, vp, ctypes.c_size_t, vp]
        lib.moments_fwd_save.restype = ctypes.c_int
        lib.moments_bwd_saved.argtypes = [dp] + [vp] * 5 + [vp, ctypes.c_size_t] + [vp] * 7 + [vp, ctypes.c_size_t, vp]
        lib.moments_bwd_saved.restype = ctypes.c_int
        lib.moments_rot_workspace_size.argtypes = [dp, ctypes.c_int]
        lib.moments_rot_workspace_size.restype = ctypes.c_int64
        lib.moments_rot_fwd.argtypes = [dp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.moments_rot_fwd.restype = ctypes.c_int
        lib.moments_rot_bwd.argtypes = [dp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.moments_rot_bwd.restype = ctypes.c_int
        lib.moments_strerror.argtypes = [ctypes.c_int]
        lib.moments_strerror.restype = ctypes.c_char_p
        lib.moments_last_hip_error.argtypes = []
        lib.moments_last_hip_error.restype = ctypes.c_int
        lib.moments_kernel_chunk_len.argtypes = []
        lib.moments_kernel_chunk_len.restype = ctypes.c_int64
        lib.moments_profile_enable.argtypes = [ctypes.c_int]
        lib.moments_profile_enable.restype = ctypes.c_int
        lib.moments_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                             ctypes.POINTER(ctypes.c_int64),
                                             ctypes.POINTER(ctypes.c_double)]
        lib.moments_profile_read.restype = ctypes.c_int
        lib.moments_profile_reset.argtypes = []
        lib.moments_profile_reset.restype = None
        _lib = lib
    return _lib


def check(code):
    if code != OK:
        lib = load()
        msg = lib.moments_strerror(code).decode()
        if code == EHIP:
            msg += f" [hipError {lib.moments_last_hip_error()}]"
        raise MomentsError(code, msg)
    return code
