"""The allocation-free forward (moments_fwd_static, static device scratch)
against moments_fwd (caller workspace) through the C ABI: two calls in a row,
the second on a smaller problem, each bitwise equal to the workspace path; a
problem beyond the scratch is rejected before anything is launched."""
import ctypes

import pytest
import torch

import mamba_ssm_chunkwise_amd as M
import workloads as W
from mamba_ssm_chunkwise_amd import _lib
from parity_util import desc_of

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # bf16, transposed kernels, several workgroups per chain (carry pass + partial moments)
    W.small("static_bf16", dtype="bf16", b=2, h=4, s=512, c=2, p=32, r=128, chunk_len=64, valid_len=500,
            rot_kind=W.ROT_PAIRWISE, rope_dim=64, seed=31, angle_step=0.05, da_mu=-1.0),
    # smaller, float32, general kernels
    W.small("static_f32", dtype="f32", b=1, h=3, s=96, c=2, p=24, r=40, chunk_len=16, valid_len=77,
            rot_kind=W.ROT_QUAT, rope_dim=0, quat_blocks=6, seed=32),
]


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _static_call(w, t, m2, m1):
    d = desc_of(w)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return _lib.load().moments_fwd_static(ctypes.byref(d), _ptr(t["xhat"]), _ptr(t["bhat"]), _ptr(t["da"]),
                                          _ptr(t["rot"]), _ptr(t["h0"]), _ptr(m2), _ptr(m1), st)


def test_static_forward_matches_workspace_forward():
    for w in CASES:
        print(f"[static] {w}", flush=True)
        assert M.moments_workspace_size(desc_of(w), False) <= _lib.STATIC_SCRATCH_BYTES
        t = {k: (None if v is None else v.to(DEV)) for k, v in W.generate(w, device="cpu").items()}
        ref2, ref1 = M.moments_fwd(desc_of(w), t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"])
        m2 = torch.full((w.b, w.h, w.r, w.r), float("nan"), device=DEV)
        m1 = torch.full((w.b, w.h, w.p, w.r), float("nan"), device=DEV)
        assert _static_call(w, t, m2, m1) == 0
        torch.cuda.synchronize()
        assert torch.equal(m2, ref2) and torch.equal(m1, ref1), w.name


def test_static_forward_rejects_problems_beyond_the_scratch():
    w = W.BF16_PAIRWISE          # its forward workspace is gigabytes
    assert M.moments_workspace_size(desc_of(w), False) > _lib.STATIC_SCRATCH_BYTES
    d = desc_of(w)
    fake = ctypes.c_void_p(1 << 20)   # never dereferenced: the size check comes first
    rc = _lib.load().moments_fwd_static(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake,
                                        ctypes.c_void_p())
    assert rc == _lib.ESCRATCH
