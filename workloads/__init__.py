"""Seeded synthetic workloads for the state-moments path.

This module only draws inputs. It holds none of the moments arithmetic and is
the one thing the CPU oracle and the HIP path share. Every tensor is drawn with
a ``torch.Generator`` seeded per workload, in a fixed order:
xhat, bhat, da, rotation increments, h0, d_m2, d_m1.

The rotation input is cumulative, as the pages' ``RotPrim`` takes it (cumulative
angles ``[b,s,h,a]`` or cumulative unit quaternions ``[b,s,h,J,4]``, (w,x,y,z)):

* angles: inclusive cumsum over the sequence of i.i.d. U(-w, w) increments,
  summed in float64 and then cast;
* quaternions: per-token increments from an axis-angle vector v ~ N(0, sd^2)^3,
  q = (cos(|v|/2), sin(|v|/2) v/|v|), composed left to right
  (Q_t = Q_{t-1} * q_t) by a doubling prefix product in float64 with
  renormalisation after every doubling step, then cast.

The composition here only prepares the cumulative input of the moments path
(a doubling product in float64, an algorithm neither implementation uses). The
rotation-sequence producer, which composes increments itself, is tested on the
raw increments (``generate(..., increments=True)["rot_inc"]``), never on this
composition.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

ROT_NONE, ROT_PAIRWISE, ROT_HALF, ROT_QUAT = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" | "bf16"
    b: int
    s: int
    c: int
    h: int
    p: int
    r: int
    chunk_len: int
    valid_len: int
    rot_kind: int
    rope_dim: int = 0     # complex modes: rotated coordinates (even); a = rope_dim // 2 angles
    quat_blocks: int = 0  # quaternion mode: J
    angle_step: float = 0.05   # increments U(-angle_step, angle_step)
    quat_sd: float = 0.05      # axis-angle standard deviation
    da_mu: float = -1.0        # da = -softplus(N(da_mu, 1)) + da_shift
    da_shift: float = 0.0
    h0_sd: Optional[float] = 0.1  # None -> h0 is absent (zero initial state)
    seed: int = 1000

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def rot_width(self) -> int:
        if self.rot_kind in (ROT_PAIRWISE, ROT_HALF):
            return self.rope_dim // 2
        if self.rot_kind == ROT_QUAT:
            return 4 * self.quat_blocks
        return 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the benchmark definition, named by what they are.
TINY_F32_PAIRWISE = Workload("tiny_f32_pairwise_s64", "f32", b=1, s=64, c=1, h=2, p=8, r=8,
                             chunk_len=16, valid_len=64, rot_kind=ROT_PAIRWISE, rope_dim=8,
                             angle_step=0.1, da_mu=0.0, h0_sd=0.1, seed=1000)
F32_HALFSPLIT = Workload("f32_halfsplit_b2_s2048", "f32", b=2, s=2048, c=2, h=16, p=64, r=64,
                         chunk_len=64, valid_len=1900, rot_kind=ROT_HALF, rope_dim=32,
                         angle_step=0.05, da_mu=-1.0, h0_sd=None, seed=1001)
BF16_QUAT = Workload("bf16_quat_b4_s4096", "bf16", b=4, s=4096, c=1, h=32, p=64, r=128,
                     chunk_len=64, valid_len=4096, rot_kind=ROT_QUAT, quat_blocks=8,
                     quat_sd=0.05, da_mu=-1.0, h0_sd=0.1, seed=1002)
BF16_PAIRWISE = Workload("bf16_pairwise_b8_s8192", "bf16", b=8, s=8192, c=2, h=64, p=64, r=128,
                         chunk_len=128, valid_len=8192, rot_kind=ROT_PAIRWISE, rope_dim=64,
                         angle_step=0.05, da_mu=-1.0, h0_sd=0.1, seed=1003)
BF16_QUAT_LONG = Workload("bf16_quat_long_s65536", "bf16", b=1, s=65536, c=4, h=32, p=128, r=128,
                          chunk_len=128, valid_len=60000, rot_kind=ROT_QUAT, quat_blocks=32,
                          quat_sd=0.05, da_mu=-2.0, h0_sd=0.1, seed=1004)

ALL = (TINY_F32_PAIRWISE, F32_HALFSPLIT, BF16_QUAT, BF16_PAIRWISE, BF16_QUAT_LONG)
BY_NAME = {w.name: w for w in ALL}


def _quat_prefix(q: torch.Tensor, dim: int) -> torch.Tensor:
    """Inclusive left-to-right prefix product of quaternions along ``dim``
    (float64, doubling steps, renormalised after each step)."""
    q = q.movedim(dim, 0).contiguous()
    n = q.shape[0]
    k = 1
    while k < n:
        a, b = q[:-k], q[k:]
        aw, ax, ay, az = a.unbind(-1)
        bw, bx, by, bz = b.unbind(-1)
        prod = torch.stack([
            aw * bw - ax * bx - ay * by - az * bz,
            aw * bx + ax * bw + ay * bz - az * by,
            aw * by - ax * bz + ay * bw + az * bx,
            aw * bz + ax * by - ay * bx + az * bw,
        ], dim=-1)
        q = torch.cat([q[:k], prod], dim=0)
        q = q / q.norm(dim=-1, keepdim=True)
        k *= 2
    return q.movedim(0, dim)


def generate(w: Workload, device="cpu", with_cotangents=True, increments=False):
    """Draw one workload. Returns a dict of tensors on ``device`` in the workload's
    dtype (d_m2, d_m1 are float32): xhat[b,s,c,h,p], bhat[b,s,c,h,r], da[b,s,h],
    rot ([b,s,h,a] | [b,s,h,J,4] | None), h0[b,h,p,r] | None, d_m2[b,h,r,r],
    d_m1[b,h,p,r]. With ``increments`` it also returns the per-token rotation
    increments the cumulative ``rot`` was composed from, cast to the workload's
    dtype, as ``rot_inc`` (same shape as ``rot``; None without a rotation)."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    f32 = dict(device=device, dtype=torch.float32, generator=g)
    dt = w.torch_dtype
    out = {}
    inv = 1.0 / math.sqrt(w.r)
    out["xhat"] = (torch.randn(w.b, w.s, w.c, w.h, w.p, **f32) * inv).to(dt)
    out["bhat"] = (torch.randn(w.b, w.s, w.c, w.h, w.r, **f32) * inv).to(dt)
    out["da"] = (w.da_shift - torch.nn.functional.softplus(torch.randn(w.b, w.s, w.h, **f32) + w.da_mu)).to(dt)
    if w.rot_kind in (ROT_PAIRWISE, ROT_HALF):
        a = w.rope_dim // 2
        inc = (torch.rand(w.b, w.s, w.h, a, **f32) * 2.0 - 1.0) * w.angle_step
        out["rot"] = torch.cumsum(inc.double(), dim=1).to(dt)
        if increments:
            out["rot_inc"] = inc.to(dt)
    elif w.rot_kind == ROT_QUAT:
        v = torch.randn(w.b, w.s, w.h, w.quat_blocks, 3, **f32).double() * w.quat_sd
        phi = v.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        q = torch.cat([torch.cos(phi / 2), torch.sin(phi / 2) * v / phi], dim=-1)
        out["rot"] = _quat_prefix(q, dim=1).to(dt).contiguous()
        if increments:
            out["rot_inc"] = q.to(dt).contiguous()
    else:
        out["rot"] = None
        if increments:
            out["rot_inc"] = None
    if w.h0_sd is None:
        out["h0"] = None
    else:
        out["h0"] = (torch.randn(w.b, w.h, w.p, w.r, **f32) * w.h0_sd).to(dt)
    if with_cotangents:
        out["d_m2"] = torch.randn(w.b, w.h, w.r, w.r, **f32)
        out["d_m1"] = torch.randn(w.b, w.h, w.p, w.r, **f32)
    return out


def rotation_increments(w: Workload, device="cpu", scale=None):
    """Per-token rotation increments alone, for the rotation-sequence producer:
    the distribution ``generate`` composes (U(-angle_step, angle_step) angles, or
    unit quaternions from N(0, quat_sd^2)^3 axis-angle vectors), drawn from a
    stream of their own (seed + 7919), cast to the workload's dtype, and a
    cotangent N(0, 1) of the same shape. ``scale`` = (lo, hi) multiplies each
    quaternion by U(lo, hi) (non-unit increments). Returns (inc, d_rot)."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed + 7919)
    f32 = dict(device=device, dtype=torch.float32, generator=g)
    dt = w.torch_dtype
    if w.rot_kind in (ROT_PAIRWISE, ROT_HALF):
        inc = (torch.rand(w.b, w.s, w.h, w.rope_dim // 2, **f32) * 2.0 - 1.0) * w.angle_step
    elif w.rot_kind == ROT_QUAT:
        v = torch.randn(w.b, w.s, w.h, w.quat_blocks, 3, **f32).double() * w.quat_sd
        phi = v.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        inc = torch.cat([torch.cos(phi / 2), torch.sin(phi / 2) * v / phi], dim=-1)
        if scale is not None:
            lo, hi = scale
            inc = inc * (lo + (hi - lo) * torch.rand(inc.shape[:-1] + (1,), **f32).double())
    else:
        raise ValueError("the workload has no rotation")
    d_rot = torch.randn(inc.shape, **f32)
    return inc.to(dt).contiguous(), d_rot.to(dt).contiguous()


def small(name, dtype="f32", b=1, s=48, c=2, h=2, p=24, r=40, chunk_len=16, valid_len=None,
          rot_kind=ROT_PAIRWISE, rope_dim=16, quat_blocks=0, seed=7, h0_sd=0.1, da_mu=-0.5,
          angle_step=0.3, quat_sd=0.3, da_shift=0.0):
    """A small workload for tests (odd sizes, ragged tails)."""
    return Workload(name, dtype, b=b, s=s, c=c, h=h, p=p, r=r, chunk_len=chunk_len,
                    valid_len=s if valid_len is None else valid_len, rot_kind=rot_kind,
                    rope_dim=rope_dim, quat_blocks=quat_blocks, angle_step=angle_step,
                    quat_sd=quat_sd, da_mu=da_mu, da_shift=da_shift, h0_sd=h0_sd, seed=seed)
