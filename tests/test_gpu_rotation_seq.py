"""GPU parity of the rotation-sequence producer and its VJP (moments_rot_fwd /
moments_rot_bwd through the C ABI) against the CPU oracle (oracle/rotation_seq.py).

Same bar as the moments path: normwise and max-elementwise error (over the
largest reference magnitude) at most 1e-4 for float32, 2e-2 for bfloat16, and a
per-token bound. Shapes cover one token, exactly one and just over one segment
of the kernels' walk, ragged tails, non-unit quaternion increments, and the
four workloads that carry a rotation at full size (the long-context one on
three sampled heads; chains are independent).
"""
import sys

import numpy as np
import pytest
import torch

import mamba_ssm_chunkwise_amd as M
import workloads as W
from oracle import oracle_bwd
from oracle import rotation_seq as rs
from parity_util import TOL, max_err, rel_err, token_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np64(x):
    return x.detach().double().cpu().numpy()


def _check(name, got, ref, tol):
    g = _np64(got)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    e, m, t = rel_err(g, ref), max_err(g, ref), token_err(g, ref)
    _log(f"[compare] {name}: normwise {e:.2e} max-elementwise {m:.2e} per-token {t:.2e}")
    assert e <= tol and m <= tol and t <= tol, f"{name}: {e:.2e}/{m:.2e}/{t:.2e} above {tol:.1e}"


def _oracle(rot_kind, inc, d_rot):
    if rot_kind == W.ROT_QUAT:
        return rs.quat_prefix(inc), rs.quat_prefix_vjp(inc, d_rot)
    return rs.angle_cumsum(inc), rs.angle_cumsum_vjp(d_rot)


def _run(w, inc, d_rot):
    d = M.rot_desc(inc, w.rot_kind)
    rot = M.moments_rot_fwd(d, inc)
    d_inc = M.moments_rot_bwd(d, inc, d_rot)
    torch.cuda.synchronize()
    return rot, d_inc


SMALL = []
for dtype in ("f32", "bf16"):
    for s in (1, 16, 17, 77, 300):
        SMALL.append((W.ROT_PAIRWISE, dtype, s))
        SMALL.append((W.ROT_QUAT, dtype, s))


@pytest.mark.parametrize("rot_kind,dtype,s", SMALL)
def test_small(rot_kind, dtype, s):
    w = W.small(f"rot_{rot_kind}_{dtype}_{s}", dtype=dtype, b=2, s=s, h=3, r=16, rot_kind=rot_kind,
                rope_dim=10 if rot_kind == W.ROT_PAIRWISE else 0,
                quat_blocks=3 if rot_kind == W.ROT_QUAT else 0, angle_step=0.3, quat_sd=0.3, seed=21 + s)
    _log(f"[case] {w.name}")
    inc, d_rot = W.rotation_increments(w, DEV, scale=(0.5, 1.7))
    rot, d_inc = _run(w, inc, d_rot)
    ref_rot, ref_inc = _oracle(rot_kind, _np64(inc), _np64(d_rot))
    _check(w.name + " rot", rot, ref_rot, TOL[dtype])
    _check(w.name + " d_inc", d_inc, ref_inc, TOL[dtype])
    if rot_kind == W.ROT_QUAT:
        # rescaling an increment leaves the product unchanged
        dots = (d_inc.double() * inc.double()).sum(-1).abs().max().item()
        assert dots <= TOL[dtype] * d_inc.double().abs().max().item() * 4


def test_empty_and_errors():
    w = W.small("rot_empty", b=1, s=8, h=2, r=8, rot_kind=W.ROT_QUAT, rope_dim=0, quat_blocks=2)
    inc = torch.zeros(1, 0, 2, 2, 4, device=DEV)
    d = M.rot_desc(inc, W.ROT_QUAT)
    assert M.moments_rot_workspace_size(d, True) == 0
    M.moments_rot_fwd(d, inc)
    inc, _ = W.rotation_increments(w, DEV)
    bad = M.rot_desc(inc, W.ROT_NONE)
    with pytest.raises(ValueError):
        M.moments_rot_fwd(bad, inc)


@pytest.mark.parametrize("rot_kind", [W.ROT_PAIRWISE, W.ROT_QUAT])
def test_chained_with_moments_backward(rot_kind):
    """Increments -> producer -> moments forward/backward -> producer VJP, on the
    GPU, against the same chain on the oracle."""
    w = W.small(f"rot_chain_{rot_kind}", dtype="f32", b=2, s=96, c=2, h=3, p=24, r=40, valid_len=77,
                rot_kind=rot_kind, rope_dim=16 if rot_kind == W.ROT_PAIRWISE else 0,
                quat_blocks=6 if rot_kind == W.ROT_QUAT else 0, angle_step=0.3, quat_sd=0.3, seed=31)
    _log(f"[case] {w.name}")
    t = W.generate(w, device=DEV, increments=True)
    inc = t["rot_inc"]
    rd = M.rot_desc(inc, rot_kind)
    rot = M.moments_rot_fwd(rd, inc)
    from parity_util import desc_of
    g = M.moments_bwd(desc_of(w), t["xhat"], t["bhat"], t["da"], rot, t["h0"], t["d_m2"], t["d_m1"],
                      want=("rot",))
    d_inc = M.moments_rot_bwd(rd, inc, g["d_rot"])
    torch.cuda.synchronize()
    a = {k: (None if v is None else _np64(v)) for k, v in t.items()}
    rot_o = rs.quat_prefix(a["rot_inc"]) if rot_kind == W.ROT_QUAT else rs.angle_cumsum(a["rot_inc"])
    go = oracle_bwd(a["xhat"], a["bhat"], a["da"], rot_o, a["h0"], a["d_m2"], a["d_m1"], w.valid_len,
                    rot_kind, w.rope_dim)
    ref = (rs.quat_prefix_vjp(a["rot_inc"], go["d_rot"]) if rot_kind == W.ROT_QUAT
           else rs.angle_cumsum_vjp(go["d_rot"]))
    _check(w.name + " d_inc", d_inc, ref, TOL["f32"])


FULL = [W.F32_HALFSPLIT, W.BF16_QUAT, W.BF16_PAIRWISE, W.BF16_QUAT_LONG]


@pytest.mark.parametrize("w", FULL, ids=[w.name for w in FULL])
def test_workload(w):
    _log(f"[case] {w.name} full size")
    inc, d_rot = W.rotation_increments(w, DEV)
    rot, d_inc = _run(w, inc, d_rot)
    heads = [0, w.h // 2, w.h - 1] if w.s * w.h * max(w.quat_blocks, 1) > 10 ** 7 and w.rot_kind == W.ROT_QUAT \
        else list(range(w.h))
    a_inc, a_d = _np64(inc[:, :, heads]), _np64(d_rot[:, :, heads])
    ref_rot, ref_inc = _oracle(w.rot_kind, a_inc, a_d)
    _check(w.name + " rot", rot[:, :, heads], ref_rot, TOL[w.dtype])
    _check(w.name + " d_inc", d_inc[:, :, heads], ref_inc, TOL[w.dtype])
