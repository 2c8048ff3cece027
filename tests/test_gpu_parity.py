"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances (normwise, per output tensor, A10 reading): 1e-4 for float32 inputs,
2e-2 for bfloat16 inputs with float32 accumulation; gradients past valid_len
must be exactly zero.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from parity_util import (compare, gpu_run, oracle_run, select_chains, sub_chains)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _small(rot_kind, dtype, **kw):
    base = dict(b=2, s=96, c=2, h=3, p=24, r=40, chunk_len=16, valid_len=77, seed=11,
                angle_step=0.3, quat_sd=0.3)
    if rot_kind in (W.ROT_PAIRWISE, W.ROT_HALF):
        base["rope_dim"] = 16
    if rot_kind == W.ROT_QUAT:
        base["quat_blocks"] = 6
    base.update(kw)
    return W.small(f"small_{rot_kind}_{dtype}", dtype=dtype, rot_kind=rot_kind, **base)


SMALL = [
    (W.ROT_PAIRWISE, "f32", {}),
    (W.ROT_HALF, "f32", {}),
    (W.ROT_QUAT, "f32", {}),
    (W.ROT_NONE, "f32", {}),
    (W.ROT_PAIRWISE, "bf16", {}),
    (W.ROT_HALF, "bf16", {}),
    (W.ROT_QUAT, "bf16", {}),
    (W.ROT_PAIRWISE, "f32", dict(c=1, p=5, r=8, rope_dim=8, s=64, valid_len=64)),
    (W.ROT_QUAT, "f32", dict(c=3, p=17, r=60, quat_blocks=15, s=160, chunk_len=32, valid_len=130)),
    (W.ROT_HALF, "bf16", dict(c=4, p=33, r=128, rope_dim=64, s=128, valid_len=100)),
    (W.ROT_PAIRWISE, "f32", dict(h0_sd=None, valid_len=33)),
    (W.ROT_PAIRWISE, "f32", dict(valid_len=31)),   # a single partial chunk
    (W.ROT_QUAT, "bf16", dict(valid_len=96, p=64, r=128, quat_blocks=32, c=4)),
    # one channel; state rows crossing the 32-row blocks of the bf16 backward
    (W.ROT_QUAT, "bf16", dict(c=1, p=40, r=128, quat_blocks=8, valid_len=96)),
    (W.ROT_PAIRWISE, "bf16", dict(c=1, p=40, r=128, rope_dim=64, valid_len=90)),
    (W.ROT_NONE, "bf16", dict(c=1, p=37, r=64, valid_len=96)),
    (W.ROT_PAIRWISE, "bf16", dict(c=2, p=70, r=128, rope_dim=64, valid_len=96)),
    (W.ROT_QUAT, "bf16", dict(c=2, p=33, r=128, quat_blocks=32, valid_len=70)),
    # 128 state rows: 32 rounds of the transposed kernels (second m1 tile of the forward)
    (W.ROT_PAIRWISE, "bf16", dict(c=2, p=128, r=128, rope_dim=64, valid_len=96)),
    # rows that allow 16-byte staging except for the rotation input: an odd number
    # of angles, an odd number of quaternion blocks (element-wise staging)
    (W.ROT_PAIRWISE, "bf16", dict(c=2, p=16, r=32, rope_dim=6, valid_len=90)),
    (W.ROT_QUAT, "bf16", dict(c=1, p=16, r=32, quat_blocks=3, valid_len=96)),
    # half-split with 16-byte staging: caller columns scattered to the interleaved order
    (W.ROT_HALF, "bf16", dict(c=2, p=32, r=128, rope_dim=64, valid_len=96)),
    # bf16 without an initial state (h0 = NULL), general and transposed kernels
    (W.ROT_PAIRWISE, "bf16", dict(h0_sd=None)),
    (W.ROT_PAIRWISE, "bf16", dict(c=2, p=64, r=128, rope_dim=64, valid_len=96, h0_sd=None)),
    (W.ROT_QUAT, "bf16", dict(c=1, p=64, r=128, quat_blocks=8, valid_len=96, h0_sd=None)),
    # positive decay increments (da mostly > 0: the states grow along the chunk)
    (W.ROT_PAIRWISE, "f32", dict(da_mu=-4.0, da_shift=0.06)),
    (W.ROT_HALF, "bf16", dict(c=2, p=64, r=128, rope_dim=64, valid_len=96, da_mu=-4.0, da_shift=0.06)),
    (W.ROT_QUAT, "bf16", dict(c=4, p=33, r=128, quat_blocks=32, valid_len=100, da_mu=-4.0, da_shift=0.04)),
    # four channels (backward over token pairs): rotation rows that are not a
    # multiple of 16 bytes, no rotation, no initial state, a partial last chunk
    (W.ROT_PAIRWISE, "bf16", dict(c=4, p=16, r=32, rope_dim=6, valid_len=90)),
    (W.ROT_NONE, "bf16", dict(c=4, p=37, r=64, valid_len=95)),
    (W.ROT_QUAT, "bf16", dict(c=4, p=128, r=128, quat_blocks=32, valid_len=77, h0_sd=None)),
    # ... with fewer state rows than one round holds (rows 3..7 of the round idle)
    (W.ROT_PAIRWISE, "bf16", dict(c=4, p=3, r=24, rope_dim=8, valid_len=45)),
]


@pytest.mark.parametrize("rot_kind,dtype,kw", SMALL, ids=[f"{a}-{b}-{i}" for i, (a, b, _) in enumerate(SMALL)])
def test_small_parity(rot_kind, dtype, kw):
    w = _small(rot_kind, dtype, **kw)
    t = W.generate(w, device="cpu")
    _log(f"[small] {w}")
    gpu = gpu_run(w, {k: (None if v is None else v.to(DEV)) for k, v in t.items()})
    ref = oracle_run(w, t)
    errs = compare(w, gpu, ref)
    _log(f"[small] errors {errs}")


# Enough chunks that a workgroup walks several of them (2 or more chunks per
# group), with weak decay (the carry cotangent reaches back over whole groups)
# and strong decay (it vanishes after a chunk or two).
GROUPED = [
    (W.ROT_PAIRWISE, dict(b=2, h=8, s=4224, valid_len=4200, c=2, p=8, r=32, rope_dim=16, da_mu=-6.0)),
    (W.ROT_PAIRWISE, dict(b=2, h=8, s=4224, valid_len=4200, c=2, p=8, r=32, rope_dim=16, da_mu=2.5)),
    (W.ROT_QUAT, dict(b=2, h=8, s=4224, valid_len=4224, c=1, p=12, r=32, quat_blocks=4, da_mu=1.5)),
    (W.ROT_NONE, dict(b=3, h=6, s=4096, valid_len=4000, c=2, p=8, r=48, da_mu=1.0)),
    # 512 chains: one group per chain (the forward carries its state rows itself)
    (W.ROT_PAIRWISE, dict(b=8, h=64, s=256, valid_len=250, c=2, p=16, r=64, rope_dim=32, da_mu=-1.0)),
    (W.ROT_HALF, dict(b=8, h=64, s=256, valid_len=256, c=1, p=20, r=64, rope_dim=64, da_mu=0.5)),
    # ... with a partial last round of rows (p not a multiple of 4)
    (W.ROT_QUAT, dict(b=8, h=64, s=128, valid_len=120, c=2, p=18, r=64, quat_blocks=16, da_mu=-0.5)),
    # four channels: the token-pair walk over several groups (group fix-up on pair tokens)
    (W.ROT_QUAT, dict(b=1, h=4, s=2048, valid_len=2000, c=4, p=16, r=32, quat_blocks=8, da_mu=1.5)),
]


@pytest.mark.parametrize("rot_kind,kw", GROUPED, ids=[f"{a}-{i}" for i, (a, _) in enumerate(GROUPED)])
def test_grouped_walk_parity(rot_kind, kw):
    base = dict(chunk_len=32, seed=21, angle_step=0.05, quat_sd=0.05)
    base.update(kw)
    w = W.small(f"grouped_{rot_kind}", dtype="bf16", rot_kind=rot_kind, **base)
    t = W.generate(w, device="cpu")
    _log(f"[grouped] {w}")
    gpu = gpu_run(w, {k: (None if v is None else v.to(DEV)) for k, v in t.items()})
    ref = oracle_run(w, t)
    errs = compare(w, gpu, ref)
    _log(f"[grouped] errors {errs}")


@pytest.mark.parametrize("valid_len", [0, 1, 96, 500])
def test_valid_len_edges(valid_len):
    w = _small(W.ROT_PAIRWISE, "f32", valid_len=valid_len)
    t = W.generate(w, device="cpu")
    gpu = gpu_run(w, {k: (None if v is None else v.to(DEV)) for k, v in t.items()})
    ref = oracle_run(w, t)
    if valid_len == 0:
        for k, v in gpu.items():
            if v is not None:
                assert torch.count_nonzero(v).item() == 0, k
    else:
        compare(w, gpu, ref)


def test_inputs_past_valid_len_are_never_read():
    """NaN past valid_len changes nothing, bit for bit (chunk_mask; skipped chunks)."""
    w = _small(W.ROT_QUAT, "f32", valid_len=45)
    t = {k: (None if v is None else v.to(DEV)) for k, v in W.generate(w, device="cpu").items()}
    a = gpu_run(w, t)
    u = dict(t)
    for k in ("xhat", "bhat", "da", "rot"):
        u[k] = t[k].clone()
        u[k][:, 45:] = float("nan")
    b = gpu_run(w, u)
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


def test_deterministic():
    w = _small(W.ROT_HALF, "bf16")
    t = {k: (None if v is None else v.to(DEV)) for k, v in W.generate(w, device="cpu").items()}
    a = gpu_run(w, t)
    b = gpu_run(w, t)
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


OPTIONAL = [
    ("f32", W.ROT_PAIRWISE, {}),
    # the transposed bf16 kernels (c <= 2, 128 state columns)
    ("bf16", W.ROT_PAIRWISE, dict(c=2, p=64, r=128, rope_dim=64, valid_len=96)),
    ("bf16", W.ROT_QUAT, dict(c=1, p=40, r=128, quat_blocks=8, valid_len=90)),
    # four channels (the transposed backward over odd pair tokens)
    ("bf16", W.ROT_HALF, dict(c=4, p=33, r=128, rope_dim=64, valid_len=100)),
]
WANTS = [("da", "h0"), ("xhat",), ("bhat", "rot"), ("rot",), ()]


@pytest.mark.parametrize("dtype,rot_kind,kw", OPTIONAL, ids=[f"{a}-{b}-{i}" for i, (a, b, _) in enumerate(OPTIONAL)])
def test_optional_gradients(dtype, rot_kind, kw):
    """NULL gradient pointers skip those gradients; the ones asked for are
    bitwise the same as in a full call."""
    import mamba_ssm_chunkwise_amd as M
    from parity_util import desc_of
    w = _small(rot_kind, dtype, **kw)
    t = {k: (None if v is None else v.to(DEV)) for k, v in W.generate(w, device="cpu").items()}
    full = gpu_run(w, t)
    _log(f"[optional] {w}")
    for want in WANTS:
        part = M.moments_bwd(desc_of(w), t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], t["d_m2"],
                             t["d_m1"], want=want)
        torch.cuda.synchronize()
        for k in ("xhat", "bhat", "da", "rot", "h0"):
            if k in want:
                assert torch.equal(part["d_" + k], full["d_" + k]), (want, k)
            else:
                assert part["d_" + k] is None, (want, k)


NONUNIT = [
    ("f32", dict(c=3, p=17, r=60, quat_blocks=15, s=160, chunk_len=32, valid_len=130)),
    ("bf16", dict(c=1, p=24, r=40, quat_blocks=6)),
    ("bf16", dict(c=2, p=64, r=128, quat_blocks=32, valid_len=96)),
    ("bf16", dict(c=4, p=33, r=128, quat_blocks=32, valid_len=100)),
]


@pytest.mark.parametrize("dtype,kw", NONUNIT, ids=[f"{a}-{i}" for i, (a, _) in enumerate(NONUNIT)])
def test_nonunit_quaternions(dtype, kw):
    """Quaternions scaled off the unit sphere by U(0.5, 1.7) per block: the
    quaternion gradient is exact for all quaternions ("backward.rs", module doc),
    and the rotation is applied as given, not renormalised."""
    w = _small(W.ROT_QUAT, dtype, **kw)
    t = W.generate(w, device="cpu")
    g = torch.Generator().manual_seed(77)
    scale = 0.5 + 1.2 * torch.rand(t["rot"].shape[:-1] + (1,), generator=g, dtype=torch.float64)
    t["rot"] = (t["rot"].double() * scale).to(t["rot"].dtype)
    _log(f"[nonunit] {w}")
    gpu = gpu_run(w, {k: (None if v is None else v.to(DEV)) for k, v in t.items()})
    ref = oracle_run(w, t)
    compare(w, gpu, ref)


def test_pooled_first_moment():
    """The pages' pooled m1[b,h,r] = m1.sum(p); their pooled cotangent is d_m1
    broadcast over p."""
    w = _small(W.ROT_PAIRWISE, "f32")
    t = W.generate(w, device="cpu")
    pooled = torch.randn(w.b, w.h, 1, w.r)
    t["d_m1"] = pooled.expand(w.b, w.h, w.p, w.r).contiguous()
    gpu = gpu_run(w, {k: (None if v is None else v.to(DEV)) for k, v in t.items()})
    ref = oracle_run(w, t)
    compare(w, gpu, ref)
    g1 = gpu["m1"].sum(2).double().cpu().numpy()
    assert np.allclose(g1, ref["m1"].sum(2), rtol=1e-4, atol=1e-4 * np.abs(ref["m1"]).max())


# ------------------------------------------------------------------ workloads
def _chains_for(w):
    """A sample of whole chains: the first, the last and a middle one."""
    n = w.b * w.h
    return sorted({0, n - 1, n // 2}) if n > 2 else list(range(n))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w", W.ALL, ids=[w.name for w in W.ALL])
def test_workload_parity(w):
    """Each benchmark workload at full size, on the launch configuration the
    benchmark uses; the oracle recomputes a sample of whole (b,h) chains."""
    _log(f"[workload] {w.name}: generating on the GPU")
    t = W.generate(w, device=DEV)
    gpu = gpu_run(w, t)
    chains = list(range(w.b * w.h)) if w.b * w.h * w.s <= 4096 else _chains_for(w)
    _log(f"[workload] {w.name}: oracle on chains {chains}")
    sub = sub_chains({k: (None if v is None else v.cpu()) for k, v in t.items()}, chains, w.h)
    ws = w.replace(b=len(chains), h=1)
    ref = oracle_run(ws, sub)
    picked = {k: (None if v is None else select_chains(v, k, chains, w.h)) for k, v in gpu.items()}
    errs = compare(ws, picked, ref)
    _log(f"[workload] {w.name}: errors {errs}")
    # exact zeros past valid_len over the whole batch, not only the sample
    V = min(w.valid_len, w.s)
    for k in ("d_xhat", "d_bhat", "d_da", "d_rot"):
        if gpu.get(k) is not None:
            assert torch.count_nonzero(gpu[k][:, V:]).item() == 0, k
