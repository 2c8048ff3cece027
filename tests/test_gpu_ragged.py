"""GPU parity with per-sequence valid lengths (a ragged batch, desc.valid_lens).

Each sequence bi must give what the oracle gives for that sequence alone with
valid_len = min(max(valid_lens[bi], 0), desc.valid_len, s), and its gradients
must be exactly zero past that length. A sequence whose length equals the
batch bound must come out bit-identical to the run without per-sequence
lengths (the same kernels and grouping run; only masks change). Cases cover
every kernel family: the forward that carries its own state (512 chains), the
forward after a carry pass, the transposed bf16 backward, the general
backward (four channels), fp32, a zero and a negative length, a bound below
some lengths, the saved-carry variant, and the headline workload.
"""
import sys

import pytest
import torch

import mamba_ssm_chunkwise_amd as M
import workloads as W
from parity_util import compare, desc_of, gpu_run, oracle_run, select_chains, sub_chains

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _eff(w, lens):
    V = min(w.valid_len, w.s)
    return [max(0, min(int(v), V)) for v in lens]


def _ragged_run(w, t, lens, saved=False):
    d = desc_of(w)
    M.set_valid_lens(d, torch.tensor(lens, dtype=torch.int32, device=DEV))
    if saved:
        m2, m1, sv = M.moments_fwd_save(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"])
        g = M.moments_bwd_saved(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], sv, t["d_m2"], t["d_m1"])
    else:
        m2, m1 = M.moments_fwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"])
        g = M.moments_bwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], t["d_m2"], t["d_m1"])
    torch.cuda.synchronize()
    return {"m2": m2, "m1": m1, **g}


def _slice_b(x, bi):
    return None if x is None else x[bi:bi + 1]


def _check(w, t, lens, out, heads=None, saved=False):
    eff = _eff(w, lens)
    plain = None
    for bi, V in enumerate(eff):
        wb = w.replace(b=1, valid_len=V, name=f"{w.name}[b{bi},V={V}]")
        tb = {k: _slice_b(v, bi) for k, v in t.items()}
        gb = {k: _slice_b(v, bi) for k, v in out.items()}
        if heads is None:
            ref = oracle_run(wb, tb)
            compare(wb, gb, ref)
        else:
            sub = sub_chains(tb, heads, w.h)
            ws = wb.replace(h=1, b=len(heads))
            ref = oracle_run(ws, sub)
            compare(ws, {k: (None if v is None else select_chains(v, k, heads, w.h)) for k, v in gb.items()}, ref)
        if V == min(w.valid_len, w.s):
            if plain is None:
                plain = gpu_run(w, t) if not saved else _plain_saved(w, t)
            for k, v in out.items():
                if v is not None:
                    assert torch.equal(v[bi], plain[k][bi]), f"{k}[{bi}] differs from the run without lengths"


def _plain_saved(w, t):
    d = desc_of(w)
    m2, m1, sv = M.moments_fwd_save(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"])
    g = M.moments_bwd_saved(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], sv, t["d_m2"], t["d_m1"])
    torch.cuda.synchronize()
    return {"m2": m2, "m1": m1, **g}


def _small(name, dtype, rot_kind, **kw):
    base = dict(b=3, s=96, c=2, h=2, p=24, r=40, chunk_len=16, valid_len=96, seed=51, angle_step=0.3,
                quat_sd=0.3)
    if rot_kind in (W.ROT_PAIRWISE, W.ROT_HALF):
        base["rope_dim"] = 16
    if rot_kind == W.ROT_QUAT:
        base["quat_blocks"] = 6
    base.update(kw)
    return W.small(name, dtype=dtype, rot_kind=rot_kind, **base)


CASES = [
    (_small("rg_bf16_pair", "bf16", W.ROT_PAIRWISE), [77, 0, 96], None),
    (_small("rg_bf16_half", "bf16", W.ROT_HALF, p=16, r=32), [33, 96, -5], None),
    (_small("rg_bf16_quat_c4", "bf16", W.ROT_QUAT, b=2, c=4, p=33, r=128, quat_blocks=32), [70, 31], None),
    (_small("rg_f32_half", "f32", W.ROT_HALF), [40, 96, 17], None),
    (_small("rg_f32_pair_bound", "f32", W.ROT_PAIRWISE, b=2, valid_len=60), [96, 20], None),
    (_small("rg_bf16_none", "bf16", W.ROT_NONE, b=2, c=1, p=37, r=64), [1, 95], None),
    # 512 chains: one workgroup per chain, the forward carries its own state
    (_small("rg_bf16_pair_carried", "bf16", W.ROT_PAIRWISE, b=4, h=128, p=8, r=32, s=64, valid_len=64),
     [64, 33, 1, 50], [0, 77, 127]),
    # 16 chains of 64 chunks: groups of two chunks, the forward carries its state through each
    # group from the group-entry states its carry pass stores; one sequence ends mid-group
    (_small("rg_bf16_quat_grouped", "bf16", W.ROT_QUAT, b=2, h=8, c=2, p=16, r=32, quat_blocks=8, s=2048,
            valid_len=2048, chunk_len=64), [1500, 2048], [0, 7]),
    # four channels and 128 columns over 512 group workgroups: the carry walk's group forms
    # stage each chunk in one LDS buffer, so that two workgroups share a CU
    (_small("rg_bf16_quat_c4_grouped", "bf16", W.ROT_QUAT, b=2, h=8, c=4, p=32, r=128, quat_blocks=32,
            s=2048, valid_len=2048, chunk_len=64), [2048, 1200], [0, 7]),
]


@pytest.mark.parametrize("w,lens,heads", CASES, ids=[c[0].name for c in CASES])
def test_small(w, lens, heads):
    _log(f"[case] {w.name} lens {lens}")
    t = W.generate(w, device=DEV)
    out = _ragged_run(w, t, lens)
    _check(w, t, lens, out, heads)


def test_saved_carry():
    w = _small("rg_saved_carried", "bf16", W.ROT_QUAT, b=4, h=128, c=1, p=16, r=64, quat_blocks=8, s=128,
               valid_len=128)
    lens = [128, 100, 31, 65]
    _log(f"[case] {w.name} lens {lens}")
    t = W.generate(w, device=DEV)
    out = _ragged_run(w, t, lens, saved=True)
    _check(w, t, lens, out, heads=[5, 127], saved=True)


def test_headline_workload():
    w = W.BF16_PAIRWISE
    lens = [8192, 4000, 7777, 1, 8192, 6000, 2048, 5000]
    _log(f"[case] {w.name} lens {lens}")
    t = W.generate(w, device=DEV)
    out = _ragged_run(w, t, lens)
    _check(w, t, lens, out, heads=[0, 63])


def test_binding_checks():
    w = _small("rg_bind", "f32", W.ROT_PAIRWISE)
    d = desc_of(w)
    with pytest.raises(ValueError, match="int32"):
        M.set_valid_lens(d, torch.tensor([1, 2, 3], dtype=torch.int64, device=DEV))
    with pytest.raises(ValueError, match="shape"):
        M.set_valid_lens(d, torch.tensor([1, 2], dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError, match="GPU"):
        M.set_valid_lens(d, torch.tensor([1, 2, 3], dtype=torch.int32))
