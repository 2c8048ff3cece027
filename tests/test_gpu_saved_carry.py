"""GPU parity of the saved-carry variant (moments_fwd_save / moments_bwd_saved).

The forward leaves the state entering every kernel chunk (and the chunk decays)
in a caller buffer; the backward reads them instead of running its carry pass.
Checked, through the C ABI:
- the moments equal those of moments_fwd;
- the saved states equal the entering states of the chunkwise block form at the
  kernels' chunk length (fp64, oracle/chunk_form.py), in the documented layout
  (internal column order: half-split pairs interleaved), and the decays equal
  exp(sum of da) over each chunk;
- the backward's gradients meet the oracle at the usual tolerance and agree
  with moments_bwd.
Cases cover the forward that carries its own state (one workgroup per chain,
which writes the buffer from the kernel), the forward after a carry pass
(which writes it there), fp32, four channels, and the headline workload.
"""
import sys

import numpy as np
import pytest
import torch

import mamba_ssm_chunkwise_amd as M
import workloads as W
from oracle import chunk_form as cf
from parity_util import TOL, compare, desc_of, oracle_run, select_chains, sub_chains

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _align256(n):
    return (n + 255) // 256 * 256


def _saved_views(w, saved, ell):
    V = min(w.valid_len, w.s)
    nk = -(-V // ell)
    chains = w.b * w.h
    n = chains * nk * w.p * w.r
    states = saved[:4 * n].view(torch.float32).reshape(chains, nk, w.p, w.r)
    off = _align256(4 * n)
    dec = saved[off:off + 4 * chains * nk].view(torch.float32).reshape(chains, nk)
    return states, dec, nk


def _internal_order(w):
    """Caller column of each internal column (half-split pairs interleaved)."""
    if w.rot_kind == W.ROT_HALF:
        cols = []
        for i in range(w.r // 2):
            cols += [i, w.r // 2 + i]
        return np.array(cols)
    return np.arange(w.r)


def _np64(x):
    return None if x is None else x.detach().double().cpu().numpy()


def _check_saved(w, t, saved, chains):
    ell = M.kernel_chunk_len()
    states, dec, nk = _saved_views(w, saved, ell)
    perm = _internal_order(w)
    V = min(w.valid_len, w.s)
    tol = TOL[w.dtype]
    for ch in chains:
        bi, hi = divmod(ch, w.h)
        f = cf._chain_forward(_np64(t["xhat"][bi, :, :, hi]), _np64(t["bhat"][bi, :, :, hi]),
                              _np64(t["da"][bi, :, hi]), None,
                              None if t["h0"] is None else _np64(t["h0"][bi, hi]), V, W.ROT_NONE, 0, ell)
        ref = f["E"][:nk][:, :, perm]
        got = states[ch].double().cpu().numpy()
        err = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
        ref_dec = f["dec"][: nk - 1, -1]
        got_dec = dec[ch, : nk - 1].double().cpu().numpy()
        derr = np.abs(got_dec - ref_dec).max() / max(np.abs(ref_dec).max(), 1e-30) if nk > 1 else 0.0
        _log(f"[saved] {w.name} chain {ch}: states {err:.2e} decays {derr:.2e}")
        assert err <= tol and derr <= 1e-5, (err, derr)


def _run(w, chains, full_oracle):
    _log(f"[case] {w.name}")
    t = W.generate(w, device=DEV)
    d = desc_of(w)
    m2a, m1a = M.moments_fwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"])
    m2, m1, saved = M.moments_fwd_save(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"])
    torch.cuda.synchronize()
    for a, b, k in ((m2, m2a, "m2"), (m1, m1a, "m1")):
        e = ((a - b).norm() / b.norm().clamp_min(1e-30)).item()
        assert e <= 1e-6, f"{k}: saved-carry forward differs from moments_fwd by {e:.2e}"
    _check_saved(w, t, saved, chains)
    g_saved = M.moments_bwd_saved(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], saved, t["d_m2"],
                                  t["d_m1"])
    g_plain = M.moments_bwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], t["d_m2"], t["d_m1"])
    torch.cuda.synchronize()
    tol = TOL[w.dtype]
    for k, v in g_plain.items():
        if v is None:
            continue
        e = ((g_saved[k].double() - v.double()).norm() / v.double().norm().clamp_min(1e-30)).item()
        _log(f"[saved] {w.name} {k} vs moments_bwd {e:.2e}")
        assert e <= tol
    oc = chains
    if full_oracle:
        ref = oracle_run(w, t)
        gpu = {"m2": m2, "m1": m1, **g_saved}
        compare(w, gpu, ref)
    else:
        sub = sub_chains(t, oc, w.h)
        ws = w.replace(b=len(oc), h=1)
        ref = oracle_run(ws, sub)
        gpu = {k: (None if v is None else select_chains(v, k, oc, w.h))
               for k, v in {"m2": m2, "m1": m1, **g_saved}.items()}
        compare(ws, gpu, ref)


def _small(name, dtype, rot_kind, **kw):
    base = dict(b=2, s=96, c=2, h=3, p=24, r=40, chunk_len=16, valid_len=77, seed=41, angle_step=0.3,
                quat_sd=0.3)
    if rot_kind in (W.ROT_PAIRWISE, W.ROT_HALF):
        base["rope_dim"] = 16
    if rot_kind == W.ROT_QUAT:
        base["quat_blocks"] = 6
    base.update(kw)
    return W.small(name, dtype=dtype, rot_kind=rot_kind, **base)


CASES = [
    # several groups per chain: the carry pass writes the buffer
    (_small("sv_bf16_pair_groups", "bf16", W.ROT_PAIRWISE), [0, 5]),
    (_small("sv_bf16_half_groups", "bf16", W.ROT_HALF, p=16, r=32), [1, 4]),
    (_small("sv_bf16_quat_c4", "bf16", W.ROT_QUAT, c=4, p=33, r=128, quat_blocks=32, valid_len=70), [2]),
    (_small("sv_f32_pair", "f32", W.ROT_PAIRWISE), [0, 3]),
    (_small("sv_f32_half_h0none", "f32", W.ROT_HALF, h0_sd=None, p=16, r=32), [5]),
    # 512 chains: one workgroup per chain, the forward kernel writes the buffer
    (_small("sv_bf16_pair_carried", "bf16", W.ROT_PAIRWISE, b=2, h=256, p=8, r=32, valid_len=90), [0, 300, 511]),
    (_small("sv_bf16_quat_carried", "bf16", W.ROT_QUAT, b=4, h=128, c=1, p=16, r=64, quat_blocks=8,
            valid_len=96, s=128), [7, 511]),
    (_small("sv_bf16_half_carried", "bf16", W.ROT_HALF, b=2, h=256, p=8, r=32, valid_len=64, s=64), [3, 200]),
]


@pytest.mark.parametrize("w,chains", CASES, ids=[c[0].name for c in CASES])
def test_small(w, chains):
    _run(w, chains, full_oracle=w.b * w.h <= 8)


def test_headline_workload():
    w = W.BF16_PAIRWISE
    _run(w, [0, 511], full_oracle=False)
