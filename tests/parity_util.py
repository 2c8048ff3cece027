"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding and the CPU oracle on the same (cast) inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch

import mamba_ssm_chunkwise_amd as M
import workloads as W
from oracle import oracle_bwd, oracle_fwd

TOL = {"f32": 1e-4, "bf16": 2e-2}
GRADS = ("d_xhat", "d_bhat", "d_da", "d_rot", "d_h0")


def desc_of(w: W.Workload):
    return M.Desc(w.b, w.s, w.c, w.h, w.p, w.r, w.chunk_len, w.valid_len,
                  M.BF16 if w.dtype == "bf16" else M.F32, w.rot_kind, w.rope_dim, w.quat_blocks)


def gpu_run(w, t, bwd=True):
    """t: dict of device tensors from workloads.generate. Returns device outputs."""
    d = desc_of(w)
    m2, m1 = M.moments_fwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"])
    out = {"m2": m2, "m1": m1}
    if bwd:
        g = M.moments_bwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], t["d_m2"], t["d_m1"])
        out.update(g)
    torch.cuda.synchronize()
    return out


def _np64(x):
    return None if x is None else x.detach().double().cpu().numpy()


def sub_chains(t, chains, h):
    """Slice inputs down to the listed flat (b*h + h) chains, as a problem with
    b = len(chains), h = 1 (chains are independent)."""
    out = {}
    bs = [c // h for c in chains]
    hs = [c % h for c in chains]
    for k, v in t.items():
        if v is None:
            out[k] = None
            continue
        if k in ("xhat", "bhat"):
            out[k] = torch.stack([v[b, :, :, hh:hh + 1] for b, hh in zip(bs, hs)])
        elif k in ("da", "rot"):
            out[k] = torch.stack([v[b, :, hh:hh + 1] for b, hh in zip(bs, hs)])
        else:  # h0, d_m2, d_m1: [b, h, ...]
            out[k] = torch.stack([v[b, hh:hh + 1] for b, hh in zip(bs, hs)])
    return out


def oracle_run(w, t, bwd=True):
    """CPU oracle on tensors (any device); returns fp64 numpy dict."""
    a = {k: _np64(v) for k, v in t.items()}
    m2, m1 = oracle_fwd(a["xhat"], a["bhat"], a["da"], a["rot"], a["h0"], w.valid_len, w.rot_kind,
                        w.rope_dim)
    out = {"m2": m2, "m1": m1}
    if bwd:
        out.update(oracle_bwd(a["xhat"], a["bhat"], a["da"], a["rot"], a["h0"], a["d_m2"], a["d_m1"],
                              w.valid_len, w.rot_kind, w.rope_dim))
    return out


def select_chains(x, name, chains, h):
    """Pick the listed chains out of a full-size output, shaped like sub_chains."""
    bs = [c // h for c in chains]
    hs = [c % h for c in chains]
    if name in ("d_xhat", "d_bhat"):
        return torch.stack([x[b, :, :, hh:hh + 1] for b, hh in zip(bs, hs)])
    if name in ("d_da", "d_rot"):
        return torch.stack([x[b, :, hh:hh + 1] for b, hh in zip(bs, hs)])
    return torch.stack([x[b, hh:hh + 1] for b, hh in zip(bs, hs)])


def rel_err(gpu, ref):
    """Normwise relative error ||gpu - ref||_F / ||ref||_F (ref != 0)."""
    num = np.linalg.norm((gpu - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    return num / den if den > 0 else num


def max_err(gpu, ref):
    """Largest elementwise error over the largest reference magnitude."""
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(gpu - ref).max() if ref.size else 0.0
    return num / den if den > 0 else num


def token_err(gpu, ref):
    """Worst per-token error of a [b, s, ...] gradient: max over tokens t of
    ||gpu_t - ref_t|| / max(||ref_t||, rms_t ||ref_t||), with the norms over every
    axis but the token axis. A value wrong at one token scores about 1."""
    d = np.moveaxis(gpu - ref, 1, 0).reshape(ref.shape[1], -1)
    r = np.moveaxis(ref, 1, 0).reshape(ref.shape[1], -1)
    rn = np.linalg.norm(r, axis=1)
    rms = np.sqrt(np.mean(rn ** 2)) if rn.size else 0.0
    if rms == 0.0:
        return float(np.linalg.norm(d))
    return float((np.linalg.norm(d, axis=1) / np.maximum(rn, rms)).max())


def compare(w, gpu, ref, tol=None, names=None):
    """Checks every output to the tolerance and returns {name: (normwise, max
    elementwise over max|ref|)} errors. Each tensor must meet the normwise bound
    and |gpu - ref| <= tol * max|ref| elementwise; d_da and d_rot must also meet
    the per-token bound (token_err <= tol); gradients past valid_len must be
    exactly zero."""
    tol = TOL[w.dtype] if tol is None else tol
    errs = {}
    tok = {}
    for k in names or ("m2", "m1") + GRADS:
        if k not in ref or ref[k] is None:
            continue
        g = _np64(gpu[k])
        assert g is not None, f"{k} missing from the GPU outputs"
        assert np.all(np.isfinite(g)), f"{k} has non-finite values"
        errs[k] = (rel_err(g, ref[k]), max_err(g, ref[k]))
        if k in ("d_da", "d_rot"):
            tok[k] = token_err(g, ref[k])
    report = ", ".join(f"{k} {e:.2e}/{m:.2e}" for k, (e, m) in errs.items())
    report += "".join(f", {k} per-token {v:.2e}" for k, v in tok.items())
    print(f"[compare] {w.name}: normwise/max-elementwise {report}", flush=True)
    bad = [k for k, (e, m) in errs.items() if not (e <= tol and m <= tol)]
    bad += [k for k, v in tok.items() if not v <= tol]
    assert not bad, f"{w.name}: errors above {tol:.1e} in {bad}: {report}"
    V = min(w.valid_len, w.s)
    for k in ("d_xhat", "d_bhat", "d_da", "d_rot"):
        if k in gpu and gpu[k] is not None:
            tail = gpu[k][:, V:]
            assert torch.count_nonzero(tail).item() == 0, f"{k} is not exactly zero past valid_len"
    return {k: e for k, (e, m) in errs.items()}
