"""Loop transcription of the pages' chunkwise algebra, numpy fp64 (test infrastructure).

Follows the burn-mamba ``recalculated.rs`` source page (chunk_decay, chunk_states,
chunk_writes, rotate_chunk, chunk_mask, moments_phys_fwd) and the ``backward.rs``
source page (module doc "Gradient math"; boundary_carries; the reverse chunk loop
of moments_phys_bwd with G, d_W = L^T G and the rev-cumsum d_da identity;
d_theta_chunk; d_quat_chunk). Written from the formulas, in this file's own
code, for small inputs only. It is used to pin the C oracle: chunk-length
invariance (this form at any chunk length l equals the per-token recurrence) and
the d_da identity (checked here against the direct double sum as well).

The per-p first moment m1[b,h,p,r] is returned; the pages' pooled m1[b,h,r] is
its sum over p, and the pages' pooled cotangent is obtained by passing d_m1
broadcast over p.
"""
from __future__ import annotations

import numpy as np

from .oracle import ROT_HALF, ROT_NONE, ROT_PAIRWISE, ROT_QUAT


def chunk_decay(da_l):
    """a = inclusive cumsum of da in the chunk; d_t = exp(a_t);
    L[t,j] = exp(a_t - a_j) on and below the diagonal, 0 strictly above."""
    a = np.cumsum(da_l)
    d = np.exp(a)
    below = np.tril(np.ones((len(a), len(a)), dtype=bool))
    diff = np.where(below, a[:, None] - a[None, :], -np.inf)
    L = np.exp(diff)
    return a, d, L


def chunk_states(xh, bh, d, L, h_in):
    """h~[t] = d_t h_in + sum_{j<=t, c} L[t,j] xhat[j,c] (outer) bhat[j,c].
    xh [l,c,p], bh [l,c,r] -> [l,p,r]."""
    l = xh.shape[0]
    out = d[:, None, None] * h_in[None]
    for t in range(l):
        for j in range(t + 1):
            out[t] += L[t, j] * np.einsum("cp,cr->pr", xh[j], bh[j])
    return out


def chunk_writes(xh, bh):
    """W_j = sum_c xhat[j,c] (outer) bhat[j,c] -> [l,p,r]."""
    return np.einsum("jcp,jcr->jpr", xh, bh)


def quat_mul(a, b):
    """Hamilton product on a trailing (w,x,y,z) axis."""
    aw, ax, ay, az = a[..., 0], a[..., 1], a[..., 2], a[..., 3]
    bw, bx, by, bz = b[..., 0], b[..., 1], b[..., 2], b[..., 3]
    return np.stack([
        aw * bw - ax * bx - ay * by - az * bz,
        aw * bx + ax * bw + ay * bz - az * by,
        aw * by - ax * bz + ay * bw + az * bx,
        aw * bz + ax * by - ay * bx + az * bw,
    ], axis=-1)


def quat_conj(q):
    return q * np.array([1.0, -1.0, -1.0, -1.0])


def rotate_chunk(v, rot_l, rot_kind, rope_dim, transpose):
    """v [l,p,r]; rot_l [l,a] angles or [l,J,4] quaternions. transpose=False is the
    de-rotation R(-theta) / left product by Q; True its transpose R(+theta) /
    left product by conj(Q)."""
    out = v.copy()
    l, p, r = v.shape
    if rot_kind in (ROT_PAIRWISE, ROT_HALF):
        if rope_dim == 0:
            return out
        a = rope_dim // 2
        th = rot_l[:, :a] if transpose else -rot_l[:, :a]
        cs, sn = np.cos(th)[:, None, :], np.sin(th)[:, None, :]
        if rot_kind == ROT_PAIRWISE:
            i0, i1 = np.arange(0, rope_dim, 2), np.arange(1, rope_dim, 2)
        else:
            i0, i1 = np.arange(a), r // 2 + np.arange(a)
        x0, x1 = v[:, :, i0], v[:, :, i1]
        out[:, :, i0] = cs * x0 - sn * x1
        out[:, :, i1] = sn * x0 + cs * x1
    elif rot_kind == ROT_QUAT:
        J = rot_l.shape[1]
        q = rot_l[:, None, :, :]  # [l,1,J,4]
        q = quat_conj(q) if transpose else q
        blocks = v[:, :, :4 * J].reshape(l, p, J, 4)
        out[:, :, :4 * J] = quat_mul(np.broadcast_to(q, blocks.shape), blocks).reshape(l, p, 4 * J)
    return out


def chunk_mask(l, start, valid_len):
    return (start + np.arange(l) < valid_len).astype(np.float64)


def _chunk(x, n, l):
    return x[n * l:(n + 1) * l]


def moments_fwd(xhat, bhat, da, rot, h0, valid_len, rot_kind, rope_dim, l):
    """Serial chunk loop (breaks at start >= valid_len). Returns m2, m1 per-p."""
    b, s, c, h, p = xhat.shape
    r = bhat.shape[-1]
    assert s % l == 0
    nch = s // l
    m2 = np.zeros((b, h, r, r))
    m1 = np.zeros((b, h, p, r))
    for bi in range(b):
        for hi in range(h):
            hcar = np.zeros((p, r)) if h0 is None else h0[bi, hi].astype(np.float64).copy()
            for n in range(nch):
                start = n * l
                if start >= valid_len:
                    break
                _, d, L = chunk_decay(_chunk(da[bi, :, hi], n, l))
                xh = _chunk(xhat[bi, :, :, hi, :], n, l)
                bh = _chunk(bhat[bi, :, :, hi, :], n, l)
                st = chunk_states(xh, bh, d, L, hcar)
                hcar = st[l - 1].copy()
                rl = None if rot is None else _chunk(rot[bi, :, hi], n, l)
                ph = rotate_chunk(st, rl, rot_kind, rope_dim, False)
                ph = ph * chunk_mask(l, start, valid_len)[:, None, None]
                flat = ph.reshape(l * p, r)
                m2[bi, hi] += flat.T @ flat
                m1[bi, hi] += ph.sum(0)
    return m2, m1


def rev_cumsum(v):
    return np.cumsum(v[::-1])[::-1]


def moments_bwd(xhat, bhat, da, rot, h0, dm2, dm1, valid_len, rot_kind, rope_dim, l,
                dda_form="identity"):
    """Recompute backward in reverse chunk order. dda_form: "identity" (the
    rev-cumsum form) or "double_sum" (the direct sum over pairs j < s <= t)."""
    b, s, c, h, p = xhat.shape
    r = bhat.shape[-1]
    nch = s // l
    processed = min(-(-valid_len // l), nch)
    g = {"d_xhat": np.zeros(xhat.shape), "d_bhat": np.zeros(bhat.shape), "d_da": np.zeros(da.shape),
         "d_rot": None if rot is None else np.zeros(rot.shape), "d_h0": np.zeros((b, h, p, r))}
    for bi in range(b):
        for hi in range(h):
            # boundary carries h_-(n)
            carries = []
            hcar = np.zeros((p, r)) if h0 is None else h0[bi, hi].astype(np.float64).copy()
            for n in range(processed):
                carries.append(hcar.copy())
                a, _, _ = chunk_decay(_chunk(da[bi, :, hi], n, l))
                scale = np.exp(a[-1] - a)
                xh = _chunk(xhat[bi, :, :, hi, :], n, l)
                bh = _chunk(bhat[bi, :, :, hi, :], n, l)
                hcar = np.exp(a[-1]) * hcar + np.einsum("j,jcp,jcr->pr", scale, xh, bh)
            S = dm2[bi, hi] + dm2[bi, hi].T
            dcar = np.zeros((p, r))
            for n in reversed(range(processed)):
                start = n * l
                _, d, L = chunk_decay(_chunk(da[bi, :, hi], n, l))
                xh = _chunk(xhat[bi, :, :, hi, :], n, l)
                bh = _chunk(bhat[bi, :, :, hi, :], n, l)
                st = chunk_states(xh, bh, d, L, carries[n])
                rl = None if rot is None else _chunk(rot[bi, :, hi], n, l)
                ph = rotate_chunk(st, rl, rot_kind, rope_dim, False)
                mask = chunk_mask(l, start, valid_len)[:, None, None]
                dph = (ph @ S + dm1[bi, hi][None]) * mask
                dst = rotate_chunk(dph, rl, rot_kind, rope_dim, True)
                if rot_kind in (ROT_PAIRWISE, ROT_HALF) and rope_dim > 0:
                    a_n = rope_dim // 2
                    if rot_kind == ROT_PAIRWISE:
                        i0, i1 = np.arange(0, rope_dim, 2), np.arange(1, rope_dim, 2)
                    else:
                        i0, i1 = np.arange(a_n), r // 2 + np.arange(a_n)
                    dth = (dph[:, :, i0] * ph[:, :, i1] - dph[:, :, i1] * ph[:, :, i0]).sum(1)
                    g["d_rot"][bi, start:start + l, hi, :a_n] = dth
                elif rot_kind == ROT_QUAT:
                    J = rot.shape[3]
                    blk = lambda t: t[:, :, :4 * J].reshape(l, p, J, 4)  # noqa: E731
                    dq = quat_mul(blk(dph), quat_conj(blk(st))).sum(1)
                    g["d_rot"][bi, start:start + l, hi] = dq
                G = dst.copy()
                G[l - 1] += dcar
                dcar = np.einsum("t,tpr->pr", d, G)
                dW = np.einsum("tj,tpr->jpr", L, G)
                g["d_xhat"][bi, start:start + l, :, hi, :] = np.einsum("jcr,jpr->jcp", bh, dW)
                g["d_bhat"][bi, start:start + l, :, hi, :] = np.einsum("jcp,jpr->jcr", xh, dW)
                W = chunk_writes(xh, bh)
                scal = np.einsum("tpr,pr->t", G, carries[n]) * d
                A = np.einsum("tpr,jpr->tj", G, W) * L
                if dda_form == "identity":
                    dda = rev_cumsum(scal + A.sum(1)) - rev_cumsum(A.sum(0))
                else:
                    dda = np.zeros(l)
                    for s_ in range(l):
                        dda[s_] = scal[s_:].sum() + sum(A[t, j] for t in range(s_, l) for j in range(s_))
                g["d_da"][bi, start:start + l, hi] = dda
            g["d_h0"][bi, hi] = dcar
    return g
