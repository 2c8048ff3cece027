"""Chunkwise block form of the physical-frame state moments, numpy fp64 (TEST INFRASTRUCTURE).

A second CPU formulation, organised by chunks of any length l, used only to pin
the C oracle (``moments_oracle.c``), which follows the per-token recurrence:

* chunk-length invariance: the "backward.rs" page (module doc, "Gradient math")
  states the decays d_t and L[t,j] as products of exp(da) over the tokens in
  between, so the chunked states equal the recurrence exactly at every l;
* the decay gradient: the page's reverse-cumsum identity for d_da, its direct
  double sum over pairs j < s <= t, and a log-decay cotangent form derived below
  must agree with each other and with the recurrence.

Everything is written from the equations, with the chunks as a leading array
axis (so each step is one batched numpy operation over all chunks of a chain):

  a[n,t]    inclusive cumsum of da inside chunk n (log-decay)
  T[n,t,j]  exp(a[n,t] - a[n,j]) for j <= t, else 0 (causal transfer)
  U[n,j]    sum_c xhat[n,j,c] (outer) bhat[n,j,c] (injections)
  Z[n]      T[n] U[n] (chunk-local states, zero entering state)
  E[n]      state entering chunk n: E[0] = h0, E[n+1] = exp(a[n,l-1]) E[n] + Z[n,l-1]
  H[n,t]    exp(a[n,t]) E[n] + Z[n,t]
  C[n,t]    de-rotated rows: complex pairs through complex numbers
            (x + i y) -> exp(-i theta) (x + i y); quaternion 4-blocks through
            the 4x4 matrix of left multiplication by Q
  m2 = sum C^T C, m1 = sum C over positions < valid_len.

The backward is the adjoint of this block form. With dC = mask (C S + d_m1),
S = d_m2 + d_m2^T, the direct state cotangent is the inverse rotation of dC;
the cotangent Gt[n,t] adds, at the chunk's last token, the cotangent D[n+1] of
the next chunk's entering state; D[n] = sum_t exp(a[n,t]) Gt[n,t]; the
injection cotangent is dU[n] = T[n]^T Gt[n], giving d_xhat = dU bhat and
d_bhat = dU^T xhat. The angle gradient is the page's sum over rows of
d_cx c_y - d_cy c_x, taken here as Im(conj(dz) z) of the complex pairs; the
quaternion gradient is the page's sum over rows of d_c (x) conj(h~).

Decay gradient, three forms:
  "log"        dL/da[n,k] = <Gt[n,k], H[n,k]> - <dU[n,k], U[n,k]> (H depends on a
               only through exp(a_t) and exp(-a_j)), then d_da = suffix sums of it
               inside the chunk (a is a prefix sum of da);
  "identity"   scal[t] = exp(a_t) <Gt[t], E>, A[t,j] = T[t,j] <Gt[t], U[j]>,
               d_da = revcumsum(scal + rowsum A) - revcumsum(colsum A)
               (the page's identity);
  "double_sum" d_da[s] = sum_{t>=s} scal[t] + sum_{j<s<=t} A[t,j], brute force.

m1 is returned per row p ([b,h,p,r]); the pages' pooled m1[b,h,r] is its sum
over p. For small inputs only.
"""
from __future__ import annotations

import numpy as np

from .oracle import ROT_HALF, ROT_NONE, ROT_PAIRWISE, ROT_QUAT  # noqa: F401


def _pair_index(rot_kind, rope_dim, r):
    a = rope_dim // 2
    if rot_kind == ROT_PAIRWISE:
        return 2 * np.arange(a), 2 * np.arange(a) + 1
    return np.arange(a), r // 2 + np.arange(a)


def _left_matrix(q):
    """4x4 matrix of v -> q (x) v (Hamilton product), q [..., 4] = (w, x, y, z)."""
    w, x, y, z = q[..., 0], q[..., 1], q[..., 2], q[..., 3]
    rows = [[w, -x, -y, -z], [x, w, -z, y], [y, z, w, -x], [z, -y, x, w]]
    return np.stack([np.stack(rw, axis=-1) for rw in rows], axis=-2)


def _hamilton(a, b):
    """(a (x) b) on a trailing (w, x, y, z) axis, via a's left-multiplication matrix."""
    return np.einsum("...ij,...j->...i", _left_matrix(a), b)


def _conj(q):
    return q * np.array([1.0, -1.0, -1.0, -1.0])


class _Rotation:
    """De-rotation of state rows and its transpose for one chain's chunks.
    rot: [N, l, A] angles or [N, l, J, 4] quaternions (or None)."""

    def __init__(self, rot, rot_kind, rope_dim, r):
        self.kind = rot_kind if rot is not None else ROT_NONE
        self.r = r
        if self.kind in (ROT_PAIRWISE, ROT_HALF):
            if rope_dim == 0:
                self.kind = ROT_NONE
                return
            self.i0, self.i1 = _pair_index(rot_kind, rope_dim, r)
            self.phase = np.exp(-1j * rot[..., :rope_dim // 2])[:, :, None, :]   # [N, l, 1, A]
        elif self.kind == ROT_QUAT:
            self.J = rot.shape[2]
            self.q = rot
            self.Lq = _left_matrix(rot)[:, :, None]                                # [N, l, 1, J, 4, 4]

    def _z(self, v):
        return v[..., self.i0] + 1j * v[..., self.i1]

    def _put(self, v, z):
        out = v.copy()
        out[..., self.i0], out[..., self.i1] = z.real, z.imag
        return out

    def _blocks(self, v):
        return v[..., :4 * self.J].reshape(v.shape[:-1] + (self.J, 4))

    def _put_blocks(self, v, b):
        out = v.copy()
        out[..., :4 * self.J] = b.reshape(v.shape[:-1] + (4 * self.J,))
        return out

    def forward(self, v):
        """v [N, l, p, r] -> de-rotated rows."""
        if self.kind in (ROT_PAIRWISE, ROT_HALF):
            return self._put(v, self._z(v) * self.phase)
        if self.kind == ROT_QUAT:
            return self._put_blocks(v, np.einsum("...jab,...jb->...ja", self.Lq, self._blocks(v)))
        return v.copy()

    def transpose(self, v):
        if self.kind in (ROT_PAIRWISE, ROT_HALF):
            return self._put(v, self._z(v) * np.conj(self.phase))
        if self.kind == ROT_QUAT:
            return self._put_blocks(v, np.einsum("...jba,...jb->...ja", self.Lq, self._blocks(v)))
        return v.copy()

    def param_grad(self, dc, c, h):
        """Gradient with respect to the rotation input, summed over the rows p:
        complex, Im(conj(dz) z) with z the de-rotated pair; quaternion, d_c (x) conj(h~)."""
        if self.kind in (ROT_PAIRWISE, ROT_HALF):
            return (np.conj(self._z(dc)) * self._z(c)).imag.sum(2)
        if self.kind == ROT_QUAT:
            return _hamilton(self._blocks(dc), _conj(self._blocks(h))).sum(2)
        return None


def _chunks(x, N, l):
    return x[:N * l].reshape((N, l) + x.shape[1:])


def _chain_forward(xh, bh, da, rot, h0, V, rot_kind, rope_dim, l):
    """One chain: returns everything the backward reuses."""
    s, c, p = xh.shape
    r = bh.shape[-1]
    N = min(-(-V // l), s // l)
    a = np.cumsum(_chunks(da, N, l), axis=1)                     # [N, l]
    dec = np.exp(a)
    causal = np.tril(np.ones((l, l), dtype=bool))
    T = np.where(causal, np.exp(np.where(causal, a[:, :, None] - a[:, None, :], 0.0)), 0.0)
    X, B = _chunks(xh, N, l), _chunks(bh, N, l)                  # [N, l, c, p], [N, l, c, r]
    U = np.einsum("njcp,njcr->njpr", X, B)
    Z = np.einsum("ntj,njpr->ntpr", T, U)
    E = np.zeros((N + 1, p, r))
    E[0] = 0.0 if h0 is None else h0
    for n in range(N):
        E[n + 1] = dec[n, -1] * E[n] + Z[n, -1]
    H = dec[:, :, None, None] * E[:N, None] + Z
    R = _Rotation(None if rot is None else _chunks(rot, N, l), rot_kind, rope_dim, r)
    C = R.forward(H)
    mask = (np.arange(N * l).reshape(N, l) < V).astype(np.float64)[:, :, None, None]
    return dict(N=N, a=a, dec=dec, T=T, X=X, B=B, U=U, E=E, H=H, R=R, C=C, mask=mask)


def moments_fwd_chunked(xhat, bhat, da, rot, h0, valid_len, rot_kind, rope_dim, l):
    """m2 [b,h,r,r], m1 [b,h,p,r] from the block form at chunk length l (s % l == 0)."""
    b, s, c, h, p = xhat.shape
    r = bhat.shape[-1]
    assert s % l == 0
    V = min(valid_len, s)
    m2 = np.zeros((b, h, r, r))
    m1 = np.zeros((b, h, p, r))
    for bi in range(b):
        for hi in range(h):
            if V == 0:
                continue
            f = _chain_forward(xhat[bi, :, :, hi], bhat[bi, :, :, hi], da[bi, :, hi],
                               None if rot is None else rot[bi, :, hi],
                               None if h0 is None else h0[bi, hi], V, rot_kind, rope_dim, l)
            Cm = (f["C"] * f["mask"]).reshape(-1, p, r)
            m2[bi, hi] = np.einsum("kpa,kpb->ab", Cm, Cm)
            m1[bi, hi] = Cm.sum(0)
    return m2, m1


def _suffix_sum(v, axis=-1):
    return np.flip(np.cumsum(np.flip(v, axis), axis), axis)


def moments_bwd_chunked(xhat, bhat, da, rot, h0, dm2, dm1, valid_len, rot_kind, rope_dim, l, dda="log"):
    """The block form's adjoint: d_xhat, d_bhat, d_da, d_rot, d_h0 (fp64).
    dda selects the decay-gradient form: "log", "identity" or "double_sum"."""
    b, s, c, h, p = xhat.shape
    r = bhat.shape[-1]
    assert s % l == 0
    V = min(valid_len, s)
    g = {"d_xhat": np.zeros(xhat.shape), "d_bhat": np.zeros(bhat.shape), "d_da": np.zeros(da.shape),
         "d_rot": None if (rot is None or rot_kind == ROT_NONE) else np.zeros(rot.shape),
         "d_h0": np.zeros((b, h, p, r))}
    for bi in range(b):
        for hi in range(h):
            if V == 0:
                continue
            f = _chain_forward(xhat[bi, :, :, hi], bhat[bi, :, :, hi], da[bi, :, hi],
                               None if rot is None else rot[bi, :, hi],
                               None if h0 is None else h0[bi, hi], V, rot_kind, rope_dim, l)
            N, R, T, dec = f["N"], f["R"], f["T"], f["dec"]
            S = dm2[bi, hi] + dm2[bi, hi].T
            dC = (f["C"] @ S + dm1[bi, hi]) * f["mask"]
            Gd = R.transpose(dC)                                      # direct cotangent of H
            Gt = Gd.copy()
            D = np.zeros((p, r))                                      # nothing leaves the last chunk
            for n in reversed(range(N)):
                Gt[n, -1] += D
                D = np.einsum("t,tpr->pr", dec[n], Gt[n])
            g["d_h0"][bi, hi] = D
            dU = np.einsum("ntj,ntpr->njpr", T, Gt)
            n_tok = N * l
            g["d_xhat"][bi, :n_tok, :, hi] = np.einsum("njpr,njcr->njcp", dU, f["B"]).reshape(n_tok, c, p)
            g["d_bhat"][bi, :n_tok, :, hi] = np.einsum("njpr,njcp->njcr", dU, f["X"]).reshape(n_tok, c, r)
            if dda == "log":
                ga = np.einsum("ntpr,ntpr->nt", Gt, f["H"]) - np.einsum("ntpr,ntpr->nt", dU, f["U"])
                dd = _suffix_sum(ga, axis=1)
            else:
                scal = dec * np.einsum("ntpr,npr->nt", Gt, f["E"][:N])
                A = T * np.einsum("ntpr,njpr->ntj", Gt, f["U"])
                if dda == "identity":
                    dd = _suffix_sum(scal + A.sum(2), axis=1) - _suffix_sum(A.sum(1), axis=1)
                else:
                    dd = np.zeros((N, l))
                    for n in range(N):
                        for s_ in range(l):
                            dd[n, s_] = scal[n, s_:].sum() + sum(A[n, t, j] for t in range(s_, l)
                                                                 for j in range(s_))
            g["d_da"][bi, :n_tok, hi] = dd.reshape(n_tok)
            pg = R.param_grad(dC, f["C"], f["H"])
            if g["d_rot"] is not None and pg is not None:
                if rot_kind == ROT_QUAT:
                    g["d_rot"][bi, :n_tok, hi] = pg.reshape((n_tok,) + pg.shape[2:])
                else:
                    g["d_rot"][bi, :n_tok, hi, :rope_dim // 2] = pg.reshape(n_tok, -1)
    return g
