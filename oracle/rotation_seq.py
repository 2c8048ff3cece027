"""Rotation-sequence producer and its VJP, numpy fp64 (TEST INFRASTRUCTURE).

The moments path takes the per-token rotation as a cumulative quantity (the
"recalculated.rs" source page: ``RotPrim`` holds cumulative angles
``[b, s, h, a]`` or cumulative unit quaternions ``[b, s, h, J, 4]``, the
counterpart of the model's rotation sequence; ``quat_mul_prim`` is the Hamilton
product on a packed (w, x, y, z) axis). The step that builds those cumulative
values from per-token increments is not printed on the pages; this module takes
the plainest reading:

* complex angles: theta[t] = sum_{t' <= t} inc[t'] (inclusive sum over the
  sequence axis, per (b, h, angle));
* quaternions: composed left to right, each step renormalised,
      Q[-1] = 1,   Q[t] = N(Q[t-1] (x) q[t]),   N(v) = v / |v|,
  per (b, h, block). For unit increments N changes nothing in exact arithmetic;
  for any nonzero increments Q[t] is the normalised product q[0] (x) ... (x) q[t]
  (the Hamilton product is bilinear, so normalising early only rescales).

Both run over the whole sequence: positions past a chain's valid length get a
rotation too, which the moments path never reads, and their cotangents there
arrive as zeros.

The backward maps cotangents of the cumulative values back to the increments:
* angles: d_inc[t] = sum_{t' >= t} d_theta[t'];
* quaternions: reverse-mode through each step, with Y[t] = Q[t-1] (x) q[t] and
  g[t] the cotangent reaching Q[t] (its own d_Q[t] plus what step t+1 sends back):
      d_Y[t]   = (g[t] - Q[t] <Q[t], g[t]>) / |Y[t]|     (through N)
      d_q[t]   = conj(Q[t-1]) (x) d_Y[t]                  (v -> a (x) v has transpose v -> conj(a) (x) v)
      g[t-1]  += d_Y[t] (x) conj(q[t])                    (v -> v (x) b has transpose v -> v (x) conj(b))

Plain loops over the sequence, vectorised over every other axis. Pins:
``tests/test_rotation_seq.py``.
"""
from __future__ import annotations

import numpy as np


def hamilton(a, b):
    """Hamilton product a (x) b over a trailing (w, x, y, z) axis."""
    aw, ax, ay, az = np.moveaxis(a, -1, 0)
    bw, bx, by, bz = np.moveaxis(b, -1, 0)
    return np.stack([
        aw * bw - ax * bx - ay * by - az * bz,
        aw * bx + ax * bw + ay * bz - az * by,
        aw * by - ax * bz + ay * bw + az * bx,
        aw * bz + ax * by - ay * bx + az * bw,
    ], axis=-1)


def conj(q):
    out = -np.asarray(q, dtype=np.float64)
    out[..., 0] = -out[..., 0]
    return out


def angle_cumsum(inc):
    """inc [b, s, h, a] -> inclusive sum over s."""
    return np.cumsum(np.asarray(inc, dtype=np.float64), axis=1)


def angle_cumsum_vjp(d_theta):
    """d_theta [b, s, h, a] -> d_inc[t] = sum_{t' >= t} d_theta[t']."""
    d = np.asarray(d_theta, dtype=np.float64)
    return np.flip(np.cumsum(np.flip(d, axis=1), axis=1), axis=1)


def quat_prefix(q):
    """q [b, s, h, J, 4] increments -> Q [b, s, h, J, 4], Q[t] = N(Q[t-1] (x) q[t])."""
    q = np.asarray(q, dtype=np.float64)
    out = np.empty_like(q)
    prev = np.zeros(q.shape[:1] + q.shape[2:])
    prev[..., 0] = 1.0
    for t in range(q.shape[1]):
        y = hamilton(prev, q[:, t])
        prev = y / np.linalg.norm(y, axis=-1, keepdims=True)
        out[:, t] = prev
    return out


def quat_prefix_vjp(q, d_Q):
    """Cotangent of the increments q [b, s, h, J, 4] given d_Q = cotangent of
    quat_prefix(q); reverse-mode through each composition and normalisation."""
    q = np.asarray(q, dtype=np.float64)
    d_Q = np.asarray(d_Q, dtype=np.float64)
    s = q.shape[1]
    # the forward values every backward step needs
    ident = np.zeros(q.shape[:1] + q.shape[2:])
    ident[..., 0] = 1.0
    Q = quat_prefix(q)
    Y = np.empty_like(q)
    for t in range(s):
        Y[:, t] = hamilton(Q[:, t - 1] if t > 0 else ident, q[:, t])
    d_q = np.empty_like(q)
    g = np.zeros_like(ident)
    for t in range(s - 1, -1, -1):
        g = g + d_Q[:, t]
        Qt = Q[:, t]
        nY = np.linalg.norm(Y[:, t], axis=-1, keepdims=True)
        dY = (g - Qt * np.sum(Qt * g, axis=-1, keepdims=True)) / nY
        Qprev = Q[:, t - 1] if t > 0 else ident
        d_q[:, t] = hamilton(conj(Qprev), dY)
        g = hamilton(dY, conj(q[:, t]))
    return d_q
