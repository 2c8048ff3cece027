"""Pins of the rotation-sequence producer and its VJP (CPU oracle, not GPU).

The producer composes per-token increments into the cumulative rotation the
moments path takes ("recalculated.rs" page, ``RotPrim``: cumulative angles or
cumulative unit quaternions; ``quat_mul_prim``: the Hamilton product). Each pin
takes a route of its own: scipy's rotation composition, products of 4x4
left-multiplication matrices, a closed form for increments about one axis,
central differences, the scale invariance of a normalised product, and the
gradient of the whole moments objective with respect to the increments.
"""
import numpy as np
import pytest
from scipy.spatial.transform import Rotation

import workloads as W
from oracle import ROT_PAIRWISE, ROT_QUAT, oracle_bwd, oracle_fwd
from oracle import rotation_seq as rs


def _rand_quats(shape, seed, scale=(0.5, 1.7)):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=shape + (4,))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    return q * rng.uniform(*scale, size=shape + (1,))


def _rel(x, y):
    return np.abs(x - y).max() / max(np.abs(y).max(), 1e-300)


def test_quat_prefix_matches_scipy_composition():
    """Q[t] is the rotation q[0] then ... composed as scipy composes (r0 * r1 * ...
    is the Hamilton product q0 (x) q1 (x) ...), up to the sign of the quaternion."""
    q = _rand_quats((2, 9, 3, 2), seed=1, scale=(1.0, 1.0))
    Q = rs.quat_prefix(q)
    for bi in range(2):
        for hi in range(3):
            for j in range(2):
                acc = None
                for t in range(9):
                    w, x, y, z = q[bi, t, hi, j]
                    rt = Rotation.from_quat([x, y, z, w])
                    acc = rt if acc is None else acc * rt
                    x, y, z, w = acc.as_quat(canonical=False)
                    ref = np.array([w, x, y, z])
                    got = Q[bi, t, hi, j]
                    sign = 1.0 if np.dot(ref, got) >= 0 else -1.0
                    assert np.abs(got - sign * ref).max() < 1e-12


def _left_matrix(q):
    w, x, y, z = q
    return np.array([[w, -x, -y, -z], [x, w, -z, y], [y, z, w, -x], [z, -y, x, w]])


def test_quat_prefix_is_normalised_matrix_product():
    """Non-unit increments: Q[t] = P / |P| with P = L(q0) L(q1) ... L(qt) e_w,
    L(q) the 4x4 matrix of v -> q (x) v (so the order q0 (x) q1 (x) ... is fixed)."""
    q = _rand_quats((1, 11, 2, 3), seed=2)
    Q = rs.quat_prefix(q)
    for hi in range(2):
        for j in range(3):
            M = np.eye(4)
            for t in range(11):
                M = M @ _left_matrix(q[0, t, hi, j])
                P = M[:, 0]
                assert np.abs(Q[0, t, hi, j] - P / np.linalg.norm(P)).max() < 1e-12


def test_quat_prefix_coaxial_closed_form():
    """Increments about one fixed axis n compose to (cos(S/2), sin(S/2) n) with S
    the running sum of their angles, whatever their norms."""
    rng = np.random.default_rng(3)
    s, J = 40, 3
    n = rng.normal(size=(J, 3))
    n /= np.linalg.norm(n, axis=-1, keepdims=True)
    phi = rng.uniform(-0.4, 0.4, size=(s, J))
    scale = rng.uniform(0.3, 2.0, size=(s, J, 1))
    q = np.concatenate([np.cos(phi / 2)[..., None], np.sin(phi / 2)[..., None] * n], axis=-1) * scale
    Q = rs.quat_prefix(q[None, :, None])[0, :, 0]
    S = np.cumsum(phi, axis=0)
    ref = np.concatenate([np.cos(S / 2)[..., None], np.sin(S / 2)[..., None] * n], axis=-1)
    assert np.abs(Q - ref).max() < 1e-12


def test_angle_cumsum_closed_forms():
    inc = np.full((1, 7, 1, 2), 0.25)
    assert np.allclose(rs.angle_cumsum(inc)[0, :, 0, 0], 0.25 * np.arange(1, 8))
    d = np.zeros((1, 7, 1, 2))
    d[0, 4, 0, 1] = 1.0
    # a unit cotangent at t=4 reaches every increment at t <= 4
    assert np.array_equal(rs.angle_cumsum_vjp(d)[0, :, 0, 1], [1, 1, 1, 1, 1, 0, 0])


def _fd(f, x, eps=1e-6):
    g = np.zeros_like(x)
    flat, gf = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + eps
        fp = f(x)
        flat[i] = old - eps
        fm = f(x)
        flat[i] = old
        gf[i] = (fp - fm) / (2 * eps)
    return g


def test_angle_vjp_finite_differences():
    rng = np.random.default_rng(4)
    inc = rng.uniform(-0.3, 0.3, size=(2, 6, 2, 3))
    d = rng.normal(size=inc.shape)
    g = _fd(lambda x: np.sum(d * rs.angle_cumsum(x)), inc.copy())
    assert _rel(rs.angle_cumsum_vjp(d), g) < 1e-8


@pytest.mark.parametrize("unit", [True, False])
def test_quat_vjp_finite_differences(unit):
    q = _rand_quats((1, 7, 2, 2), seed=5, scale=(1.0, 1.0) if unit else (0.5, 1.7))
    d = np.random.default_rng(6).normal(size=q.shape)
    g = _fd(lambda x: np.sum(d * rs.quat_prefix(x)), q.copy())
    assert _rel(rs.quat_prefix_vjp(q, d), g) < 1e-7


def test_quat_vjp_scale_invariance():
    """Q does not change when one increment is rescaled, so its gradient is
    orthogonal to that increment: <d_q[t], q[t]> = 0 for every t."""
    q = _rand_quats((2, 25, 2, 3), seed=7)
    d = np.random.default_rng(8).normal(size=q.shape)
    dq = rs.quat_prefix_vjp(q, d)
    dots = np.sum(dq * q, axis=-1)
    assert np.abs(dots).max() < 1e-12 * np.abs(dq).max() * 10


@pytest.mark.parametrize("rot_kind", [ROT_PAIRWISE, ROT_QUAT])
def test_moments_gradient_through_producer(rot_kind):
    """d/d(increments) of <d_m2, m2> + <d_m1, m1> with the moments' rotation
    composed by the producer: the oracle's cumulative-rotation gradient pushed
    through the producer's VJP equals central differences of the whole objective."""
    w = W.small("prod", b=1, s=10, c=1, h=1, p=3, r=8, rot_kind=rot_kind,
                rope_dim=8 if rot_kind == ROT_PAIRWISE else 0,
                quat_blocks=2 if rot_kind == ROT_QUAT else 0, valid_len=9, seed=11)
    a = {k: (None if v is None else v.double().numpy().copy())
         for k, v in W.generate(w, increments=True).items()}
    inc = a["rot_inc"]
    if rot_kind == ROT_QUAT:
        inc = inc * np.random.default_rng(12).uniform(0.7, 1.3, size=inc.shape[:-1] + (1,))
        make = rs.quat_prefix
    else:
        make = rs.angle_cumsum

    def objective(x):
        m2, m1 = oracle_fwd(a["xhat"], a["bhat"], a["da"], make(x), a["h0"], w.valid_len, rot_kind,
                            w.rope_dim)
        return np.sum(a["d_m2"] * m2) + np.sum(a["d_m1"] * m1)

    g = oracle_bwd(a["xhat"], a["bhat"], a["da"], make(inc), a["h0"], a["d_m2"], a["d_m1"],
                   w.valid_len, rot_kind, w.rope_dim)
    d_cum = g["d_rot"]
    got = rs.quat_prefix_vjp(inc, d_cum) if rot_kind == ROT_QUAT else rs.angle_cumsum_vjp(d_cum)
    ref = _fd(objective, inc.copy())
    assert _rel(got, ref) < 1e-6


def test_generator_composition_agrees():
    """The input generator's doubling product (a different algorithm, only used to
    prepare the moments path's cumulative input) agrees with the producer."""
    w = W.small("gen", b=2, s=37, h=3, r=16, rot_kind=ROT_QUAT, rope_dim=0, quat_blocks=2, seed=13)
    t = W.generate(w, increments=True)
    Q = rs.quat_prefix(t["rot_inc"].double().numpy())
    assert np.abs(Q - t["rot"].double().numpy()).max() < 1e-6
    w = W.small("gen", b=2, s=37, h=3, r=16, rot_kind=ROT_PAIRWISE, rope_dim=8, seed=14)
    t = W.generate(w, increments=True)
    assert np.abs(rs.angle_cumsum(t["rot_inc"].double().numpy()) - t["rot"].double().numpy()).max() < 1e-5
