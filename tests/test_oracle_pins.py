"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own loops: each check uses an independent
route (the pages' chunkwise algebra at several chunk lengths, closed forms,
complex-number or 2x2-complex-matrix rotations, torch float64 autograd, central
finite differences, invariants). A plausible slip in the oracle (a dropped term,
a wrong sign, a transposed operand, an off-by-one in the mask) fails at least one.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import ROT_HALF, ROT_NONE, ROT_PAIRWISE, ROT_QUAT, oracle_bwd, oracle_fwd
from oracle import chunk_form as cf


def _np(t):
    return {k: (None if v is None else v.double().numpy().copy()) for k, v in t.items()}


def _case(rot_kind, r=12, p=5, c=2, s=40, valid_len=None, seed=3, rope_dim=None, quat_blocks=None,
          h=2, b=1, h0=True):
    if rope_dim is None:
        rope_dim = 8 if rot_kind in (ROT_PAIRWISE, ROT_HALF) else 0
    if quat_blocks is None:
        quat_blocks = 2 if rot_kind == ROT_QUAT else 0
    w = W.small("pin", b=b, s=s, c=c, h=h, p=p, r=r, chunk_len=8, valid_len=valid_len,
                rot_kind=rot_kind, rope_dim=rope_dim, quat_blocks=quat_blocks, seed=seed,
                h0_sd=0.3 if h0 else None)
    return w, _np(W.generate(w))


def _fwd(w, a, **kw):
    return oracle_fwd(a["xhat"], a["bhat"], a["da"], a["rot"], a["h0"], w.valid_len, w.rot_kind,
                      w.rope_dim, **kw)


def _bwd(w, a, **kw):
    return oracle_bwd(a["xhat"], a["bhat"], a["da"], a["rot"], a["h0"], a["d_m2"], a["d_m1"],
                      w.valid_len, w.rot_kind, w.rope_dim, **kw)


def _rel(x, y):
    return np.abs(x - y).max() / max(np.abs(y).max(), 1e-300)


MODES = [(ROT_PAIRWISE, 12), (ROT_HALF, 12), (ROT_QUAT, 12), (ROT_NONE, 12)]


# ---------------------------------------------------------------- chunkwise form
@pytest.mark.parametrize("rot_kind,r", MODES)
@pytest.mark.parametrize("l", [1, 2, 4, 8, 20, 40])
def test_chunk_length_invariance(rot_kind, r, l):
    """The chunkwise block form (forward and its adjoint), at any chunk length,
    equals the per-token recurrence ("backward.rs", "Gradient math": d_t and
    L[t,j] are products of exp(da) over the tokens in between)."""
    w, a = _case(rot_kind, r=r, valid_len=37)
    m2, m1 = _fwd(w, a)
    q2, q1 = cf.moments_fwd_chunked(a["xhat"], a["bhat"], a["da"], a["rot"], a["h0"], w.valid_len,
                                    w.rot_kind, w.rope_dim, l)
    assert _rel(q2, m2) < 1e-12 and _rel(q1, m1) < 1e-12
    go = _bwd(w, a)
    gp = cf.moments_bwd_chunked(a["xhat"], a["bhat"], a["da"], a["rot"], a["h0"], a["d_m2"], a["d_m1"],
                                w.valid_len, w.rot_kind, w.rope_dim, l)
    for k, v in go.items():
        if v is not None:
            assert _rel(gp[k], v) < 1e-11, k


@pytest.mark.parametrize("rot_kind,r", MODES[:3])
def test_dda_identity_brute_force(rot_kind, r):
    """"backward.rs", "Gradient math": sum_{t>=s} scal_t + sum_{j<s<=t} A[t,j]
    (brute force) equals rev_cumsum(scal + rowsum A) - rev_cumsum(colsum A), and
    the log-decay cotangent form; all equal the recurrence's exp(da_t) <dH_t, H_{t-1}>."""
    w, a = _case(rot_kind, r=r, s=24, valid_len=21)
    args = (a["xhat"], a["bhat"], a["da"], a["rot"], a["h0"], a["d_m2"], a["d_m1"], w.valid_len,
            w.rot_kind, w.rope_dim, 8)
    gi = cf.moments_bwd_chunked(*args, dda="identity")
    gd = cf.moments_bwd_chunked(*args, dda="double_sum")
    gl = cf.moments_bwd_chunked(*args, dda="log")
    go = _bwd(w, a)
    assert _rel(gi["d_da"], gd["d_da"]) < 1e-12
    assert _rel(gl["d_da"], gd["d_da"]) < 1e-12
    assert _rel(go["d_da"], gd["d_da"]) < 1e-12


CKPT_CASES = [
    dict(rot_kind=ROT_PAIRWISE, r=8, rope_dim=6),
    dict(rot_kind=ROT_HALF, r=8, rope_dim=8),
    dict(rot_kind=ROT_QUAT, r=8, quat_blocks=2),
    dict(rot_kind=ROT_NONE, r=8),
]


@pytest.mark.parametrize("kw", CKPT_CASES)
def test_backward_across_checkpoint_segments(kw):
    """The oracle's backward replays the states from checkpoints every 256 tokens:
    at V = 577 it walks three segments (the last one partial). Its gradients equal
    the block form's adjoint at l = 1, 8 and 24 (no checkpoints there), and central
    differences along random directions."""
    w, a = _case(s=600, valid_len=577, p=3, c=2, h=1, seed=9, **kw)
    go = _bwd(w, a)
    for l in (1, 8, 24):
        gp = cf.moments_bwd_chunked(a["xhat"], a["bhat"], a["da"], a["rot"], a["h0"], a["d_m2"],
                                    a["d_m1"], w.valid_len, w.rot_kind, w.rope_dim, l)
        for k, v in go.items():
            if v is not None:
                assert _rel(gp[k], v) < 1e-10, (l, k)
    rng = np.random.default_rng(13)
    eps = 1e-6
    for name in ("xhat", "bhat", "da", "rot", "h0"):
        if a[name] is None or go["d_" + name] is None:
            continue
        v = rng.standard_normal(a[name].shape)
        fd = (_objective(w, a, {name: a[name] + eps * v}) - _objective(w, a, {name: a[name] - eps * v})) / (2 * eps)
        an = (go["d_" + name] * v).sum()
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


# ---------------------------------------------------------------- rotation invariants
@pytest.mark.parametrize("rot_kind,r", MODES[:3])
def test_orthogonality_trace(rot_kind, r):
    """De-rotation is orthogonal per token (unit Q): tr(m2) = sum_t ||H_t||_F^2,
    which is tr(m2) of the same inputs without rotation. m2 is symmetric PSD."""
    w, a = _case(rot_kind, r=r, valid_len=33)
    if rot_kind == ROT_QUAT:   # the draws are float32-rounded: make them unit in fp64
        a["rot"] = a["rot"] / np.linalg.norm(a["rot"], axis=-1, keepdims=True)
    m2, _ = _fwd(w, a)
    n2, _ = oracle_fwd(a["xhat"], a["bhat"], a["da"], None, a["h0"], w.valid_len, ROT_NONE, 0)
    assert abs(np.trace(m2[0, 0]) - np.trace(n2[0, 0])) < 1e-12 * np.trace(n2[0, 0])
    for bh in np.ndindex(m2.shape[:2]):
        assert np.allclose(m2[bh], m2[bh].T, atol=1e-12)
        assert np.linalg.eigvalsh(m2[bh]).min() > -1e-10
    # coordinates outside the rope width pass through: that block equals the
    # rotation-free Gram block
    width = {ROT_PAIRWISE: 8, ROT_QUAT: 8}.get(rot_kind)
    if width is not None:
        assert _rel(m2[..., width:, width:], n2[..., width:, width:]) < 1e-12


def _derotate_complex(bv, theta, rot_kind, r):
    """De-rotation R(-theta) of one vector via complex numbers: z' = exp(-i theta) z."""
    out = bv.copy()
    a = theta.shape[-1]
    if rot_kind == ROT_PAIRWISE:
        i0, i1 = 2 * np.arange(a), 2 * np.arange(a) + 1
    else:
        i0, i1 = np.arange(a), r // 2 + np.arange(a)
    z = (bv[i0] + 1j * bv[i1]) * np.exp(-1j * theta)
    out[i0], out[i1] = z.real, z.imag
    return out


def _qmat(q):
    """Quaternion -> 2x2 complex matrix (a ring homomorphism)."""
    w, x, y, z = q
    return np.array([[w + 1j * x, y + 1j * z], [-y + 1j * z, w - 1j * x]])


def _derotate_quat(bv, Q):
    """Left product Q (x) v on 4-blocks, computed through 2x2 complex matrices."""
    out = bv.copy()
    for j in range(Q.shape[0]):
        M = _qmat(Q[j]) @ _qmat(bv[4 * j:4 * j + 4])
        out[4 * j:4 * j + 4] = [M[0, 0].real, M[0, 0].imag, M[0, 1].real, M[0, 1].imag]
    return out


def _derot(w, a, t, bi, hi, vec):
    if w.rot_kind in (ROT_PAIRWISE, ROT_HALF):
        return _derotate_complex(vec, a["rot"][bi, t, hi], w.rot_kind, w.r)
    if w.rot_kind == ROT_QUAT:
        return _derotate_quat(vec, a["rot"][bi, t, hi])
    return vec


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("rot_kind,r", MODES)
def test_closed_form_zero_injection(rot_kind, r):
    """xhat = 0: H_t = exp(a_t) h0 with a_t the inclusive cumsum of da, so
    m2 = sum_t exp(2 a_t) (h0 M_t^T)^T (h0 M_t^T) and m1 = sum_t exp(a_t) h0 M_t^T."""
    w, a = _case(rot_kind, r=r, valid_len=29)
    a["xhat"][:] = 0.0
    m2, m1 = _fwd(w, a)
    for bi, hi in np.ndindex(w.b, w.h):
        acum = np.cumsum(a["da"][bi, :, hi])
        e2 = np.zeros((w.r, w.r))
        e1 = np.zeros((w.p, w.r))
        for t in range(w.valid_len):
            C = np.stack([_derot(w, a, t, bi, hi, row) for row in a["h0"][bi, hi]]) * np.exp(acum[t])
            e2 += C.T @ C
            e1 += C
        assert _rel(m2[bi, hi], e2) < 1e-12 and _rel(m1[bi, hi], e1) < 1e-12


@pytest.mark.parametrize("rot_kind,r", MODES)
def test_closed_form_no_memory(rot_kind, r):
    """exp(da) = 0 and c = 1: H_t = xhat_t bhat_t^T, so
    m2 = sum_t ||xhat_t||^2 (M_t bhat_t)(M_t bhat_t)^T and m1 = sum_t xhat_t (M_t bhat_t)^T."""
    w, a = _case(rot_kind, r=r, c=1, valid_len=31)
    a["da"][:] = -1e4   # exp underflows to exactly 0 in fp64
    m2, m1 = _fwd(w, a)
    for bi, hi in np.ndindex(w.b, w.h):
        e2 = np.zeros((w.r, w.r))
        e1 = np.zeros((w.p, w.r))
        for t in range(w.valid_len):
            x = a["xhat"][bi, t, 0, hi]
            mb = _derot(w, a, t, bi, hi, a["bhat"][bi, t, 0, hi])
            e2 += (x @ x) * np.outer(mb, mb)
            e1 += np.outer(x, mb)
        assert _rel(m2[bi, hi], e2) < 1e-12 and _rel(m1[bi, hi], e1) < 1e-12


def test_closed_form_pure_accumulation():
    """da = 0, no rotation, h0 = 0, c = 1: H_t = X_{<=t}^T B_{<=t}, a running sum
    computed here with numpy cumsum; m2 = sum_t H_t^T H_t, m1 = sum_t H_t."""
    w, a = _case(ROT_NONE, r=9, c=1, h0=False, valid_len=40)
    a["da"][:] = 0.0
    m2, m1 = _fwd(w, a)
    for bi, hi in np.ndindex(w.b, w.h):
        outer = np.einsum("tp,tr->tpr", a["xhat"][bi, :, 0, hi], a["bhat"][bi, :, 0, hi])
        Hs = np.cumsum(outer, axis=0)
        assert _rel(m2[bi, hi], np.einsum("tpr,tpq->rq", Hs, Hs)) < 1e-12
        assert _rel(m1[bi, hi], Hs.sum(0)) < 1e-12


def test_pooled_m1_form():
    """The pages' pooled m1[b,h,r] is the per-p m1 summed over p, and the pooled
    cotangent is the per-p cotangent broadcast over p (moments_phys_bwd adds
    d_m1 expanded over per_head_dim)."""
    w, a = _case(ROT_PAIRWISE)
    _, m1 = _fwd(w, a)
    q2, q1 = cf.moments_fwd_chunked(a["xhat"], a["bhat"], a["da"], a["rot"], a["h0"], w.valid_len,
                                    w.rot_kind, w.rope_dim, 8)
    assert _rel(m1.sum(2), q1.sum(2)) < 1e-12
    pooled = np.random.default_rng(0).standard_normal((w.b, w.h, w.r))
    a["d_m1"] = np.broadcast_to(pooled[:, :, None, :], a["d_m1"].shape).copy()
    g = _bwd(w, a)
    # f = <d_m2, m2> + <pooled, m1.sum(p)>: check against a finite difference in h0
    v = np.random.default_rng(1).standard_normal(a["h0"].shape)
    eps = 1e-6

    def f(h0):
        m2_, m1_ = oracle_fwd(a["xhat"], a["bhat"], a["da"], a["rot"], h0, w.valid_len, w.rot_kind,
                              w.rope_dim)
        return (a["d_m2"] * m2_).sum() + (pooled * m1_.sum(2)).sum()
    fd = (f(a["h0"] + eps * v) - f(a["h0"] - eps * v)) / (2 * eps)
    assert abs(fd - (g["d_h0"] * v).sum()) < 1e-7 * max(1.0, abs(fd))


# ---------------------------------------------------------------- gradients
def _objective(w, a, over=None):
    b = dict(a)
    if over:
        b.update(over)
    m2, m1 = oracle_fwd(b["xhat"], b["bhat"], b["da"], b["rot"], b["h0"], w.valid_len, w.rot_kind,
                        w.rope_dim)
    return (a["d_m2"] * m2).sum() + (a["d_m1"] * m1).sum()


FD_CASES = [
    dict(rot_kind=ROT_PAIRWISE, r=8, c=2),
    dict(rot_kind=ROT_HALF, r=10, rope_dim=6, c=2),
    dict(rot_kind=ROT_QUAT, r=8, c=1),
    dict(rot_kind=ROT_QUAT, r=10, c=2, quat_blocks=2),
    dict(rot_kind=ROT_NONE, r=7, c=3),
]


@pytest.mark.parametrize("kw", FD_CASES)
@pytest.mark.parametrize("nonunit", [False, True])
def test_finite_differences(kw, nonunit):
    """Central differences (fp64, step 1e-6) of f = <d_m2,m2> + <d_m1,m1> along a
    random direction, for every input, equal <grad, direction>. With non-unit
    quaternions the analytic VJP must stay exact (backward.rs: "exact for all
    quaternions")."""
    if nonunit and kw["rot_kind"] != ROT_QUAT:
        pytest.skip("non-unit only applies to quaternions")
    w, a = _case(s=20, valid_len=17, p=4, **kw)
    if nonunit:
        a["rot"] = a["rot"] * np.random.default_rng(5).uniform(0.5, 1.7, a["rot"].shape[:-1] + (1,))
    g = _bwd(w, a)
    rng = np.random.default_rng(11)
    eps = 1e-6
    for name, gname in [("xhat", "d_xhat"), ("bhat", "d_bhat"), ("da", "d_da"), ("rot", "d_rot"),
                        ("h0", "d_h0")]:
        if a[name] is None or g[gname] is None:
            continue
        v = rng.standard_normal(a[name].shape)
        fp = _objective(w, a, {name: a[name] + eps * v})
        fm = _objective(w, a, {name: a[name] - eps * v})
        fd = (fp - fm) / (2 * eps)
        an = (g[gname] * v).sum()
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def _torch_loop(w, t):
    """Direct per-token loop in torch float64 with rotation matrices built from
    cos/sin or the Hamilton left-product matrix; used with torch autograd."""
    b, s, c, h, p = t["xhat"].shape
    r = t["bhat"].shape[-1]
    V = min(w.valid_len, s)
    m2 = torch.zeros(b, h, r, r, dtype=torch.float64)
    m1 = torch.zeros(b, h, p, r, dtype=torch.float64)
    for bi in range(b):
        for hi in range(h):
            H = t["h0"][bi, hi] if t["h0"] is not None else torch.zeros(p, r, dtype=torch.float64)
            for ti in range(V):
                H = torch.exp(t["da"][bi, ti, hi]) * H + torch.einsum(
                    "cp,cr->pr", t["xhat"][bi, ti, :, hi], t["bhat"][bi, ti, :, hi])
                M = torch.eye(r, dtype=torch.float64)
                if w.rot_kind in (ROT_PAIRWISE, ROT_HALF):
                    th = t["rot"][bi, ti, hi]

                    def E(i, j):
                        e = torch.zeros(r, r, dtype=torch.float64)
                        e[i, j] = 1.0
                        return e
                    for i in range(w.rope_dim // 2):
                        u, v = (2 * i, 2 * i + 1) if w.rot_kind == ROT_PAIRWISE else (i, r // 2 + i)
                        cs, sn = torch.cos(th[i]), torch.sin(th[i])
                        M = (M - E(u, u) - E(v, v) + cs * E(u, u) + sn * E(u, v) - sn * E(v, u)
                             + cs * E(v, v))
                elif w.rot_kind == ROT_QUAT:
                    blocks = []
                    for j in range(w.quat_blocks):
                        q = t["rot"][bi, ti, hi, j]
                        wq, x, y, z = q[0], q[1], q[2], q[3]
                        blocks.append(torch.stack([torch.stack([wq, -x, -y, -z]),
                                                   torch.stack([x, wq, -z, y]),
                                                   torch.stack([y, z, wq, -x]),
                                                   torch.stack([z, -y, x, wq])]))
                    rest = r - 4 * w.quat_blocks
                    if rest:
                        blocks.append(torch.eye(rest, dtype=torch.float64))
                    M = torch.block_diag(*blocks)
                C = H @ M.T
                m2[bi, hi] = m2[bi, hi] + C.T @ C
                m1[bi, hi] = m1[bi, hi] + C
    return m2, m1


@pytest.mark.parametrize("kw", FD_CASES[:4])
def test_torch_autograd(kw):
    """torch float64 autograd of a direct loop (a library routine, independent of
    both hand-written backwards) matches every oracle gradient."""
    w, a = _case(s=12, valid_len=10, p=3, h=1, **kw)
    g = _bwd(w, a)
    t = {k: (None if v is None else torch.tensor(v, requires_grad=k in
                                                 ("xhat", "bhat", "da", "rot", "h0")))
         for k, v in a.items()}
    m2, m1 = _torch_loop(w, t)
    ((t["d_m2"] * m2).sum() + (t["d_m1"] * m1).sum()).backward()
    for name in ("xhat", "bhat", "da", "rot", "h0"):
        assert _rel(g["d_" + name], t[name].grad.numpy()) < 1e-12, name


# ---------------------------------------------------------------- masking and structure
@pytest.mark.parametrize("rot_kind,r", MODES[:3])
def test_valid_len_masking(rot_kind, r):
    """Gradients at t >= valid_len are exactly zero; outputs and gradients do not
    depend on inputs at t >= valid_len (chunk_mask; skipped chunks are never
    entered)."""
    w, a = _case(rot_kind, r=r, valid_len=23)
    m2, m1 = _fwd(w, a)
    g = _bwd(w, a)
    for k in ("d_xhat", "d_bhat", "d_da", "d_rot"):
        assert np.all(g[k][:, 23:] == 0.0), k
    rng = np.random.default_rng(2)
    b = dict(a)
    for k in ("xhat", "bhat", "da", "rot"):
        b[k] = a[k].copy()
        b[k][:, 23:] = rng.standard_normal(b[k][:, 23:].shape)
    n2, n1 = _fwd(w, b)
    gb = _bwd(w, b)
    assert np.array_equal(n2, m2) and np.array_equal(n1, m1)
    for k in g:
        if g[k] is not None:
            assert np.array_equal(g[k], gb[k]), k


def test_valid_len_zero_and_overlong():
    w, a = _case(ROT_PAIRWISE, valid_len=0)
    m2, m1 = _fwd(w, a)
    g = _bwd(w, a)
    assert not m2.any() and not m1.any()
    assert all(not v.any() for v in g.values() if v is not None)
    w2, a2 = _case(ROT_PAIRWISE, valid_len=40)
    w3 = w2.replace(valid_len=10 ** 6)
    assert np.array_equal(_fwd(w2, a2)[0], _fwd(w3, a2)[0])


def test_dm2_only_symmetric_part_and_linearity():
    """Only d_m2 + d_m2^T enters (moments_phys_bwd forms d_m2 + d_m2^T); the
    gradients are linear in (d_m2, d_m1)."""
    w, a = _case(ROT_QUAT, r=8)
    g0 = _bwd(w, a)
    K = np.random.default_rng(4).standard_normal(a["d_m2"].shape)
    b = dict(a)
    b["d_m2"] = a["d_m2"] + K - np.swapaxes(K, -1, -2)
    g1 = _bwd(w, b)
    for k in g0:
        assert _rel(g1[k], g0[k]) < 1e-12, k
    c = dict(a)
    c["d_m2"], c["d_m1"] = 2.5 * a["d_m2"], 2.5 * a["d_m1"]
    g2 = _bwd(w, c)
    for k in g0:
        assert _rel(g2[k], 2.5 * g0[k]) < 1e-12, k


def test_chain_subset_and_row_groups():
    """Computing a subset of chains, or splitting rows over threads, changes
    nothing but summation order."""
    w, a = _case(ROT_HALF, b=2, h=3, p=6)
    m2, m1 = _fwd(w, a, npg=1, nthreads=1)
    s2, s1 = _fwd(w, a, chains=[4, 1], npg=3, nthreads=4)
    for ch in (1, 4):
        bi, hi = divmod(ch, w.h)
        assert _rel(s2[bi, hi], m2[bi, hi]) < 1e-13 and _rel(s1[bi, hi], m1[bi, hi]) < 1e-13
    g = _bwd(w, a, npg=1, nthreads=1)
    gs = _bwd(w, a, chains=[4], npg=6, nthreads=3)
    for k in g:
        assert _rel(_pick(gs[k], k, 1, 1), _pick(g[k], k, 1, 1)) < 1e-12, k


def _pick(x, name, bi, hi):
    if name in ("d_xhat", "d_bhat"):
        return x[bi, :, :, hi]
    if name == "d_h0":
        return x[bi, hi]
    return x[bi, :, hi]
