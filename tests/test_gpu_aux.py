"""GPU checks of the auxiliary machinery: the environment-gated finiteness
check (MOMENTS_CHECK_FINITE) of every forward and backward entry point."""
import os

import pytest
import torch

import mamba_ssm_chunkwise_amd as M
import workloads as W
from parity_util import desc_of

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture
def check_finite():
    old = os.environ.get("MOMENTS_CHECK_FINITE")
    os.environ["MOMENTS_CHECK_FINITE"] = "1"
    yield
    if old is None:
        del os.environ["MOMENTS_CHECK_FINITE"]
    else:
        os.environ["MOMENTS_CHECK_FINITE"] = old


def _case(dtype):
    w = W.small(f"fin_{dtype}", dtype=dtype, b=2, s=96, c=2, h=3, p=24, r=40, valid_len=77,
                rot_kind=W.ROT_PAIRWISE, rope_dim=16, seed=61)
    return w, W.generate(w, device=DEV)


def _calls(w, t):
    d = desc_of(w)
    M.moments_fwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"])
    M.moments_bwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], t["d_m2"], t["d_m1"])
    _, _, sv = M.moments_fwd_save(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"])
    M.moments_bwd_saved(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], sv, t["d_m2"], t["d_m1"])
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_finite_outputs_pass(check_finite, dtype):
    w, t = _case(dtype)
    _calls(w, t)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nan_past_valid_len_is_not_reported(check_finite, dtype):
    w, t = _case(dtype)
    t["xhat"][:, w.valid_len:] = float("nan")
    t["da"][:, w.valid_len + 3:] = float("inf")
    _calls(w, t)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nan_input_is_reported(check_finite, dtype):
    w, t = _case(dtype)
    t["bhat"][1, 10, 0, 2, 5] = float("nan")
    d = desc_of(w)
    with pytest.raises(M.MomentsError) as e:
        M.moments_fwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"])
    assert e.value.code == -6
    with pytest.raises(M.MomentsError) as e:
        M.moments_bwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], t["d_m2"], t["d_m1"])
    assert e.value.code == -6


def test_off_by_default():
    assert os.environ.get("MOMENTS_CHECK_FINITE", "") in ("", "0")
    w, t = _case("f32")
    t["bhat"][1, 10, 0, 2, 5] = float("nan")
    d = desc_of(w)
    m2, _ = M.moments_fwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"])
    torch.cuda.synchronize()
    assert not torch.isfinite(m2[1]).all()
