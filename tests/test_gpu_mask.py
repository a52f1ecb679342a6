"""GPU mask builder vs the oracle: bit-exact CSR."""

import numpy as np
import pytest

from oracle import mask as om
from synth import get_workload

pytestmark = pytest.mark.gpu


def _gpu_csr(bsa, params):
    rp, ci = bsa.build_block_mask(params)
    rp = rp.cpu().numpy()
    return rp, ci[: int(rp[-1])].cpu().numpy()


def _check(bsa, params):
    spec = om.spec_from_params(params)
    want_rp, want_ci = om.to_csr(om.block_mask(spec))
    rp, ci = _gpu_csr(bsa, params)
    assert np.array_equal(rp, want_rp), params
    assert np.array_equal(ci, want_ci), params
    # with the optional row order: same CSR, plus rows by descending length (stable)
    rp2, ci2, ro = bsa.build_block_mask(params, with_order=True)
    rp2 = rp2.cpu().numpy()
    assert np.array_equal(rp2, want_rp), params
    assert np.array_equal(ci2[: int(rp2[-1])].cpu().numpy(), want_ci), params
    lens = np.diff(want_rp).astype(np.int64)
    nb = len(lens)
    is_long = (2 * lens * nb >= 3 * int(want_rp[-1])) & (lens > 0)
    long_rows = np.nonzero(is_long)[0]
    long_rows = long_rows[np.argsort(-lens[long_rows], kind="stable")]
    want_order = np.concatenate([long_rows, np.nonzero(~is_long)[0], [len(long_rows)]])
    assert np.array_equal(ro.cpu().numpy(), want_order), params


def test_tiny_lvsa(gpu_lib):
    _check(gpu_lib, get_workload("tiny_fp32").mask_params(0))


@pytest.mark.parametrize("step", [0, 1, 2, 3])
def test_lvsa_32k(gpu_lib, step):
    _check(gpu_lib, get_workload("lvsa_32k").mask_params(step))


def test_lvsa_32k_column_anchors(gpu_lib):
    p = get_workload("lvsa_32k").mask_params(5)
    p["anchor_rows"] = 0
    _check(gpu_lib, p)


def test_radial_196k(gpu_lib):
    _check(gpu_lib, get_workload("radial_196k").mask_params(0))


def test_all_kind_and_block64(gpu_lib):
    p = get_workload("lvsa_32k").mask_params(2)
    _check(gpu_lib, dict(p, block=64))
    _check(gpu_lib, dict(p, kind=0))
    _check(gpu_lib, dict(get_workload("radial_196k").mask_params(0), frames=40, block=64))


def test_random_small_specs(gpu_lib):
    r = np.random.default_rng(123)
    for _ in range(120):
        P = int(r.integers(1, 40))
        p = dict(kind=int(r.integers(0, 3)), frames=int(r.integers(1, 12)), frame_tokens=P,
                 block=int(r.choice([1, 2, 3, 4, 8, 16, 64])), window=int(r.integers(0, 4)),
                 anchor_period=int(r.integers(0, 6)), anchor_step=int(r.integers(0, 20)),
                 anchor_rows=int(r.integers(0, 2)), radial_w=int(r.integers(0, 3 * P)))
        _check(gpu_lib, p)


def test_single_block(gpu_lib):
    _check(gpu_lib, dict(kind=2, frames=1, frame_tokens=1, block=1, window=0, anchor_period=0,
                         anchor_step=0, anchor_rows=0, radial_w=0))


def test_schedule_of_lvsa_32k(gpu_lib):
    """The anchor-frame rows (all 256 blocks, about twice the mean) are the long rows."""
    p = get_workload("lvsa_32k").mask_params(0)
    rp, ci, ro = gpu_lib.build_block_mask(p, with_order=True)
    ro = ro.cpu().numpy()
    lens = np.diff(rp.cpu().numpy())
    nh = int(ro[-1])
    assert nh == int((lens == 256).sum()) > 0
    assert (lens[ro[:nh]] == 256).all() and (lens[ro[nh:-1]] < 256).all()


def test_repeatable(gpu_lib):
    p = get_workload("radial_196k").mask_params(0)
    a = _gpu_csr(gpu_lib, p)
    b = _gpu_csr(gpu_lib, p)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
