"""The host-side block-CSR checker (bsa_check_csr, also run on device outputs
under BSA_DEBUG) against the oracle's masks and routes, and against corrupted
copies of them (CPU only: the checker reads host arrays)."""

import os

import numpy as np
import pytest

import block_sparse_spatiotemporal_build_amd as bsa
from oracle import mask as om
from oracle import svg_ear as oe
from synth import gen, get_workload


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bsa.LIB_PATH):
        pytest.fail("libbsa.so is not built (run __graft_entry__.build())")
    return bsa.load()


def _mask_csrs():
    out = []
    wl = get_workload("lvsa_32k")
    for s in wl.anchor_steps:
        out.append((f"lvsa step {s}", om.to_csr(om.block_mask(om.spec_from_params(wl.mask_params(s))))))
    rad = get_workload("radial_196k")
    out.append(("radial 196k", om.to_csr(om.block_mask(om.spec_from_params(rad.mask_params(0))))))
    return out


def test_oracle_masks_pass(lib):
    for name, (rp, ci) in _mask_csrs():
        nb = rp.size - 1
        bsa.check_csr(rp, ci, nb, nb)


def test_oracle_routes_pass(lib):
    # a small clustered case: every head's route CSR at several densities
    rng = np.random.default_rng(5)
    Cq, Ck, N = 7, 11, 400
    nq = np.diff(np.sort(np.concatenate([[0, N], rng.choice(np.arange(1, N), Cq - 1, replace=False)])))
    nk = np.diff(np.sort(np.concatenate([[0, N], rng.choice(np.arange(1, N), Ck - 1, replace=False)])))
    nk[3] = 0  # an empty key cluster
    score = rng.random((Cq, Ck)) ** 3
    for ppm in (0, 10000, 150000, 600000, 1000000):
        rp, col, kept = oe.select_route(score, nq, nk, int(nk.sum()), ppm)
        bsa.check_csr(rp, col, Cq, Ck)
        assert int(rp[-1]) == int(kept.sum())


def _valid():
    rp, ci = om.to_csr(om.block_mask(om.spec_from_params(get_workload("lvsa_32k").mask_params(1))))
    return rp.astype(np.int32), ci.astype(np.int32), rp.size - 1


def test_corruptions_are_named(lib):
    rp, ci, nb = _valid()
    row = 5
    a, b = int(rp[row]), int(rp[row + 1])
    assert b - a >= 2
    # columns out of order within a row
    c = ci.copy()
    c[a], c[a + 1] = c[a + 1], c[a]
    with pytest.raises(bsa.BsaError, match="not strictly ascending"):
        bsa.check_csr(rp, c, nb, nb)
    # a repeated column
    c = ci.copy()
    c[a + 1] = c[a]
    with pytest.raises(bsa.BsaError, match="not strictly ascending"):
        bsa.check_csr(rp, c, nb, nb)
    # a column past the last block
    c = ci.copy()
    c[b - 1] = nb
    with pytest.raises(bsa.BsaError, match="outside"):
        bsa.check_csr(rp, c, nb, nb)
    c[b - 1] = -1
    with pytest.raises(bsa.BsaError, match="outside"):
        bsa.check_csr(rp, c, nb, nb)
    # row_ptr not monotone, not starting at 0, past the capacity
    r = rp.copy()
    r[row + 1] = r[row] - 1
    with pytest.raises(bsa.BsaError, match="decreases"):
        bsa.check_csr(r, ci, nb, nb)
    r = rp.copy()
    r[0] = 1
    with pytest.raises(bsa.BsaError, match="not 0"):
        bsa.check_csr(r, ci, nb, nb)
    with pytest.raises(bsa.BsaError, match="capacity"):
        bsa.check_csr(rp, ci, nb, nb, capacity=int(rp[-1]) - 1)


def test_empty_rows_and_empty_csr(lib):
    bsa.check_csr(np.zeros(4, np.int32), np.zeros(0, np.int32), 3, 5, 0)
    bsa.check_csr(np.array([0, 0, 2, 2], np.int32), np.array([1, 4], np.int32), 3, 5)
