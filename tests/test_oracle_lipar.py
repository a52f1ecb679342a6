"""Pins of the LIPAR pruning / restoration oracle (CPU).

The LIPAR page (section 2, B. pipeline) prints no numbers for the pruning rule,
so the oracle is pinned by its special cases, by invariants that a wrong
frame, axis, comparison or chain would break, and by brute force on tiny
inputs."""

import numpy as np
import pytest

from oracle import lipar as ol


def _video(F, P, D, seed=0):
    r = np.random.default_rng(seed)
    return r.standard_normal((F * P, D))


def test_static_video_keeps_only_the_first_frame():
    F, P, D = 5, 7, 8
    x = np.tile(_video(1, P, D), (F, 1))
    for tau in (0.0, 0.5, 10.0):
        keep, idx, y = ol.prune(x, F, tau)
        assert keep.sum() == P and np.array_equal(idx, np.arange(P))
        assert np.array_equal(ol.restore(y, keep, F), x)


def test_negative_tau_keeps_everything_and_restore_is_identity():
    F, P, D = 4, 6, 5
    x = _video(F, P, D, 1)
    keep, idx, y = ol.prune(x, F, -1.0)
    assert keep.all() and np.array_equal(y, x)
    assert np.array_equal(ol.restore(y, keep, F), x)


def test_threshold_is_strict_on_the_mean_absolute_difference():
    """Frame 1 differs from frame 0 by exactly tau in mean |.| on patch 0 and by
    slightly more on patch 1 (values exact in binary)."""
    F, P, D, tau = 2, 2, 4, 0.25
    x = np.zeros((F * P, D))
    x[P + 0] = [0.25, -0.25, 0.25, -0.25]          # sum |d| = 1.0 = tau * D: not kept
    x[P + 1] = [0.25, -0.25, 0.25, -0.25 - 2**-20]  # just above: kept
    keep = ol.keep_flags(x, F, tau)
    assert keep.tolist() == [True, True, False, True]


def test_difference_is_against_the_adjacent_frame_not_frame_zero():
    """A patch that drifts by tau/2 per frame never passes against its neighbour,
    although it moves far from frame 0."""
    F, P, D, tau = 6, 1, 3, 1.0
    x = np.zeros((F, D))
    for f in range(F):
        x[f] = 0.5 * f
    keep = ol.keep_flags(x, F, tau)
    assert keep.tolist() == [True] + [False] * (F - 1)


def test_restored_tokens_copy_the_latest_kept_frame():
    F, P, D = 6, 3, 4
    x = _video(F, P, D, 2)
    # patch 1 stays within tau of its neighbour in frames 2..4
    tau = 0.3
    for f in (2, 3, 4):
        x[f * P + 1] = x[(f - 1) * P + 1] + 0.1
    keep, idx, y = ol.prune(x, F, tau)
    out = ol.restore(y, keep, F)
    assert keep.reshape(F, P)[2:5, 1].tolist() == [False, False, False]
    for f in (2, 3, 4):
        assert np.array_equal(out[f * P + 1], x[1 * P + 1])
    assert np.array_equal(out[keep], x[keep])


def test_restoration_error_obeys_the_triangle_bound():
    """sum_c |restored - x| of a pruned token (f, p) is at most (f - f0) tau D,
    f0 = the latest kept frame of p before f."""
    F, P, D, tau = 12, 9, 6, 0.6
    r = np.random.default_rng(3)
    x = np.zeros((F, P, D))
    x[0] = r.standard_normal((P, D))
    for f in range(1, F):
        step = r.choice([0.1, 1.5], size=(P, 1))            # small or large changes
        x[f] = x[f - 1] + step * r.standard_normal((P, D))
    x = x.reshape(F * P, D)
    keep, idx, y = ol.prune(x, F, tau)
    out = ol.restore(y, keep, F)
    kf = keep.reshape(F, P)
    assert 0 < keep.sum() < F * P
    for f in range(F):
        for p in range(P):
            f0 = max(g for g in range(f + 1) if kf[g, p])
            err = np.abs(out[f * P + p] - x[f * P + p]).sum()
            assert err <= (f - f0) * tau * D + 1e-9


def _brute(x, F, tau):
    N, D = x.shape
    P = N // F
    keep = []
    for f in range(F):
        for p in range(P):
            if f == 0:
                keep.append(True)
                continue
            s = 0.0
            for c in range(D):
                s += abs(float(x[f * P + p, c]) - float(x[(f - 1) * P + p, c]))
            keep.append(s > tau * D)
    kept = [n for n in range(N) if keep[n]]
    out = [None] * N
    for f in range(F):
        for p in range(P):
            n = f * P + p
            out[n] = list(x[n]) if keep[n] else list(out[n - P])
    return keep, kept, out


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    r = np.random.default_rng(10 + seed)
    F, P, D = int(r.integers(1, 6)), int(r.integers(1, 5)), int(r.integers(1, 6))
    x = np.round(r.standard_normal((F * P, D)) * 4) / 4    # coarse values: many near-equal frames
    tau = float(r.choice([0.0, 0.25, 0.5, 1.0]))
    keep, idx, y = ol.prune(x, F, tau)
    bk, bkept, bout = _brute(x, F, tau)
    assert keep.tolist() == bk and idx.tolist() == bkept
    assert np.array_equal(ol.restore(y, keep, F), np.array(bout))


def _bf16_exact(vals):
    a = np.asarray(vals, np.float64)
    assert np.array_equal(a.astype(np.float32).astype(np.float64), a)
    b = a.astype(np.float32).view(np.uint32)
    assert not (b & 0xFFFF).any(), "not a bf16 value"
    return a


def threshold_fixtures():
    """Two hand-derived one-patch cases (D = 8, two frames), each with the keep
    flag of frame 1 that the reading fixes:

    * "sum at the threshold, far exponents": frame 0 = (2^-30, 0, ...), frame 1
      = (1, 1, 2^-30, 0, ...), tau = 0.25.  Exactly, |1 - 2^-30| + 1 + 2^-30 = 2
      = tau * D, so the token is not kept (kept needs > tau * D).  A difference
      taken in float32 rounds 1 - 2^-30 to 1 and would keep it.
    * "sum between the float and double thresholds": frame 0 = 0, frame 1 =
      (204 * 2^-8, 204 * 2^-16, 204 * 2^-24, 7 * 2^-27, 0, ...), whose sum is
      107374183 * 2^-27 = 0.8000000045 (each entry is a bf16 value), tau = 0.1.
      float32(0.1) * 8 = 0.8000000119 >= the sum: not kept; the float64 value
      of 0.1 would give 0.8 < the sum and keep it."""
    a = np.zeros((2, 8))
    a[0, 0] = 2.0 ** -30
    a[1, :3] = [1.0, 1.0, 2.0 ** -30]
    b = np.zeros((2, 8))
    b[1, :4] = [204 * 2.0 ** -8, 204 * 2.0 ** -16, 204 * 2.0 ** -24, 7 * 2.0 ** -27]
    assert b[1].sum() == 107374183 * 2.0 ** -27
    return [("far exponents", _bf16_exact(a), 0.25, False), ("float tau", _bf16_exact(b), 0.1, False)]


def test_threshold_fixtures():
    for name, x, tau, kept in threshold_fixtures():
        keep = ol.keep_flags(x, 2, tau)
        assert keep[0] and keep[1] == kept, name
    # the same cases just past the threshold are kept
    _, x, _, _ = threshold_fixtures()[0]
    assert ol.keep_flags(x, 2, float(np.nextafter(np.float32(0.25), np.float32(0))))[1]
    _, x, _, _ = threshold_fixtures()[1]
    assert ol.keep_flags(x, 2, float(np.nextafter(np.float32(0.1), np.float32(0))))[1]
