"""Pins of the k-means / cluster-order oracle (CPU).

The SVG-EAR page names the clustering only; the oracle's reading (Lloyd's
k-means from given centres, a final assignment, stable cluster order) is
pinned against scikit-learn's Lloyd k-means, against brute-force loops on tiny
inputs, against torch's bf16 rounding, and by invariants that a wrong update,
tie rule or order would break."""

import numpy as np
import pytest
import torch

from oracle import kmeans as ok


def _blobs(N, C, D, sigma, seed):
    r = np.random.default_rng(seed)
    centres = r.standard_normal((C, D)) * 3.0
    lab = r.integers(0, C, N)
    return centres[lab] + sigma * r.standard_normal((N, D)), r


@pytest.mark.parametrize("seed", range(5))
def test_lloyd_matches_scikit_learn(seed):
    from sklearn.cluster import KMeans
    x, r = _blobs(240, 6, 5, 1.5, seed)
    init = x[r.choice(len(x), 6, replace=False)]
    for iters in (1, 3, 8):
        # scikit-learn moves empty clusters elsewhere; only compare runs without any
        c = init.copy()
        empty = False
        for _ in range(iters):
            lab = ok.assign(x, c, None)
            empty |= (np.bincount(lab, minlength=6) == 0).any()
            c = ok.update(x, lab, c)
        if empty:
            continue
        lab, cen = ok.lloyd(x, init, iters, centre_dtype=None)
        km = KMeans(n_clusters=6, init=init, n_init=1, max_iter=iters, tol=0.0, algorithm="lloyd").fit(x)
        assert np.array_equal(lab, km.labels_)
        assert np.allclose(cen, km.cluster_centers_, rtol=1e-10, atol=1e-10)


def _brute(x, init, iters):
    """Squared distances by loops (not the expanded form), lowest index on ties."""
    N, D = len(x), len(x[0])
    c = [list(map(float, row)) for row in init]

    def nearest(p):
        best, bi = None, -1
        for j, cj in enumerate(c):
            d = sum((p[t] - cj[t]) ** 2 for t in range(D))
            if best is None or d < best:
                best, bi = d, j
        return bi

    for _ in range(iters):
        lab = [nearest(p) for p in x]
        for j in range(len(c)):
            mem = [x[i] for i in range(N) if lab[i] == j]
            if mem:
                c[j] = [sum(m[t] for m in mem) / len(mem) for t in range(D)]
    return [nearest(p) for p in x], c


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("centre_dtype", [None, "bf16"])
def test_brute_force_tiny(seed, centre_dtype):
    """Small integer data, centres that stay exact in bf16 (sums of few small
    integers over counts that are powers of two are not guaranteed, so the data
    are multiples of 1/2 and the check is on the first step's labels plus the
    whole run in float64 mode)."""
    r = np.random.default_rng(100 + seed)
    N, C, D = int(r.integers(3, 12)), int(r.integers(1, 5)), int(r.integers(1, 4))
    x = r.integers(-4, 5, (N, D)) / 2.0
    init = r.integers(-4, 5, (C, D)) / 2.0
    lab0 = ok.assign(x, init, centre_dtype)          # init is exact in bf16
    blab, _ = _brute(x.tolist(), init.tolist(), 0)
    assert lab0.tolist() == blab
    if centre_dtype is None:
        lab, cen = ok.lloyd(x, init, 4, None)
        blab, bcen = _brute(x.tolist(), init.tolist(), 4)
        assert lab.tolist() == blab
        assert np.allclose(cen, np.array(bcen), rtol=0, atol=1e-12)


def test_ties_go_to_the_lowest_index():
    x = np.array([[0.0, 0.0], [1.0, 0.0]])
    init = np.array([[0.5, 1.0], [0.5, -1.0], [0.5, 1.0]])   # every point equidistant to all three
    assert ok.assign(x, init).tolist() == [0, 0]


def test_empty_cluster_keeps_its_centre_and_one_cluster_is_the_mean():
    x, _ = _blobs(50, 2, 3, 0.5, 7)
    init = np.vstack([x[:1], [[1e3, 1e3, 1e3]]])
    lab, cen = ok.lloyd(x, init, 3, None)
    assert (lab == 0).all()
    assert np.array_equal(cen[1], init[1])
    assert np.allclose(cen[0], x.mean(axis=0), rtol=0, atol=1e-12)


def test_objective_never_increases():
    x, r = _blobs(400, 8, 6, 2.0, 9)
    c = x[r.choice(400, 8, replace=False)]
    prev = np.inf
    for _ in range(12):
        lab = ok.assign(x, c, None)
        sse = ((x - c[lab]) ** 2).sum()
        assert sse <= prev + 1e-9
        prev = sse
        c = ok.update(x, lab, c)


def test_token_permutation_equivariance():
    x, r = _blobs(120, 4, 3, 1.0, 11)
    init = x[:4].copy()
    sh = r.permutation(120)
    lab, cen = ok.lloyd(x, init, 5)
    lab2, cen2 = ok.lloyd(x[sh], init, 5)
    assert np.array_equal(lab2, lab[sh])
    assert np.allclose(cen2, cen, rtol=1e-12, atol=1e-12)


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(12)
    x = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-6, 6, 20000),
                        [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, 65504.0]])
    want = torch.tensor(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(ok.round_bf16(x), want)


def test_cluster_order_gather_and_scatter():
    r = np.random.default_rng(13)
    C, N = 7, 60
    lab = r.integers(0, C, N)
    lab[lab == 3] = 2                                      # an empty cluster
    perm, off = ok.cluster_order(lab, C)
    want = [i for a in range(C) for i in range(N) if lab[i] == a]
    assert perm.tolist() == want
    assert off.tolist() == [sum(1 for v in lab if v < a) for a in range(C + 1)]
    assert off[3] == off[4]
    x = r.standard_normal((N, 5))
    g = ok.gather_rows(x, perm)
    for a in range(C):
        assert (lab[perm[off[a]:off[a + 1]]] == a).all()
    assert np.array_equal(ok.scatter_rows(g, perm), x)
    assert np.array_equal(g[0], x[perm[0]])
