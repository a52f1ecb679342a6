"""GPU token clustering (k-means, cluster order, row gather / scatter) vs the oracle.

Labels are integers decided by float distances.  They are checked against the
textbook algorithm (``oracle.kmeans`` with ``centre_dtype=None``: squared
Euclidean distances in float64 to float64 centres, the form pinned against
scikit-learn).  The device takes the decision with the centres rounded to bf16
and fp32 accumulation; ``_check_valid`` bounds what that rounding can change.
Where the textbook nearest centre is unique by more than twice that bound the
labels must equal it; everywhere they must be a textbook nearest centre
within it.  Where the data are well separated, whole Lloyd runs must equal the
textbook run exactly.  Ten Lloyd steps on overlapping clusters amplify single
near-tie decisions, so there the final labels are checked for validity, the
k-means objective against the textbook run's, and (a secondary check) the
labels against the oracle run that takes its decisions at the device's
precision (``centre_dtype="bf16"``).  The cluster order and the row copies are
bit-exact."""

import numpy as np
import pytest
import torch

from helpers import to_device
from oracle import kmeans as ok
from synth import gen, get_workload

pytestmark = pytest.mark.gpu


def _rounding_bound(x, cent):
    """[N, C]: a bound on |device distance - textbook distance| per (token,
    centre).  Rounding a centre to bf16 moves each coordinate by at most 2^-8
    of itself, which moves |c|^2 - 2 x.c by at most 2^-7 (|c|^2 (1 + 2^-8) +
    sum |x_i c_i|); fp32 accumulation adds at most 1e-5 (|c|^2 + 2 sum |x_i c_i|)."""
    c2 = (cent * cent).sum(1)[None, :]
    xc = np.abs(x) @ np.abs(cent).T
    return 2.0 ** -7 * (c2 * (1 + 2.0 ** -8) + xc) + 1e-5 * (c2 + 2.0 * xc)


def _check_valid(x, labels, cent):
    """Each label's textbook distance interval (distance +- its bound) reaches
    below every other centre's interval top, and where the textbook nearest
    centre's interval lies below every other interval the label is exactly
    that centre.  Returns the share of tokens with such a unique answer."""
    cent = np.asarray(cent, np.float64)
    d = (cent * cent).sum(1)[None, :] - 2.0 * (x @ cent.T)
    eps = _rounding_bound(x, cent)
    rows = np.arange(len(x))
    assert (d[rows, labels] - eps[rows, labels] <= (d + eps).min(axis=1)).all()
    best = d.argmin(axis=1)
    lo = d - eps
    lo[rows, best] = np.inf
    clear = d[rows, best] + eps[rows, best] < lo.min(axis=1) if d.shape[1] > 1 else np.ones(len(x), bool)
    assert np.array_equal(labels[clear], best[clear])
    return clear.mean()


def _objective(x, labels, cent):
    return float(((x - cent[labels]) ** 2).sum())


def _tokens(B, H, N, C, sigma, seed):
    r = np.random.default_rng(seed)
    cen = r.standard_normal((B * H, C, 128))
    cen /= np.linalg.norm(cen, axis=2, keepdims=True)
    lab = r.integers(0, C, (B * H, N))
    x = np.stack([cen[i][lab[i]] for i in range(B * H)]) + sigma * r.standard_normal((B * H, N, 128))
    bits = gen.store(x.reshape(B, H, N, 128).astype(np.float32), "bf16")
    init = (cen + 0.05 * r.standard_normal(cen.shape) / np.sqrt(128)).astype(np.float32)
    return bits, init


# (20000, 600): one tile group of 79 tiles per cluster in the scan (C > 512)
@pytest.mark.parametrize("N,C,iters", [(3000, 37, 5), (257, 32, 3), (700, 100, 0), (1000, 500, 4), (20000, 600, 2)])
def test_well_separated_matches_oracle(gpu_lib, N, C, iters):
    B, H = 1, 3
    bits, init = _tokens(B, H, N, C, 0.05, N + C)
    x = to_device(bits, "bf16")
    labels, cent, perm, off = gpu_lib.kmeans(x, C, iters, torch.from_numpy(init))
    torch.cuda.synchronize()
    lab_h, cent_h, perm_h, off_h = (t.cpu().numpy() for t in (labels, cent, perm, off))
    for r in range(B * H):
        xf = gen.to_f64(bits[0, r], "bf16")
        rl, rc = ok.lloyd(xf, init[r].astype(np.float64), iters, centre_dtype=None)
        assert np.array_equal(lab_h[r], rl), r
        assert np.abs(cent_h[r] - rc).max() < 1e-5
        p, o = ok.cluster_order(lab_h[r], C)
        assert np.array_equal(perm_h[r], p) and np.array_equal(off_h[r], o)


def test_empty_and_single_clusters(gpu_lib):
    N = 900
    bits, init = _tokens(1, 2, N, 4, 0.05, 5)
    far = np.full((2, 3, 128), 50.0, np.float32)
    init6 = np.concatenate([init, far], axis=1)                   # clusters 4..6 never win
    x = to_device(bits, "bf16")
    labels, cent, perm, off = gpu_lib.kmeans(x, 7, 3, torch.from_numpy(init6))
    torch.cuda.synchronize()
    c = cent.cpu().numpy()
    assert np.array_equal(c[:, 4:], init6[:, 4:])
    o = off.cpu().numpy()
    assert (o[:, 4] == N).all() and (o[:, 7] == N).all()
    labels1, cent1, _, off1 = gpu_lib.kmeans(x, 1, 2, torch.from_numpy(init[:, :1].copy()))
    torch.cuda.synchronize()
    assert (labels1.cpu().numpy() == 0).all()
    for r in range(2):
        mean = gen.to_f64(bits[0, r], "bf16").mean(axis=0)
        assert np.abs(cent1.cpu().numpy()[r, 0] - mean).max() < 1e-5


def test_assignment_and_update_steps_on_overlapping_clusters(gpu_lib):
    """The SVG-EAR mixture (sigma 0.3 around unit centres, 32,760 tokens, 500 key
    clusters): zero steps = one assignment to the initial centres; one step's
    centres = the means of that assignment."""
    wl = gen.scaled(get_workload("svg_ear_32k"), H=2)
    d = gen.make_gmm_tokens(wl)
    x = to_device(d["k"], "bf16")
    init = torch.from_numpy(d["centres_k"])
    lab0, cent0, _, _ = gpu_lib.kmeans(x, wl.n_k_clusters, 0, init)
    lab1, cent1, perm1, off1 = gpu_lib.kmeans(x, wl.n_k_clusters, 1, init)
    torch.cuda.synchronize()
    for r in range(2):
        xf = gen.to_f64(d["k"][0, r], "bf16")
        l0 = lab0.cpu().numpy()[r]
        assert np.array_equal(cent0.cpu().numpy()[r], d["centres_k"][r])
        assert _check_valid(xf, l0, d["centres_k"][r].astype(np.float64)) > 0.8
        want = ok.update(xf, l0, d["centres_k"][r].astype(np.float64))
        assert np.abs(cent1.cpu().numpy()[r] - want).max() < 1e-5
        l1 = lab1.cpu().numpy()[r]
        _check_valid(xf, l1, cent1.cpu().numpy()[r].astype(np.float64))
        p, o = ok.cluster_order(l1, wl.n_k_clusters)
        assert np.array_equal(perm1.cpu().numpy()[r], p) and np.array_equal(off1.cpu().numpy()[r], o)


@pytest.mark.parametrize("which", ["q", "k"])
def test_svg_ear_32k_ten_steps(gpu_lib, which):
    """Ten Lloyd steps on the 32,760-token workload as the benchmark launches
    them (all 12 heads; queries: 100 clusters, keys: 500): for heads 0 and 7,
    valid final labels for the final centres (textbook distances), the exact
    cluster order, a k-means objective within 1e-4 of the textbook run from
    the same centres, and label agreement with the textbook run and (closer)
    with the oracle run that decides at the device's precision."""
    wl = get_workload("svg_ear_32k")
    d = gen.make_gmm_tokens(wl)
    C = wl.n_q_clusters if which == "q" else wl.n_k_clusters
    x = to_device(d[which], "bf16")
    init = d["centres_" + which]
    labels, cent, perm, off = gpu_lib.kmeans(x, C, wl.kmeans_iters, torch.from_numpy(init))
    torch.cuda.synchronize()
    for r in (0, 7):
        xf = gen.to_f64(d[which][0, r], "bf16")
        lab = labels.cpu().numpy()[r]
        cen = cent.cpu().numpy()[r].astype(np.float64)
        _check_valid(xf, lab, cen)
        p, o = ok.cluster_order(lab, C)
        assert np.array_equal(perm.cpu().numpy()[r], p) and np.array_equal(off.cpu().numpy()[r], o)
        tl, tc = ok.lloyd(xf, init[r].astype(np.float64), wl.kmeans_iters, centre_dtype=None)
        assert _objective(xf, lab, cen) <= _objective(xf, tl, tc) * (1 + 1e-4)
        assert (tl == lab).mean() > 0.95
        rl, rc = ok.lloyd(xf, init[r].astype(np.float64), wl.kmeans_iters, centre_dtype="bf16")
        assert (rl == lab).mean() > 0.999
        assert np.abs(rc - cen).max() < 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gather_scatter_roundtrip(gpu_lib, dtype):
    B, H, N, D = 2, 3, 1001, 128 if dtype == "bf16" else 64
    r = np.random.default_rng(20)
    x = r.standard_normal((B, N, H, D)).astype(np.float32)          # stored [B, N, H, D]
    stored = gen.store(x, dtype)
    dev = to_device(stored, dtype).permute(0, 2, 1, 3)              # a strided [B, H, N, D] view
    perm = np.stack([r.permutation(N) for _ in range(B * H)]).astype(np.int32)
    pt = torch.from_numpy(perm).cuda()
    g = gpu_lib.gather_rows(dev, pt)
    back = gpu_lib.scatter_rows(g, pt)
    torch.cuda.synchronize()
    ref = gen.to_f64(np.ascontiguousarray(stored.transpose(0, 2, 1, 3)), dtype).reshape(B * H, N, D)
    gh = g.float().cpu().numpy().reshape(B * H, N, D)
    for i in range(B * H):
        assert np.array_equal(gh[i], ok.gather_rows(ref[i], perm[i]))
    assert torch.equal(back.view(torch.int16 if dtype == "bf16" else torch.int32),
                       dev.view(torch.int16 if dtype == "bf16" else torch.int32))


def test_gather_skips_out_of_range_entries(gpu_lib):
    x = torch.randn(1, 1, 10, 128, device="cuda").to(torch.bfloat16)
    perm = torch.tensor([[3, -1, 10, 0, 1, 2, 4, 5, 6, 7]], dtype=torch.int32, device="cuda")
    out = torch.full_like(x, 7.0)
    gpu_lib.gather_rows(x, perm, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out[0, 0, 0], x[0, 0, 3])
    assert (out[0, 0, 1:3].float() == 7.0).all()
    assert torch.equal(out[0, 0, 3:], x[0, 0, [0, 1, 2, 4, 5, 6, 7]])


def test_batch_of_sequences(gpu_lib):
    """B = 2 sequences of 2 heads each: every (batch, head) clusters on its own."""
    B, H, N, C = 2, 2, 700, 20
    bits, init = _tokens(B, H, N, C, 0.05, 77)
    x = to_device(bits, "bf16")
    labels, cent, perm, off = gpu_lib.kmeans(x, C, 3, torch.from_numpy(init))
    torch.cuda.synchronize()
    for r in range(B * H):
        b, h = divmod(r, H)
        xf = gen.to_f64(bits[b, h], "bf16")
        rl, rc = ok.lloyd(xf, init[r].astype(np.float64), 3, centre_dtype=None)
        assert np.array_equal(labels.cpu().numpy()[r], rl), r
        assert np.abs(cent.cpu().numpy()[r] - rc).max() < 1e-5


def test_order_outputs_are_optional(gpu_lib):
    """perm / offsets may be NULL: labels and centres are those of the full call."""
    import ctypes
    bits, init = _tokens(1, 2, 1500, 30, 0.05, 78)
    x = to_device(bits, "bf16")
    labels, cent, _, _ = gpu_lib.kmeans(x, 30, 3, torch.from_numpy(init))
    lib = gpu_lib.load()
    c2 = torch.from_numpy(init).cuda().contiguous().clone()
    l2 = torch.empty_like(labels)
    ws = torch.empty(gpu_lib.kmeans_workspace(x, 30), dtype=torch.uint8, device="cuda")
    st = lib.bsa_kmeans(gpu_lib._ptr(x), 0, ctypes.byref(gpu_lib._shape_of(x)), 30, 3, gpu_lib._ptr(c2),
                        gpu_lib._ptr(l2), None, None, gpu_lib._ptr(ws), ws.numel(), gpu_lib._stream(x.device))
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(l2, labels) and torch.equal(c2, cent)
