"""GPU centroid compensation with error-aware routing vs the oracle, step by step.

Centroids and scores are compared with the float64 oracle; the selection is
checked bit-exactly on a score array the oracle produced (rounded to fp32, the
precision the device selects in); the compensated attention is checked on the
oracle's route.  The fused call is checked against the step-by-step device
path (bitwise) and its route overlap with the oracle's is reported.
"""

import math

import numpy as np
import pytest
import torch

from helpers import assert_parity, to_device, to_f64
from oracle import attention as oa
from oracle import svg_ear as oe
from synth import gen, get_workload

pytestmark = pytest.mark.gpu


def _small(seed=51, Cq=8, Ck=20, frames=2, fh=10, fw=30, H=2, D=128):
    wl = gen.scaled(get_workload("svg_ear_32k"), H=H, D=D, frames=frames, frame_h=fh, frame_w=fw,
                    n_q_clusters=Cq, n_k_clusters=Ck, kmeans_iters=3, seed=seed)
    return wl, gen.make_clustered(wl)


def _dev(d):
    q, k, v = (to_device(d[n], "bf16") for n in ("q", "k", "v"))
    qo = torch.from_numpy(d["q_off"]).cuda()
    ko = torch.from_numpy(d["k_off"]).cuda()
    return q, k, v, qo, ko


def _head(d, r):
    B_H = d["q"].shape[0] * d["q"].shape[1]
    b, h = divmod(r, d["q"].shape[1])
    q, k, v = (gen.to_f64(d[n][b, h], "bf16") for n in ("q", "k", "v"))
    return q, k, v, d["q_off"][r], d["k_off"][r]


def _check_steps(bsa, wl, d, ppm, attn_clusters=None):
    q, k, v, qo, ko = _dev(d)
    scale = 1.0 / math.sqrt(wl.D)
    qc, kc0, vc0 = bsa.cluster_centroids(q, k, v, qo, ko)
    score, kc, vc = bsa.route_scores(k, v, qo, ko, qc, scale)
    torch.cuda.synchronize()
    nh = wl.B * wl.H
    oracle_scores32 = np.empty((nh, wl.n_q_clusters, wl.n_k_clusters), np.float32)
    refs = []
    for r in range(nh):
        hq, hk, hv, hqo, hko = _head(d, r)
        cents = oe.centroids(hq, hk, hv, hqo, hko)
        # centroids from the centroid call and (keys, values) from the score pass
        for name, got in (("cq", qc[r]), ("ck", kc0[r]), ("vk", vc0[r]), ("ck", kc[r]), ("vk", vc[r])):
            g = to_f64(got)
            assert np.abs(g - cents[name]).max() <= 1e-5 * max(1.0, np.abs(cents[name]).max()), name
        sc = oe.route_scores(hk, hv, hko, cents, scale)
        gs = to_f64(score[r])
        assert np.abs(gs - sc).max() <= 1e-3 * sc.max(), (r, np.abs(gs - sc).max(), sc.max())
        oracle_scores32[r] = sc.astype(np.float32)
        refs.append((hq, hk, hv, hqo, hko, cents))

    # selection: bit-exact given the oracle's scores in fp32
    s32 = torch.from_numpy(oracle_scores32).cuda()
    rrow, rcol = bsa.route_select(s32, q, qo, ko, ppm)
    torch.cuda.synchronize()
    rrow_h, rcol_h = rrow.cpu().numpy(), rcol.cpu().numpy()
    kept_all = []
    for r in range(nh):
        hq, hk, hv, hqo, hko, cents = refs[r]
        want_rp, want_col, kept = oe.select_route(oracle_scores32[r].astype(np.float64), cents["nq"],
                                                  cents["nk"], wl.N, ppm)
        assert np.array_equal(rrow_h[r], want_rp), r
        assert np.array_equal(rcol_h[r][: want_rp[-1]], want_col), r
        kept_all.append(kept)

    # attention on the oracle's route (the route the device just reproduced)
    out, lse = bsa.compensated_attn_fwd(q, k, v, qo, ko, rrow, rcol, kc, vc, scale)
    torch.cuda.synchronize()
    got = to_f64(out)
    glse = lse.cpu().numpy()
    for r in range(nh):
        hq, hk, hv, hqo, hko, cents = refs[r]
        b, h = divmod(r, wl.H)
        ref, rlse = oe.compensated_attention(hq, hk, hv, hqo, hko, kept_all[r], cents, scale, attn_clusters)
        rows = ~np.isnan(ref[:, 0])
        assert_parity(got[b, h][rows], ref[rows], "bf16", f"compensated attention head {r}")
        assert np.abs(glse[b, h][rows] - rlse[rows]).max() < 2e-3
    return dict(q=q, k=k, v=v, qo=qo, ko=ko, score=score, rrow=rrow, rcol=rcol, out=out, lse=lse,
                kc=kc, vc=vc, s32=oracle_scores32)


@pytest.mark.parametrize("ppm", [150000, 0, 1000000, 400000])
def test_small_steps(gpu_lib, ppm):
    wl, d = _small()
    _check_steps(gpu_lib, wl, d, ppm)


def test_batch2_steps(gpu_lib):
    """Two sequences in one call: every step against the oracle for all four (batch, head) pairs."""
    wl = gen.scaled(get_workload("svg_ear_32k"), B=2, H=2, D=128, frames=2, frame_h=10, frame_w=30,
                    n_q_clusters=8, n_k_clusters=20, kmeans_iters=3, seed=55)
    _check_steps(gpu_lib, wl, gen.make_clustered(wl), 150000)


def test_small_d64_and_many_proxies(gpu_lib):
    wl, d = _small(seed=52, Cq=150, Ck=40, frames=3, fh=10, fw=40, H=1, D=64)
    _check_steps(gpu_lib, wl, d, 150000)


def test_empty_clusters(gpu_lib):
    wl, d = _small(seed=53)
    # move every token of query cluster 3 and key cluster 5 into their neighbours
    d = dict(d)
    for key in ("q_off", "k_off"):
        d[key] = d[key].copy()
    d["q_off"][:, 4] = d["q_off"][:, 3]
    d["k_off"][:, 6] = d["k_off"][:, 5]
    _check_steps(gpu_lib, wl, d, 150000)


def test_fused_call_matches_steps(gpu_lib):
    wl, d = _small(seed=54)
    q, k, v, qo, ko = _dev(d)
    scale = 1.0 / math.sqrt(wl.D)
    out, lse, rrow, rcol, score = gpu_lib.centroid_compensate(q, k, v, qo, ko, 150000, return_score=True)
    qc, _, _ = gpu_lib.cluster_centroids(q, k, v, qo, ko, which="query")
    s2, kc, vc = gpu_lib.route_scores(k, v, qo, ko, qc, scale)
    r2, c2 = gpu_lib.route_select(s2, q, qo, ko, 150000)
    o2, l2 = gpu_lib.compensated_attn_fwd(q, k, v, qo, ko, r2, c2, kc, vc, scale)
    torch.cuda.synchronize()
    assert torch.equal(score, s2) and torch.equal(rrow, r2)
    assert torch.equal(out.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)


def test_equal_keys_make_compensation_exact(gpu_lib):
    """Every key of a cluster equal to its centroid: output == dense attention at any budget."""
    wl, d = _small(seed=55)
    d = dict(d)
    k = d["k"].copy()
    for r in range(wl.B * wl.H):
        b, h = divmod(r, wl.H)
        ko = d["k_off"][r]
        for c in range(len(ko) - 1):
            if ko[c + 1] > ko[c]:
                k[b, h, ko[c]:ko[c + 1]] = k[b, h, ko[c]]
    d["k"] = k
    q, kk, v, qo, ko_t = _dev(d)
    for ppm in (0, 150000):
        out, _, _, _ = gpu_lib.centroid_compensate(q, kk, v, qo, ko_t, ppm)
        torch.cuda.synchronize()
        ref, _ = oa.dense_attention(gen.to_f64(d["q"], "bf16"), gen.to_f64(k, "bf16"),
                                    gen.to_f64(d["v"], "bf16"), 1.0 / math.sqrt(wl.D))
        assert_parity(to_f64(out), ref, "bf16", f"equal keys ppm={ppm}")


def test_gather_runs_tiny_and_empty_clusters(gpu_lib):
    """Compensated attention on given routes built to walk every path of the
    exact-key gather: kept clusters of 1-17 keys (several cluster ends inside
    the 16 slots one wave stages), empty kept clusters in the middle and at the
    end of a route row, clusters longer than a 64-key sub-tile, a row that keeps
    nothing (virtual keys only), a row that keeps everything, and routes in
    non-index order.  Against the oracle on every head and query cluster."""
    wl, d = _small(seed=57, Cq=6, Ck=20)
    N = wl.N
    small = [1, 2, 3, 0, 5, 7, 15, 16, 17, 1, 1, 1, 1, 0, 33, 2, 3, 0, 64, 65, 4, 0, 9, 13, 0, 1]
    rest = N - sum(small)
    sizes = small + [50] * (rest // 50) + ([rest % 50] if rest % 50 else []) + [0]
    Ck = len(sizes)
    assert sum(sizes) == N and Ck <= 512
    k_off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    nh = wl.B * wl.H
    d = dict(d)
    d["k_off"] = np.tile(k_off, (nh, 1))
    q, k, v, qo, ko = _dev(d)
    Cq = d["q_off"].shape[1] - 1
    rng = np.random.default_rng(57)
    empties = [b for b in range(Ck) if sizes[b] == 0]
    routes = []
    for r in range(nh):
        rows = [list(range(Ck)),                                   # everything
                [],                                                # nothing: virtual keys only
                [b for b in range(len(small))],                    # the tiny and empty ones in order
                [b for b in reversed(range(Ck)) if b % 3 == 0] + [empties[1]],  # reversed, ends empty
                sorted(rng.choice(Ck, size=Ck // 2, replace=False).tolist(), key=lambda _: rng.random()),
                list(range(0, Ck, 2)) + [empties[-1]]]
        routes.append(rows[:Cq] + [rows[2]] * max(0, Cq - len(rows)))
    rrow = np.zeros((nh, Cq + 1), np.int32)
    rcol = np.zeros((nh, Cq * Ck), np.int32)
    for r in range(nh):
        pos = 0
        for a in range(Cq):
            cols = list(dict.fromkeys(routes[r][a]))  # no repeats
            rcol[r, pos:pos + len(cols)] = cols
            pos += len(cols)
            rrow[r, a + 1] = pos
    scale = 1.0 / math.sqrt(wl.D)
    qc, kc, vc = gpu_lib.cluster_centroids(q, k, v, qo, ko)
    out, lse = gpu_lib.compensated_attn_fwd(q, k, v, qo, ko, torch.from_numpy(rrow).cuda(),
                                            torch.from_numpy(rcol).cuda(), kc, vc, scale)
    torch.cuda.synchronize()
    got, glse = to_f64(out), lse.cpu().numpy()
    for r in range(nh):
        b, h = divmod(r, wl.H)
        hq, hk, hv, hqo, hko = _head(d, r)
        cents = oe.centroids(hq, hk, hv, hqo, hko)
        kept = np.zeros((Cq, Ck), bool)
        for a in range(Cq):
            kept[a, rcol[r, rrow[r, a]:rrow[r, a + 1]]] = True
        ref, rlse = oe.compensated_attention(hq, hk, hv, hqo, hko, kept, cents, scale)
        rows = ~np.isnan(ref[:, 0])
        assert_parity(got[b, h][rows], ref[rows], "bf16", f"gather runs head {r}")
        assert np.abs(glse[b, h][rows] - rlse[rows]).max() < 2e-3


@pytest.fixture(scope="module")
def svg_full():
    wl = get_workload("svg_ear_32k")
    return wl, gen.make_clustered(wl)


def test_svg_ear_32k(gpu_lib, svg_full):
    """Full workload: all centroids and scores, selection bit-exact on every head,
    attention on sampled query clusters; then the fused call's route overlap."""
    wl, d = svg_full
    res = _check_steps(gpu_lib, wl, d, wl.density_ppm, attn_clusters=[0, 37, 99])
    out, lse, rrow, rcol = gpu_lib.centroid_compensate(res["q"], res["k"], res["v"], res["qo"], res["ko"],
                                                       wl.density_ppm)
    torch.cuda.synchronize()
    # the device's own route vs the oracle's route (reported; near-ties at the cut may differ)
    rr, rc = rrow.cpu().numpy(), rcol.cpu().numpy()
    jac = []
    for r in range(wl.H):
        hq, hk, hv, hqo, hko = _head(d, r)
        mine = set()
        for a in range(wl.n_q_clusters):
            mine |= {(a, int(b)) for b in rc[r][rr[r][a]:rr[r][a + 1]]}
        _, _, kept = oe.select_route(res["s32"][r].astype(np.float64),
                                     np.diff(hqo), np.diff(hko), wl.N, wl.density_ppm)
        ref = {(int(a), int(b)) for a, b in zip(*np.nonzero(kept))}
        jac.append(len(mine & ref) / max(1, len(mine | ref)))
    print("route Jaccard per head:", [round(j, 4) for j in jac])
    assert min(jac) > 0.9


def test_fused_call_with_given_route(gpu_lib):
    """use_given_route = 1: the route is an input.  Given back the route of an
    earlier call, the output is bitwise the step-by-step attention on it (the
    same centroid and attention kernels), and within the bf16 bar of the
    earlier call's output (whose key centroids came from the score pass).  A
    route keeping every block gives dense attention."""
    wl, d = _small(seed=56)
    q, k, v, qo, ko = _dev(d)
    scale = 1.0 / math.sqrt(wl.D)
    out0, lse0, rrow, rcol = gpu_lib.centroid_compensate(q, k, v, qo, ko, 150000)
    rr_in, rc_in = rrow.clone(), rcol.clone()
    out1, lse1, rr_after, rc_after = gpu_lib.centroid_compensate(q, k, v, qo, ko, 0, rrow=rr_in, rcol=rc_in,
                                                                 use_given_route=True)
    qc, kc, vc = gpu_lib.cluster_centroids(q, k, v, qo, ko)
    o2, l2 = gpu_lib.compensated_attn_fwd(q, k, v, qo, ko, rrow, rcol, kc, vc, scale)
    torch.cuda.synchronize()
    assert torch.equal(rr_after, rrow) and torch.equal(rc_after, rcol)      # inputs left untouched
    assert torch.equal(out1.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse1, l2)
    assert_parity(to_f64(out1), to_f64(out0), "bf16", "given route vs routed call")

    # every block kept: dense attention in cluster order
    nh, Cq, Ck = wl.B * wl.H, wl.n_q_clusters, wl.n_k_clusters
    full_rp = torch.arange(0, (Cq + 1) * Ck, Ck, dtype=torch.int32).repeat(nh, 1).cuda()
    full_col = torch.arange(Ck, dtype=torch.int32).repeat(nh, Cq).cuda()
    out3, _, _, _ = gpu_lib.centroid_compensate(q, k, v, qo, ko, 0, rrow=full_rp, rcol=full_col,
                                                use_given_route=True)
    torch.cuda.synchronize()
    ref, _ = oa.dense_attention(gen.to_f64(d["q"], "bf16"), gen.to_f64(d["k"], "bf16"),
                                gen.to_f64(d["v"], "bf16"), scale)
    assert_parity(to_f64(out3), ref, "bf16", "given full route = dense attention")


@pytest.mark.parametrize("kind", ["equal", "three_values", "one_bin", "log_uniform"])
def test_selection_ties_and_large_cut_bins(gpu_lib, kind):
    """The selection on given scores, bit-exact against the oracle's sorted-prefix
    selection, where the cut falls among many equal scores ("equal",
    "three_values": the radix passes and the index-order ties), among 50,000
    distinct scores inside one first-level bin ("one_bin"), and among scores
    spread over six decades ("log_uniform": the gathered, sorted bin)."""
    r = np.random.default_rng(81)
    H, Cq, Ck, N = 2, 100, 500, 20000
    shp = torch.empty((1, H, N, 128), dtype=torch.bfloat16, device="cuda")
    q_off = np.stack([np.concatenate([[0], np.sort(r.integers(0, N, Cq - 1)), [N]]) for _ in range(H)]).astype(np.int32)
    k_off = np.stack([np.concatenate([[0], np.sort(r.integers(0, N, Ck - 1)), [N]]) for _ in range(H)]).astype(np.int32)
    if kind == "equal":
        sc = np.ones((H, Cq, Ck), np.float32)
    elif kind == "three_values":
        sc = r.choice(np.array([1.0, 2.0, 3.0], np.float32), (H, Cq, Ck))
    elif kind == "one_bin":
        sc = (1.0 + 0.05 * r.random((H, Cq, Ck))).astype(np.float32)
    else:
        sc = (10.0 ** r.uniform(-6, 0, (H, Cq, Ck))).astype(np.float32)
    qo, ko = torch.from_numpy(q_off).cuda(), torch.from_numpy(k_off).cuda()
    for ppm in (150000, 1000, 999999):
        rrow, rcol = gpu_lib.route_select(torch.from_numpy(sc).cuda(), shp, qo, ko, ppm)
        torch.cuda.synchronize()
        rr, rc = rrow.cpu().numpy(), rcol.cpu().numpy()
        for h in range(H):
            want_rp, want_col, _ = oe.select_route(sc[h].astype(np.float64), np.diff(q_off[h]), np.diff(k_off[h]),
                                                   N, ppm)
            assert np.array_equal(rr[h], want_rp), (kind, ppm, h)
            assert np.array_equal(rc[h][: want_rp[-1]], want_col), (kind, ppm, h)
