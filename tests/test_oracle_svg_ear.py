"""Pins for the oracle's centroid compensation and error-aware routing (CPU only)."""

import math

import numpy as np
import torch

from oracle import attention as oa
from oracle import svg_ear as oe


def _clustered(seed, N=60, D=8, Cq=4, Ck=6, sigma=0.5, equal_keys=False, vscale=1.0):
    r = np.random.default_rng(seed)
    lq = np.sort(r.integers(0, Cq, N))
    lk = np.sort(r.integers(0, Ck, N))
    cq = r.standard_normal((Cq, D))
    ck = r.standard_normal((Ck, D))
    q = cq[lq] + sigma * r.standard_normal((N, D))
    k = ck[lk] if equal_keys else ck[lk] + sigma * r.standard_normal((N, D))
    v = vscale * r.standard_normal((N, D))
    q_off = np.concatenate([[0], np.cumsum(np.bincount(lq, minlength=Cq))]).astype(np.int32)
    k_off = np.concatenate([[0], np.cumsum(np.bincount(lk, minlength=Ck))]).astype(np.int32)
    return q, k, v, q_off, k_off


def _dense(q, k, v, scale):
    out, lse = oa.dense_attention(q[None, None], k[None, None], v[None, None], scale)
    return out[0, 0], lse[0, 0]


def test_centroids_by_loops():
    q, k, v, qo, ko = _clustered(0)
    c = oe.centroids(q, k, v, qo, ko)
    for a in range(len(qo) - 1):
        rows = range(qo[a], qo[a + 1])
        for d in range(q.shape[1]):
            if len(rows):
                assert abs(c["cq"][a, d] - sum(q[i, d] for i in rows) / len(rows)) < 1e-12
    assert c["nk"].sum() == len(k) and c["nq"].sum() == len(q)


def test_compensation_exact_when_keys_equal_centroid():
    """Every key equal to its centroid -> compensated == dense attention at any budget."""
    q, k, v, qo, ko = _clustered(1, equal_keys=True)
    s = 0.4
    ref, rlse = _dense(q, k, v, s)
    for ppm in (0, 100_000, 500_000, 1_000_000):
        r = oe.svg_ear_head(q, k, v, qo, ko, s, ppm)
        assert np.abs(r["out"] - ref).max() < 1e-12
        assert np.abs(r["lse"] - rlse).max() < 1e-12
        assert np.abs(r["score"]).max() < 1e-25                  # nothing to correct


def test_full_budget_is_dense_attention():
    q, k, v, qo, ko = _clustered(2)
    r = oe.svg_ear_head(q, k, v, qo, ko, 0.3, 1_000_000)
    assert r["kept"][r["cents"]["nq"] > 0][:, r["cents"]["nk"] > 0].all()
    ref, _ = _dense(q, k, v, 0.3)
    assert np.abs(r["out"] - ref).max() < 1e-12


def test_zero_budget_is_centroid_attention():
    """Budget 0 -> attention over Ck virtual keys with additive bias ln n_b (torch SDPA)."""
    q, k, v, qo, ko = _clustered(3)
    s = 0.6
    r = oe.svg_ear_head(q, k, v, qo, ko, s, 0)
    assert not r["kept"].any()
    c = r["cents"]
    live = c["nk"] > 0
    bias = torch.from_numpy(np.log(c["nk"][live]))[None, :].expand(len(q), -1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(c["ck"][live])[None],
        torch.from_numpy(c["vk"][live])[None], attn_mask=bias.contiguous(), scale=s)[0].numpy()
    assert np.abs(r["out"] - ref).max() < 1e-12


def test_singleton_clusters_score_zero():
    q, k, v, qo, _ = _clustered(4, N=20)
    ko = np.arange(21, dtype=np.int32)              # every key its own cluster
    c = oe.centroids(q, k, v, qo, ko)
    sc = oe.route_scores(k, v, ko, c, 0.5)
    assert np.abs(sc).max() < 1e-28


def test_score_bruteforce_loops():
    """Score of every block by explicit loops over the proxy query's dense softmax."""
    q, k, v, qo, ko = _clustered(5, N=24, D=3, Cq=3, Ck=4)
    s = 0.8
    c = oe.centroids(q, k, v, qo, ko)
    sc = oe.route_scores(k, v, ko, c, s)
    for a in range(3):
        if c["nq"][a] == 0:
            continue
        ca = c["cq"][a]
        w = [math.exp(s * sum(ca[d] * k[j, d] for d in range(3))) for j in range(24)]
        Z = sum(w)
        for b in range(4):
            nb = int(c["nk"][b])
            if nb == 0:
                continue
            wc = math.exp(s * sum(ca[d] * c["ck"][b, d] for d in range(3)))
            e = [(sum(w[j] * v[j, d] for j in range(ko[b], ko[b + 1])) - nb * wc * c["vk"][b, d]) / Z
                 for d in range(3)]
            assert abs(sum(x * x for x in e) / nb - sc[a, b]) < 1e-12 * max(1.0, sc[a, b])


def test_score_invariances():
    q, k, v, qo, ko = _clustered(6)
    c = oe.centroids(q, k, v, qo, ko)
    sc = oe.route_scores(k, v, ko, c, 0.5)
    c2 = oe.centroids(q, k, 2 * v, qo, ko)
    assert np.allclose(oe.route_scores(k, 2 * v, ko, c2, 0.5), 4 * sc, rtol=1e-12, atol=0)
    # shuffle keys (with their values) inside each cluster
    r = np.random.default_rng(0)
    perm = np.concatenate([ko[b] + r.permutation(ko[b + 1] - ko[b]) for b in range(len(ko) - 1)])
    c3 = oe.centroids(q, k[perm], v[perm], qo, ko)
    assert np.allclose(oe.route_scores(k[perm], v[perm], ko, c3, 0.5), sc, rtol=1e-10, atol=1e-300)


def test_scores_shrink_as_clusters_tighten():
    means = []
    for sigma in (0.8, 0.2, 0.05):
        q, k, v, qo, ko = _clustered(7, N=200, D=16, Cq=5, Ck=10, sigma=sigma)
        c = oe.centroids(q, k, v, qo, ko)
        means.append(oe.route_scores(k, v, ko, c, 0.25).mean())
    assert means[0] > means[1] > means[2]


def test_selection_against_sorted_prefix():
    r = np.random.default_rng(8)
    for trial in range(30):
        Cq, Ck = int(r.integers(1, 6)), int(r.integers(1, 8))
        nq = r.integers(0, 5, Cq)
        nk = r.integers(0, 5, Ck)
        # many ties on purpose
        score = r.integers(0, 4, (Cq, Ck)).astype(float)
        N = int(max(nq.sum(), nk.sum(), 1))
        ppm = int(r.integers(0, 1_000_001))
        rp, col, kept = oe.select_route(score, nq, nk, N, ppm)
        blocks = sorted(((-score[a, b], a * Ck + b, a, b) for a in range(Cq) for b in range(Ck)
                         if nq[a] > 0 and nk[b] > 0))
        budget = N * N * ppm // 1_000_000
        want = np.zeros((Cq, Ck), bool)
        total = 0
        for _, _, a, b in blocks:
            if total + nq[a] * nk[b] > budget:
                break
            total += nq[a] * nk[b]
            want[a, b] = True
        assert np.array_equal(kept, want)
        assert np.array_equal(oe.kept_from_csr(rp, col, Cq, Ck), kept)
        for a in range(Cq):
            assert list(col[rp[a]:rp[a + 1]]) == sorted(col[rp[a]:rp[a + 1]])


def test_compensated_attention_bruteforce():
    q, k, v, qo, ko = _clustered(9, N=30, D=4, Cq=3, Ck=5)
    s = 0.5
    c = oe.centroids(q, k, v, qo, ko)
    kept = np.random.default_rng(1).random((3, 5)) < 0.4
    out, lse = oe.compensated_attention(q, k, v, qo, ko, kept, c, s)
    for a in range(3):
        for i in range(qo[a], qo[a + 1]):
            items = []
            for b in range(5):
                if kept[a, b]:
                    items += [(s * float(q[i] @ k[j]), v[j]) for j in range(ko[b], ko[b + 1])]
                elif c["nk"][b] > 0:
                    items.append((s * float(q[i] @ c["ck"][b]) + math.log(c["nk"][b]), c["vk"][b]))
            mx = max(x for x, _ in items)
            z = sum(math.exp(x - mx) for x, _ in items)
            o = sum(math.exp(x - mx) * val for x, val in items) / z
            assert np.abs(o - out[i]).max() < 1e-12
            assert abs(mx + math.log(z) - lse[i]) < 1e-12


def test_unpermuted_output_equals_original_order():
    """At full budget the cluster-ordered output, scattered back, is attention on the original order."""
    r = np.random.default_rng(10)
    N, D = 40, 6
    q0, k0, v0 = (r.standard_normal((N, D)) for _ in range(3))
    lq, lk = r.integers(0, 4, N), r.integers(0, 7, N)
    pq, pk = np.argsort(lq, kind="stable"), np.argsort(lk, kind="stable")
    qo = np.concatenate([[0], np.cumsum(np.bincount(lq, minlength=4))]).astype(np.int32)
    ko = np.concatenate([[0], np.cumsum(np.bincount(lk, minlength=7))]).astype(np.int32)
    res = oe.svg_ear_head(q0[pq], k0[pk], v0[pk], qo, ko, 0.4, 1_000_000)
    back = np.empty_like(res["out"])
    back[pq] = res["out"]
    ref, _ = _dense(q0, k0, v0, 0.4)
    assert np.abs(back - ref).max() < 1e-12


# ---- the score against the actual compensation error (the page's idea 3) ----

def _convergence_case(seed, N, sigma_q, D=16, Cq=4, key_cluster=8, sigma_k=0.5):
    """Unit query / key centres at norm 2; queries spread by sigma_q around
    theirs, keys by sigma_k (fixed, so errors stay non-zero); key clusters of
    a fixed size, so a longer sequence has more of them."""
    r = np.random.default_rng(seed)
    Ck = N // key_cluster
    lq = np.sort(r.integers(0, Cq, N))
    lk = np.repeat(np.arange(Ck), key_cluster)
    cq = r.standard_normal((Cq, D))
    ck = r.standard_normal((Ck, D))
    cq /= np.linalg.norm(cq, axis=1, keepdims=True)
    ck /= np.linalg.norm(ck, axis=1, keepdims=True)
    q = 2.0 * cq[lq] + sigma_q * r.standard_normal((N, D))
    k = 2.0 * ck[lk] + sigma_k * r.standard_normal((N, D))
    v = r.standard_normal((N, D))
    q_off = np.concatenate([[0], np.cumsum(np.bincount(lq, minlength=Cq))]).astype(np.int64)
    k_off = np.arange(0, N + 1, key_cluster, dtype=np.int64)
    return q, k, v, q_off, k_off


def _score_vs_actual(case, score_fn=None, n_cols=24):
    q, k, v, qo, ko = case
    s = 1.0 / math.sqrt(q.shape[1])
    c = oe.centroids(q, k, v, qo, ko)
    sc = (score_fn or oe.route_scores)(k, v, ko, c, s)
    cols = np.linspace(0, len(ko) - 2, n_cols).astype(int)
    act = oe.actual_errors(q, k, v, qo, ko, c, s, key_clusters=cols)
    est = sc[:, cols]
    ratio = est / act
    return dict(agg=est.sum() / act.sum(), med=float(np.median(np.abs(ratio - 1.0))), est=est, act=act)


def _rank_corr(x, y):
    rx = np.argsort(np.argsort(x.ravel())).astype(float)
    ry = np.argsort(np.argsort(y.ravel())).astype(float)
    return float(np.corrcoef(rx, ry)[0, 1])


def test_score_converges_to_actual_error_as_clusters_tighten():
    """Idea 3: the estimate converges to the actual error as clustering gets
    finer.  Query spread 0.5 -> 0.1 -> 0.02 around the proxies: the aggregate
    ratio and the per-block ratios go to 1 and the rankings agree."""
    res = [_score_vs_actual(_convergence_case(11, 512, sq)) for sq in (0.5, 0.1, 0.02)]
    gaps = [abs(r["agg"] - 1.0) for r in res]
    meds = [r["med"] for r in res]
    assert gaps[0] > gaps[1] > gaps[2] and gaps[2] < 0.01, gaps
    assert meds[0] > meds[1] > meds[2] and meds[2] < 0.01, meds
    assert _rank_corr(res[2]["est"], res[2]["act"]) > 0.999


def test_score_converges_to_actual_error_as_sequences_grow():
    """Idea 3: ... and as the sequence grows (tight query clusters, key clusters
    of a fixed size, so each one's share of the softmax normaliser shrinks)."""
    meds = [_score_vs_actual(_convergence_case(12, n, 0.02))["med"] for n in (96, 384, 1536)]
    assert meds[0] > meds[1] > meds[2] and meds[2] < 0.006, meds


def test_selection_by_score_matches_selection_by_actual_error():
    """The routing keeps the same blocks whether it ranks by the estimate or by
    the actual error (tight clusters), at the 15 % density budget: at most one
    near-tie swapped at the cut, and the actual error the estimate's selection
    removes is within 1 % of the best selection's."""
    q, k, v, qo, ko = _convergence_case(13, 512, 0.02)
    s = 1.0 / math.sqrt(q.shape[1])
    c = oe.centroids(q, k, v, qo, ko)
    est = oe.route_scores(k, v, ko, c, s)
    act = oe.actual_errors(q, k, v, qo, ko, c, s)
    _, _, kept_est = oe.select_route(est, c["nq"], c["nk"], len(q), 150_000)
    _, _, kept_act = oe.select_route(act, c["nq"], c["nk"], len(q), 150_000)
    assert kept_act.sum() > 20
    assert (kept_est ^ kept_act).sum() <= 2
    cost = np.outer(c["nq"], c["nk"])
    assert (act * cost)[kept_est].sum() >= 0.99 * (act * cost)[kept_act].sum()


def test_convergence_pin_rejects_plausible_score_mistakes():
    """The pin above fails a score that drops the 1/Z_a normalisation, drops the
    1/n_b cost, keeps n_a in the numerator, or adds the compensation term with
    the wrong sign (each written as the mistaken score it produces)."""
    case = _convergence_case(11, 512, 0.02)
    q, k, v, qo, ko = case
    s = 1.0 / math.sqrt(q.shape[1])

    def proxy_z(cents):
        L = s * (cents["cq"] @ k.T)
        return np.exp(L - L.max(axis=1, keepdims=True)).sum(axis=1)

    def wrong_sign(k_, v_, ko_, cents, sc_):
        W = np.exp(sc_ * (cents["cq"] @ k_.T))
        out = np.zeros((len(cents["nq"]), len(cents["nk"])))
        Z = W.sum(axis=1)
        for b in range(len(cents["nk"])):
            j0, j1 = ko_[b], ko_[b + 1]
            comp = cents["nk"][b] * np.exp(sc_ * cents["cq"] @ cents["ck"][b])[:, None] * cents["vk"][b]
            e = (W[:, j0:j1] @ v_[j0:j1] + comp) / Z[:, None]
            out[:, b] = (e * e).sum(axis=1) / cents["nk"][b]
        return out

    mutants = {
        "no 1/Z_a": lambda k_, v_, ko_, c_, sc_: oe.route_scores(k_, v_, ko_, c_, sc_) * proxy_z(c_)[:, None] ** 2,
        "no 1/n_b": lambda k_, v_, ko_, c_, sc_: oe.route_scores(k_, v_, ko_, c_, sc_) * c_["nk"][None, :],
        "n_a kept": lambda k_, v_, ko_, c_, sc_: oe.route_scores(k_, v_, ko_, c_, sc_) * c_["nq"][:, None],
        "sign": wrong_sign,
    }
    for name, fn in mutants.items():
        r = _score_vs_actual(case, fn)
        assert abs(r["agg"] - 1.0) > 0.5 and r["med"] > 0.5, name
