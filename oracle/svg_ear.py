"""Oracle: centroid linear compensation with error-aware routing (float64).

Test infrastructure only (see the package docstring).

Source: "SVG-EAR: Parameter-Free Linear Compensation for Sparse Video
Generation via Error-aware Routing", technical summary section 2 Method.

Inputs for one (batch, head): Q rows ordered by query cluster, K and V rows
ordered by key cluster, and CSR offsets q_off [Cq+1], k_off [Ck+1], so query
cluster a is rows [q_off[a], q_off[a+1]) and key cluster b is rows
[k_off[b], k_off[b+1]).  A "block" is a (query cluster, key cluster) pair; its
cost is n_a * n_b scores.  s is the softmax scale (1/sqrt(D)).

1. Centroids (idea 1: skipped blocks are approximated with the cluster
   centroid): c^_a = mean of Q rows of a; c_b = mean of K rows of b;
   vbar_b = mean of V rows of b.
2. Proxy logits (idea 2, efficiency: query-cluster centroids stand in for the
   queries, cost O(Cq Nk d) instead of O(Nq Nk d)): l_{a,j} = s c^_a . k_j over
   all keys j; m_a = max_j l_{a,j}; Z_a = sum_j exp(l_{a,j} - m_a).
3. Estimated compensation error of block (a, b) for the proxy query:
       e_ab = ( sum_{j in b} exp(l_{a,j} - m_a) v_j
                - n_b exp(s c^_a . c_b - m_a) vbar_b ) / Z_a      (a D-vector)
   score_ab = n_a ||e_ab||^2 / (n_a n_b) = ||e_ab||^2 / n_b, the squared output
   error of the n_a queries per unit cost.  The page states the idea (error
   estimated by lightweight probing, error-to-cost ratio) but prints no
   formula, so this exact score is a reading.  It is pinned to what the page
   does state (idea 3: as clustering tightens and sequences grow, the
   estimated error converges to the actual error): ``actual_errors`` below
   computes the actual per-cost output error of compensating one block, from
   dense attention and ``compensated_attention`` alone, and the tests require
   the ratio score / actual error to go to 1 and the two rankings to agree in
   those limits.  Also pinned: the score vanishes when a cluster's keys all
   equal their centroid or the cluster is a single key, it scales as |V|^2,
   and it is invariant to the order of keys inside a cluster.
4. Selection (idea 2, routing under a fixed density budget): over non-empty
   blocks, order by (score descending, a * Ck + b ascending) and keep the
   longest prefix whose total cost is <= floor(N * N * density_ppm / 10^6),
   computed in integers.
5. Output for a query q of cluster a: one softmax over the exact keys of the
   kept blocks of row a, plus one "virtual key" per skipped non-empty cluster b
   with logit s q . c_b + ln n_b and value vbar_b (the cluster's n_b keys are
   replaced by n_b copies of the centroid, idea 1).  The real query is used,
   not c^_a.  lse is taken over the same augmented set.
"""

import numpy as np


def centroids(q, k, v, q_off, k_off):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    Cq, Ck, D = len(q_off) - 1, len(k_off) - 1, q.shape[1]
    nq = np.diff(np.asarray(q_off, np.int64))
    nk = np.diff(np.asarray(k_off, np.int64))
    cq = np.zeros((Cq, D))
    ck = np.zeros((Ck, D))
    vk = np.zeros((Ck, D))
    for a in range(Cq):
        if nq[a]:
            cq[a] = q[q_off[a]:q_off[a + 1]].mean(axis=0)
    for b in range(Ck):
        if nk[b]:
            ck[b] = k[k_off[b]:k_off[b + 1]].mean(axis=0)
            vk[b] = v[k_off[b]:k_off[b + 1]].mean(axis=0)
    return dict(cq=cq, nq=nq, ck=ck, vk=vk, nk=nk)


def route_scores(k, v, k_off, cents, scale: float):
    """score [Cq, Ck] (float64); entries of empty clusters are 0."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    cq, nq, ck, vk, nk = (cents[x] for x in ("cq", "nq", "ck", "vk", "nk"))
    Cq, Ck = len(nq), len(nk)
    L = scale * (cq @ k.T)                              # [Cq, N]
    m = L.max(axis=1, keepdims=True)
    W = np.exp(L - m)
    Z = W.sum(axis=1)                                   # [Cq]
    lc = scale * (cq @ ck.T)                            # [Cq, Ck]
    score = np.zeros((Cq, Ck))
    for b in range(Ck):
        if nk[b] == 0:
            continue
        j0, j1 = k_off[b], k_off[b + 1]
        exact = W[:, j0:j1] @ v[j0:j1]                  # [Cq, D]
        comp = nk[b] * np.exp(lc[:, b] - m[:, 0])[:, None] * vk[b][None, :]
        e = (exact - comp) / Z[:, None]
        score[:, b] = (e * e).sum(axis=1) / nk[b]
    score[nq == 0, :] = 0.0
    return score


def actual_errors(q, k, v, q_off, k_off, cents, scale: float, key_clusters=None):
    """The actual compensation error of each block (a, b), per unit cost
    (idea 3's "actual error", the quantity the routing score estimates):

        err_ab = sum_{q in a} |O_b(q) - O(q)|^2 / (n_a n_b)

    where O(q) is dense softmax attention of the real query q over all keys and
    O_b(q) is the compensated output with only key cluster b replaced by its
    virtual key (every other block exact, ``compensated_attention`` with one
    skipped column).  Each query keeps its own max and normaliser; nothing
    here uses the proxy centroids.  Returns [Cq, len(key_clusters)] (all key
    clusters when None); empty clusters give 0."""
    from . import attention as _attn
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    nq, nk = cents["nq"], cents["nk"]
    Cq, Ck = len(nq), len(nk)
    cols = range(Ck) if key_clusters is None else list(key_clusters)
    ref, _ = _attn.dense_attention(q[None, None], k[None, None], v[None, None], scale)
    ref = ref[0, 0]
    err = np.zeros((Cq, len(cols)))
    for i, b in enumerate(cols):
        if nk[b] == 0:
            continue
        kept = np.ones((Cq, Ck), dtype=bool)
        kept[:, b] = False
        out, _ = compensated_attention(q, k, v, q_off, k_off, kept, cents, scale)
        for a in range(Cq):
            r0, r1 = q_off[a], q_off[a + 1]
            if r1 > r0:
                err[a, i] = ((out[r0:r1] - ref[r0:r1]) ** 2).sum() / (nq[a] * nk[b])
    return err


def budget(N: int, density_ppm: int) -> int:
    return (int(N) * int(N) * int(density_ppm)) // 1_000_000


def select_route(score, nq, nk, N: int, density_ppm: int):
    """Route CSR (row_ptr [Cq+1], col [nnz], ascending) and the kept matrix [Cq, Ck]."""
    score = np.asarray(score, np.float64)
    nq = np.asarray(nq, np.int64)
    nk = np.asarray(nk, np.int64)
    Cq, Ck = score.shape
    a_idx, b_idx = np.nonzero((nq[:, None] > 0) & (nk[None, :] > 0))
    lin = a_idx * Ck + b_idx
    order = np.lexsort((lin, -score[a_idx, b_idx]))
    cost = (nq[a_idx] * nk[b_idx])[order]
    within = np.cumsum(cost) <= budget(N, density_ppm)
    # longest prefix: stop at the first block that does not fit
    take = order[: int(np.argmin(within)) if not within.all() else len(order)]
    kept = np.zeros((Cq, Ck), dtype=bool)
    kept[a_idx[take], b_idx[take]] = True
    counts = kept.sum(axis=1)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    col = np.nonzero(kept)[1].astype(np.int32)
    return row_ptr, col, kept


def kept_from_csr(row_ptr, col, Cq: int, Ck: int) -> np.ndarray:
    kept = np.zeros((Cq, Ck), dtype=bool)
    for a in range(Cq):
        kept[a, col[row_ptr[a]:row_ptr[a + 1]]] = True
    return kept


def compensated_attention(q, k, v, q_off, k_off, kept, cents, scale: float, clusters=None):
    """out [N, D] and lse [N] in query-cluster order, for the query clusters given."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    N, D = q.shape
    ck, vk, nk = cents["ck"], cents["vk"], cents["nk"]
    Cq = len(q_off) - 1
    out = np.full((N, D), np.nan)
    lse = np.full(N, np.nan)
    rows = range(Cq) if clusters is None else clusters
    for a in rows:
        r0, r1 = q_off[a], q_off[a + 1]
        if r1 == r0:
            continue
        kb = np.nonzero(kept[a])[0]
        keys = (np.concatenate([np.arange(k_off[b], k_off[b + 1]) for b in kb])
                if len(kb) else np.zeros(0, np.int64))
        virt = np.nonzero(~kept[a] & (nk > 0))[0]
        qa = q[r0:r1]
        logits = np.concatenate([scale * (qa @ k[keys].T),
                                 scale * (qa @ ck[virt].T) + np.log(nk[virt])[None, :]], axis=1)
        vals = np.concatenate([v[keys], vk[virt]], axis=0)
        if logits.shape[1] == 0:
            out[r0:r1] = 0.0
            lse[r0:r1] = -np.inf
            continue
        mx = logits.max(axis=1, keepdims=True)
        w = np.exp(logits - mx)
        z = w.sum(axis=1, keepdims=True)
        out[r0:r1] = (w @ vals) / z
        lse[r0:r1] = (mx + np.log(z))[:, 0]
    return out, lse


def svg_ear_head(q, k, v, q_off, k_off, scale: float, density_ppm: int, clusters=None):
    """All five steps for one head; returns a dict of every intermediate."""
    cents = centroids(q, k, v, q_off, k_off)
    score = route_scores(k, v, k_off, cents, scale)
    row_ptr, col, kept = select_route(score, cents["nq"], cents["nk"], q.shape[0], density_ppm)
    out, lse = compensated_attention(q, k, v, q_off, k_off, kept, cents, scale, clusters)
    return dict(cents=cents, score=score, row_ptr=row_ptr, col=col, kept=kept, out=out, lse=lse)
