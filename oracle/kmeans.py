"""Oracle: k-means clustering of query / key tokens and the cluster order (float64).

Test infrastructure only (see the package docstring).

"SVG-EAR: Parameter-Free Linear Compensation for Sparse Video Generation via
Error-aware Routing", technical summary section 2 Method: query and key tokens
are grouped by semantic similarity into clusters (C_q and C_k of them), every
call; attention then works on (query cluster, key cluster) blocks of tokens
laid out cluster by cluster.

Readings (the page names the grouping, not the algorithm):
* The grouping is Lloyd's k-means on the token rows of one (batch, head): from
  given initial centres, ``iters`` steps of (assign every token to its nearest
  centre in squared Euclidean distance; move every centre to the mean of its
  tokens), then a final assignment to the final centres, so the labels and the
  returned centres belong together.  A centre with no tokens stays where it is.
* Ties go to the lowest centre index.
* Distance precision (``centre_dtype="bf16"``): the assignment compares
  |c|^2 - 2 x.c with the centres rounded to bf16 (round to nearest even), the
  precision the device takes the decision in; ``None`` keeps them in float64
  (the textbook algorithm, pinned against scikit-learn).
* The cluster order is the stable sort of the tokens by label: cluster a is
  the rows [off[a], off[a + 1]) of the permuted sequence, tokens in their
  original order inside a cluster.  perm[i] is the original index of permuted
  row i; un-permuting writes row i back to perm[i].
"""

import numpy as np

from .numerics import round_bf16


def assign(x, centres, centre_dtype="bf16"):
    """Labels [N]: argmin over centres of |c|^2 - 2 x.c (lowest index on ties)."""
    x = np.asarray(x, np.float64)
    c = np.asarray(centres, np.float64)
    if centre_dtype == "bf16":
        c = round_bf16(c)
    d = (c * c).sum(axis=1)[None, :] - 2.0 * (x @ c.T)
    return np.argmin(d, axis=1)


def update(x, labels, centres):
    """New centres: the mean of each cluster's rows; empty clusters keep theirs."""
    x = np.asarray(x, np.float64)
    c = np.array(centres, np.float64)
    counts = np.bincount(labels, minlength=c.shape[0])
    sums = np.zeros_like(c)
    np.add.at(sums, labels, x)
    nz = counts > 0
    c[nz] = sums[nz] / counts[nz, None]
    return c


def lloyd(x, init, iters: int, centre_dtype="bf16"):
    """(labels [N], centres [C, D]) after ``iters`` Lloyd steps and a final assignment."""
    c = np.array(init, np.float64)
    for _ in range(iters):
        c = update(x, assign(x, c, centre_dtype), c)
    return assign(x, c, centre_dtype), c


def cluster_order(labels, C: int):
    """(perm [N], off [C + 1]): the stable sort of the tokens by label."""
    labels = np.asarray(labels)
    perm = np.argsort(labels, kind="stable")
    off = np.concatenate([[0], np.cumsum(np.bincount(labels, minlength=C))])
    return perm, off


def gather_rows(x, perm):
    """Permuted rows: out[i] = x[perm[i]]."""
    return np.asarray(x)[np.asarray(perm)]


def scatter_rows(y, perm):
    """Un-permuted rows: out[perm[i]] = y[i]."""
    y = np.asarray(y)
    out = np.empty_like(y)
    out[np.asarray(perm)] = y
    return out
