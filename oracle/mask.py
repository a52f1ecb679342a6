"""Oracle: spatiotemporal token rule, block mask and CSR (integer, exact).

Test infrastructure only (see the package docstring).

Token order.  A video latent of F frames of P patches is flattened frame-major:
token t has frame f(t) = t // P and in-frame raster position p(t) = t % P.

Token rules (one per mask kind):

* ALL: every pair is kept (dense attention, the quadratic baseline that every
  page starts from).
* WINDOW_ANCHOR (LVSA review page, section 3 Method & Key Results, and its
  Figure 1 "extended window pattern" / Figure 2 "rotating global frames"):
  a query frame attends to the key frames within ``window`` of it, and to the
  global anchor frames A(s) = {f < F : f mod period == s mod period}, where s is
  the denoising step (the anchor set rotates by one frame per step).  With
  ``anchor_rows`` the anchor frames are global in both directions: their
  queries also attend to every key.
* RADIAL (Radial Attention headline page): the window shrinks exponentially
  with temporal distance.  With dt = f(q) - f(k): kept if dt == 0, else kept if
  |p(q) - p(k)| * 2^floor(log2 |dt|) <= W.  The integer form avoids any
  floating point in the rule.

Block rule.  Block i covers real tokens [i*b, min((i+1)*b, N)); the pair (i, j)
is kept when at least one real token pair (tq in block i, tk in block j) is
kept.  Padding tokens past N never count.

Two independent implementations are provided: ``block_mask_bruteforce``
enumerates token pairs (tiny inputs), ``block_mask`` reasons over per-frame
segments of each block (any size).  Tests require them to agree.
"""

from dataclasses import dataclass

import numpy as np

ALL, WINDOW_ANCHOR, RADIAL = 0, 1, 2


@dataclass(frozen=True)
class MaskSpec:
    kind: int
    frames: int
    frame_tokens: int
    block: int
    window: int = 0
    anchor_period: int = 0
    anchor_step: int = 0
    anchor_rows: int = 0
    radial_w: int = 0

    @property
    def N(self) -> int:
        return self.frames * self.frame_tokens

    @property
    def nb(self) -> int:
        return -(-self.N // self.block)


def spec_from_params(p: dict) -> MaskSpec:
    return MaskSpec(**{k: int(v) for k, v in p.items()})


def is_anchor(f: int, spec: MaskSpec) -> bool:
    if spec.anchor_period <= 0:
        return False
    return f % spec.anchor_period == spec.anchor_step % spec.anchor_period


def floor_log2(x: int) -> int:
    return int(x).bit_length() - 1


def token_keep(tq: int, tk: int, spec: MaskSpec) -> bool:
    """The token-level rule for one (query, key) pair of real tokens."""
    P = spec.frame_tokens
    fq, pq = divmod(tq, P)
    fk, pk = divmod(tk, P)
    if spec.kind == ALL:
        return True
    if spec.kind == WINDOW_ANCHOR:
        if abs(fq - fk) <= spec.window:
            return True
        if is_anchor(fk, spec):
            return True
        return bool(spec.anchor_rows) and is_anchor(fq, spec)
    if spec.kind == RADIAL:
        dt = abs(fq - fk)
        if dt == 0:
            return True
        return (abs(pq - pk) << floor_log2(dt)) <= spec.radial_w
    raise ValueError(f"unknown mask kind {spec.kind}")


def block_mask_bruteforce(spec: MaskSpec) -> np.ndarray:
    """Block mask by enumerating every real token pair (tiny inputs only)."""
    N, b, nb = spec.N, spec.block, spec.nb
    m = np.zeros((nb, nb), dtype=bool)
    for tq in range(N):
        for tk in range(N):
            if not m[tq // b, tk // b] and token_keep(tq, tk, spec):
                m[tq // b, tk // b] = True
    return m


def _segments(spec: MaskSpec):
    """Per-frame pieces of every block: arrays (block, frame, first pos, last pos)."""
    N, P, b = spec.N, spec.frame_tokens, spec.block
    blk, fr, lo, hi = [], [], [], []
    for i in range(spec.nb):
        t0, t1 = i * b, min((i + 1) * b, N)          # real tokens [t0, t1)
        for f in range(t0 // P, (t1 - 1) // P + 1):
            a = max(t0, f * P) - f * P
            z = min(t1, (f + 1) * P) - 1 - f * P
            blk.append(i), fr.append(f), lo.append(a), hi.append(z)
    return (np.array(blk, np.int64), np.array(fr, np.int64),
            np.array(lo, np.int64), np.array(hi, np.int64))


def block_mask(spec: MaskSpec) -> np.ndarray:
    """Block mask from per-frame segments.

    Within one (query frame, key frame) pair the window/anchor rule does not
    depend on positions, and the radial test is monotone in |p(q) - p(k)|, so a
    segment pair holds a kept token pair iff the rule holds at the smallest
    position distance between the two segments.
    """
    nb = spec.nb
    if spec.kind == ALL:
        return np.ones((nb, nb), dtype=bool)
    sb, sf, slo, shi = _segments(spec)
    m = np.zeros((nb, nb), dtype=bool)
    chunk = max(1, 4_000_000 // max(1, len(sb)))
    for c0 in range(0, len(sb), chunk):
        qb, qf = sb[c0:c0 + chunk, None], sf[c0:c0 + chunk, None]
        qlo, qhi = slo[c0:c0 + chunk, None], shi[c0:c0 + chunk, None]
        kb, kf, klo, khi = sb[None, :], sf[None, :], slo[None, :], shi[None, :]
        dt = np.abs(qf - kf)
        if spec.kind == WINDOW_ANCHOR:
            keep = dt <= spec.window
            if spec.anchor_period > 0:
                s = spec.anchor_step % spec.anchor_period
                keep = keep | (kf % spec.anchor_period == s)
                if spec.anchor_rows:
                    keep = keep | (qf % spec.anchor_period == s)
        elif spec.kind == RADIAL:
            dist = np.maximum(0, np.maximum(klo - qhi, qlo - khi))
            r = np.zeros_like(dt)
            nz = dt > 0
            # floor(log2 dt) for dt >= 1, exact in integers
            r[nz] = np.array([floor_log2(x) for x in range(int(dt.max()) + 1)])[dt[nz]]
            keep = (dt == 0) | ((dist << r) <= spec.radial_w)
        else:
            raise ValueError(f"unknown mask kind {spec.kind}")
        qi, ki = np.nonzero(keep)
        m[qb[qi, 0], kb[0, ki]] = True
    return m


def to_csr(m: np.ndarray):
    """CSR of a boolean block mask; columns ascending within each row (int32)."""
    counts = m.sum(axis=1)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    col_idx = np.nonzero(m)[1].astype(np.int32)
    return row_ptr, col_idx


def token_mask(spec: MaskSpec) -> np.ndarray:
    """Dense token-level keep matrix [N, N] of the token rule (tiny inputs only)."""
    N = spec.N
    return np.array([[token_keep(a, c, spec) for c in range(N)] for a in range(N)], dtype=bool)


def kept_token_pairs_per_query(spec: MaskSpec) -> float:
    """Average number of kept keys per query token under the token rule.

    Counted per frame pair in closed form over positions, so it runs at full
    sequence lengths; used to check the O(n log n) growth of the radial rule.
    """
    P, F = spec.frame_tokens, spec.frames
    total = 0
    for dt in range(-(F - 1), F):
        nframes = F - abs(dt)
        if spec.kind == RADIAL:
            if dt == 0:
                per = P * P
            else:
                d = spec.radial_w >> floor_log2(abs(dt))        # largest allowed distance
                d = min(d, P - 1)
                per = P + 2 * sum(P - x for x in range(1, d + 1))
        else:
            raise ValueError("only the radial rule is counted in closed form")
        total += nframes * per
    return total / spec.N
