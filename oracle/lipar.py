"""Oracle: latent inter-frame pruning and restoration (float64).

Test infrastructure only (see the package docstring).

"LIPAR: 비디오 생성 AI 를 위한 '스마트 스킵' 기술" (gist.science summary of the
LIPAR paper), section 2 Methodology, B. LIPAR pipeline:

* Latent inter-frame pruning: the latent patch difference between adjacent
  frames is computed, and patches whose difference is at most a threshold tau
  are "unchanged"; removing them shortens the token sequence.
* Restoration: before decoding, the pruned sequence is expanded back to its
  original length by duplicating the patches of the previous frame.

Readings (the page gives neither a norm nor an order):
* A token is one latent patch, a row of the [N, D] token matrix of one
  sequence; token n = f * P + p is patch p of frame f (frame-major, N = F * P).
* Difference of token (f, p), f >= 1: the sum over its D values of
  |x[f, p] - x[f - 1, p]| against the adjacent *input* frame.  The token is kept
  iff that sum exceeds tau * D (its mean absolute difference exceeds tau).
  Frame 0 has no predecessor and is always kept.  For inputs that are exact in
  bf16 the differences and their sum are exact in float64, so the decision has
  no rounding.
* tau is a single-precision parameter: the threshold is its float32 value
  times D, in float64.
* The pruned sequence holds the kept rows in token order.
* Restoration: a kept token takes its row of the pruned sequence; a pruned
  token (f, p) takes the restored row of (f - 1, p), i.e. the row of the latest
  frame f' <= f in which patch p was kept.
* The motion-detection refinement the page mentions (spatial / temporal
  neighbours) is not specified there and is not part of this reading.
"""

import numpy as np


def keep_flags(x, frames: int, tau: float):
    """keep [N] bool for one sequence x [N, D] (float64)."""
    x = np.asarray(x, np.float64)
    N, D = x.shape
    assert N % frames == 0, "N must be a multiple of the frame count"
    P = N // frames
    xf = x.reshape(frames, P, D)
    keep = np.ones((frames, P), dtype=bool)
    if frames > 1:
        diff = np.abs(xf[1:] - xf[:-1]).sum(axis=2)
        keep[1:] = diff > float(np.float32(tau)) * D
    return keep.reshape(N)


def prune(x, frames: int, tau: float):
    """(keep [N] bool, kept token indices ascending, pruned rows [n_kept, D])."""
    x = np.asarray(x, np.float64)
    keep = keep_flags(x, frames, tau)
    idx = np.flatnonzero(keep)
    return keep, idx, x[idx]


def restore(y, keep, frames: int):
    """Full-length [N, D] from the pruned rows y [n_kept, D] and the keep flags."""
    y = np.asarray(y, np.float64)
    keep = np.asarray(keep, bool)
    N = keep.size
    P = N // frames
    pos = np.cumsum(keep) - 1          # position of a kept token in the pruned sequence
    kf = keep.reshape(frames, P)
    pf = pos.reshape(frames, P)
    out = np.empty((frames, P, y.shape[1]), np.float64)
    for f in range(frames):
        if f == 0:
            out[0] = y[pf[0]]          # frame 0 is always kept
        else:
            out[f] = np.where(kf[f][:, None], y[np.maximum(pf[f], 0)], out[f - 1])
    return out.reshape(N, -1)
