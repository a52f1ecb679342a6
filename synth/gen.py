"""Seeded generators for Q, K, V and the cluster ordering of the clustered workload.

Random streams: numpy PCG64 seeded by ``SeedSequence([workload seed, tensor,
batch, head, purpose])`` so every (tensor, batch, head) slice can be drawn on
its own, in any order, and is identical on every machine with the same numpy.

bf16 tensors are handled as their raw 16-bit patterns (``uint16`` arrays):
``f32_to_bf16_bits`` rounds to nearest-even, and the widening helpers are exact.
Both the oracle and the device path start from these same bits.
"""

import dataclasses
import numpy as np

from .configs import Workload

TENSOR_ID = {"q": 0, "k": 1, "v": 2}
_PURPOSE_NOISE, _PURPOSE_FRAME, _PURPOSE_CENTRES, _PURPOSE_LABELS = 0, 1, 2, 3


def rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def normal_f32(key, shape) -> np.ndarray:
    return rng(*key).standard_normal(shape, dtype=np.float32)


# ----------------------------------------------------------------------------
# bf16 bit handling
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Widen a stored tensor (bf16 bits or float32) exactly to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def store(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x_f32) if dtype == "bf16" else np.ascontiguousarray(x_f32, np.float32)


# ----------------------------------------------------------------------------
# value recipes
# ----------------------------------------------------------------------------

def ar1_frame_component(key, frames: int, D: int, rho: float) -> np.ndarray:
    """g_0 ~ N(0, I); g_f = rho * g_{f-1} + sqrt(1 - rho^2) * eta_f  (float32 [frames, D])."""
    eta = rng(*key).standard_normal((frames, D))
    g = np.empty((frames, D))
    g[0] = eta[0]
    s = np.sqrt(1.0 - rho * rho)
    for f in range(1, frames):
        g[f] = rho * g[f - 1] + s * eta[f]
    return g.astype(np.float32)


def head_tensor(wl: Workload, name: str, b: int, h: int) -> np.ndarray:
    """One [N, D] float32 slice of q, k or v for the iid / ar1 recipes (before rounding)."""
    t = TENSOR_ID[name]
    x = normal_f32((wl.seed, t, b, h, _PURPOSE_NOISE), (wl.N, wl.D))
    if wl.values == "ar1":
        g = ar1_frame_component((wl.seed, t, b, h, _PURPOSE_FRAME), wl.frames, wl.D, wl.ar_rho)
        x = (x.reshape(wl.frames, wl.P, wl.D) + g[:, None, :]).reshape(wl.N, wl.D)
    elif wl.values != "iid":
        raise ValueError(f"head_tensor does not handle values={wl.values!r}")
    return x


def make_qkv(wl: Workload, heads=None):
    """Q, K, V as stored tensors [B, H', N, D] (uint16 bf16 bits or float32).

    ``heads`` optionally restricts generation to a list of head indices (the
    slices are still the ones the full tensor would hold).
    """
    if wl.values == "gmm":
        raise ValueError("use make_clustered for the gmm recipe")
    hs = list(range(wl.H)) if heads is None else list(heads)
    out = {}
    for name in ("q", "k", "v"):
        dt = np.uint16 if wl.dtype == "bf16" else np.float32
        arr = np.empty((wl.B, len(hs), wl.N, wl.D), dtype=dt)
        for b in range(wl.B):
            for i, h in enumerate(hs):
                arr[b, i] = store(head_tensor(wl, name, b, h), wl.dtype)
        out[name] = arr
    return out


# ----------------------------------------------------------------------------
# clustered (Gaussian-mixture) recipe
# ----------------------------------------------------------------------------

def _unit_centres(key, C: int, D: int) -> np.ndarray:
    c = rng(*key).standard_normal((C, D))
    return c / np.linalg.norm(c, axis=1, keepdims=True)


def _mixture(wl: Workload, t: int, b: int, h: int, C: int):
    centres = _unit_centres((wl.seed, t, b, h, _PURPOSE_CENTRES), C, wl.D)
    labels = rng(wl.seed, t, b, h, _PURPOSE_LABELS).integers(0, C, size=wl.N)
    noise = normal_f32((wl.seed, t, b, h, _PURPOSE_NOISE), (wl.N, wl.D))
    x = (centres[labels] + wl.gmm_sigma * noise.astype(np.float64)).astype(np.float32)
    return x, centres


def make_gmm_tokens(wl: Workload, heads=None):
    """Q, K, V of the Gaussian-mixture recipe in token order (not clustered), and
    the generating centres (float32 [B*H', C, D]) that serve as the initial
    k-means centres."""
    hs = list(range(wl.H)) if heads is None else list(heads)
    Cq, Ck = wl.n_q_clusters, wl.n_k_clusters
    dt = np.uint16 if wl.dtype == "bf16" else np.float32
    q = np.empty((wl.B, len(hs), wl.N, wl.D), dt)
    k = np.empty_like(q)
    v = np.empty_like(q)
    cq = np.empty((wl.B * len(hs), Cq, wl.D), np.float32)
    ck = np.empty((wl.B * len(hs), Ck, wl.D), np.float32)
    for b in range(wl.B):
        for i, h in enumerate(hs):
            r = b * len(hs) + i
            xq, gq = _mixture(wl, TENSOR_ID["q"], b, h, Cq)
            xk, gk = _mixture(wl, TENSOR_ID["k"], b, h, Ck)
            xv = normal_f32((wl.seed, TENSOR_ID["v"], b, h, _PURPOSE_NOISE), (wl.N, wl.D))
            q[b, i], k[b, i], v[b, i] = store(xq, wl.dtype), store(xk, wl.dtype), store(xv, wl.dtype)
            cq[r], ck[r] = gq, gk
    return dict(q=q, k=k, v=v, centres_q=cq, centres_k=ck)


def kmeans_labels(x: np.ndarray, init: np.ndarray, iters: int) -> np.ndarray:
    """Lloyd iterations in float64 from the given centres; ties go to the lowest index.

    Input preparation only: it decides the token order that both sides then
    receive, and is never itself compared.  Empty clusters keep their centre.
    """
    x = np.asarray(x, dtype=np.float64)
    c = np.array(init, dtype=np.float64)
    C = c.shape[0]

    def assign(c):
        d = (c * c).sum(1)[None, :] - 2.0 * (x @ c.T)
        return np.argmin(d, axis=1)

    for _ in range(iters):
        lab = assign(c)
        order = np.argsort(lab, kind="stable")
        counts = np.bincount(lab, minlength=C)
        starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
        nz = counts > 0
        sums = np.add.reduceat(x[order], starts[nz], axis=0)
        c[nz] = sums / counts[nz, None]
    return assign(c)


def cluster_order(labels: np.ndarray, C: int):
    """Stable permutation grouping tokens by label, and CSR offsets [C + 1]."""
    perm = np.argsort(labels, kind="stable")
    counts = np.bincount(labels, minlength=C)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return perm.astype(np.int64), off


def make_clustered(wl: Workload, heads=None):
    """Q, K, V of the Gaussian-mixture recipe, each head permuted into cluster order.

    Returns a dict with stored tensors q, k, v [B, H', N, D] (already permuted),
    q_off [B*H', Cq+1], k_off [B*H', Ck+1] (int32), and the permutations
    perm_q, perm_k [B*H', N] such that permuted[i] = original[perm[i]].
    """
    hs = list(range(wl.H)) if heads is None else list(heads)
    Cq, Ck = wl.n_q_clusters, wl.n_k_clusters
    nh = wl.B * len(hs)
    dt = np.uint16 if wl.dtype == "bf16" else np.float32
    q = np.empty((wl.B, len(hs), wl.N, wl.D), dt)
    k = np.empty_like(q)
    v = np.empty_like(q)
    q_off = np.empty((nh, Cq + 1), np.int32)
    k_off = np.empty((nh, Ck + 1), np.int32)
    perm_q = np.empty((nh, wl.N), np.int64)
    perm_k = np.empty((nh, wl.N), np.int64)
    for b in range(wl.B):
        for i, h in enumerate(hs):
            r = b * len(hs) + i
            xq, cq = _mixture(wl, TENSOR_ID["q"], b, h, Cq)
            xk, ck = _mixture(wl, TENSOR_ID["k"], b, h, Ck)
            xv = normal_f32((wl.seed, TENSOR_ID["v"], b, h, _PURPOSE_NOISE), (wl.N, wl.D))
            sq, sk, sv = store(xq, wl.dtype), store(xk, wl.dtype), store(xv, wl.dtype)
            lq = kmeans_labels(to_f64(sq, wl.dtype), cq, wl.kmeans_iters)
            lk = kmeans_labels(to_f64(sk, wl.dtype), ck, wl.kmeans_iters)
            pq, oq = cluster_order(lq, Cq)
            pk, ok = cluster_order(lk, Ck)
            q[b, i], k[b, i], v[b, i] = sq[pq], sk[pk], sv[pk]
            q_off[r], k_off[r], perm_q[r], perm_k[r] = oq, ok, pq, pk
    return dict(q=q, k=k, v=v, q_off=q_off, k_off=k_off, perm_q=perm_q, perm_k=perm_k)


def make_video(wl: Workload):
    """Latent token sequences [B, H, N, D] (bf16 bits) of the "video" recipe.

    Per (batch, head): a static background N(0, 1) per patch, plus per frame
    0.02 N(0, 1) jitter on every value; a rectangle of frame_h/4 x frame_w/5
    patches carrying its own N(0, 1) texture that moves one patch to the right
    per frame (wrapping); and the bottom eighth of the frame redrawn N(0, 1)
    every frame.  Jitter alone keeps the mean |difference| between frames near
    0.023, the object and the changing region near 1.1.
    """
    F, fh, fw, D = wl.frames, wl.frame_h, wl.frame_w, wl.D
    dt = np.uint16 if wl.dtype == "bf16" else np.float32
    out = np.empty((wl.B, wl.H, wl.N, D), dt)
    oh, ow = max(1, fh // 4), max(1, fw // 5)
    h0 = fh // 3
    ch = max(1, fh // 8)
    for b in range(wl.B):
        for h in range(wl.H):
            bg = normal_f32((wl.seed, 0, b, h, _PURPOSE_NOISE), (fh, fw, D))
            tex = normal_f32((wl.seed, 1, b, h, _PURPOSE_NOISE), (oh, ow, D))
            x = np.empty((F, fh, fw, D), np.float32)
            for f in range(F):
                fr = bg + np.float32(0.02) * normal_f32((wl.seed, 2, b, h, f), (fh, fw, D))
                cols = (np.arange(ow) + f) % fw
                fr[h0:h0 + oh][:, cols] = tex
                fr[fh - ch:] = normal_f32((wl.seed, 3, b, h, f), (ch, fw, D))
                x[f] = fr
            out[b, h] = store(x.reshape(wl.N, D), wl.dtype)
    return out


def scaled(wl: Workload, **changes) -> Workload:
    """A smaller (or otherwise changed) copy of a workload with the same recipe."""
    return dataclasses.replace(wl, **changes)
