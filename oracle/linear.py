"""Oracle: non-causal elu+1 linear attention (float64).

Test infrastructure only (see the package docstring).

The LinVideo page (technical summary, sections 1-2) replaces quadratic softmax
attention with linear attention of O(n) cost; the page gives no feature map, so
the workload fixes phi(x) = elu(x) + 1, i.e. x + 1 for x > 0 and exp(x) for
x <= 0.  Associativity turns sum_m phi(q).phi(k_m) v_m into phi(q)^T S with

    S = sum_n phi(k_n) v_n^T   (D x D),   z = sum_n phi(k_n)   (D),
    out_n = phi(q_n)^T S / (phi(q_n)^T z).

No softmax scale is applied.  phi > 0, so the denominator is positive.
"""

import numpy as np


def phi(x):
    x = np.asarray(x, np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def linear_state(k, v):
    """The state of the sequence: S [..., D, D] = sum_n phi(k_n) v_n^T and
    z [..., D] = sum_n phi(k_n), for float64 [..., N, D] keys and values."""
    fk = phi(k)
    v = np.asarray(v, np.float64)
    return np.einsum("...nd,...ne->...de", fk, v), fk.sum(axis=-2)


def linear_attention(q, k, v):
    """out [B, H, N, D], S [B, H, D, D], z [B, H, D] for float64 [B, H, N, D] inputs."""
    fq = phi(q)
    S, z = linear_state(k, v)
    num = np.einsum("bhnd,bhde->bhne", fq, S)
    den = np.einsum("bhnd,bhd->bhn", fq, z)
    return num / den[..., None], S, z


def linear_attention_rows(q_rows, S, z):
    """Apply a given state (S, z) to some query rows (float64 [..., D])."""
    fq = phi(q_rows)
    return (fq @ S) / (fq @ z)[..., None]


def causal_linear_attention(q, k, v, rows=None, S0=None, z0=None):
    """Causal elu+1 linear attention, float64 [B, H, N, D] inputs.

    Each query sees only itself and the tokens before it:
        out_n = sum_{m <= n} (phi(q_n) . phi(k_m)) v_m / sum_{m <= n} phi(q_n) . phi(k_m)
    which is phi(q_n)^T S_n / phi(q_n)^T z_n with prefix states S_n, z_n (the
    causal form used by autoregressive video models such as the Self-Forcing
    setting of the LIPAR page).  Written out as that quadratic form, one query
    row at a time; ``rows`` restricts the computation to some query rows (the
    others are NaN).

    Chunked use carries the state of the tokens before this sequence: with
    S0 [B, H, D, D] and z0 [B, H, D] (sums of phi(k) v^T and phi(k) over the
    earlier tokens) every row also sees them:
        out_n = (phi(q_n)^T S0 + sum_{m <= n} w_nm v_m) / (phi(q_n)^T z0 + sum_{m <= n} w_nm).
    The state after the sequence is S0 + S, z0 + z with S, z of
    ``linear_attention``.
    """
    fq, fk = phi(q), phi(k)
    v = np.asarray(v, np.float64)
    B, H, N, D = fq.shape
    E = v.shape[-1]
    S0 = np.zeros((B, H, D, E)) if S0 is None else np.asarray(S0, np.float64)
    z0 = np.zeros((B, H, D)) if z0 is None else np.asarray(z0, np.float64)
    out = np.full((B, H, N, E), np.nan)
    for n in (range(N) if rows is None else rows):
        w = np.einsum("bhd,bhmd->bhm", fq[:, :, n], fk[:, :, : n + 1])
        num = np.einsum("bhm,bhme->bhe", w, v[:, :, : n + 1]) + np.einsum("bhd,bhde->bhe", fq[:, :, n], S0)
        den = w.sum(axis=2) + np.einsum("bhd,bhd->bh", fq[:, :, n], z0)
        out[:, :, n] = num / den[..., None]
    return out


def mixed_attention(soft_out, lin_out, r: float):
    """LinVideo mixed attention (technical summary, section 2 A. Selective
    Transfer): a per-layer scalar r in [0, 1] blends quadratic attention
    (r = 1) and linear attention (r = 0): r * soft_out + (1 - r) * lin_out."""
    return r * np.asarray(soft_out, np.float64) + (1.0 - r) * np.asarray(lin_out, np.float64)
