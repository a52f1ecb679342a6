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


def linear_attention(q, k, v):
    """out [B, H, N, D], S [B, H, D, D], z [B, H, D] for float64 [B, H, N, D] inputs."""
    fq, fk = phi(q), phi(k)
    v = np.asarray(v, np.float64)
    S = np.einsum("bhnd,bhne->bhde", fk, v)
    z = fk.sum(axis=2)
    num = np.einsum("bhnd,bhde->bhne", fq, S)
    den = np.einsum("bhnd,bhd->bhn", fq, z)
    return num / den[..., None], S, z


def linear_attention_rows(q_rows, S, z):
    """Apply a given state (S, z) to some query rows (float64 [..., D])."""
    fq = phi(q_rows)
    return (fq @ S) / (fq @ z)[..., None]
