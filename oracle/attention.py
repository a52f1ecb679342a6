"""Oracle: block-sparse softmax self-attention (float64).

Test infrastructure only (see the package docstring).

What is computed (LVSA review page, section 1 Key Terms: block-sparse
attention; SVG-EAR page, technical summary section 1: sparse attention computes
some blocks and skips the rest).  For a query row q in block i, the key set is
K(q) = { real key t : block mask (i, blk(t)) kept }.  With logits
l_t = scale * q . k_t, m = max l, Z = sum_t exp(l_t - m):

    out(q) = sum_t exp(l_t - m) v_t / Z,     lse(q) = m + ln Z  (natural log).

Skipped blocks contribute nothing at all; padding keys past N do not exist.
A row whose key set is empty gets out = 0 and lse = -inf.

Per query block the kept key blocks are concatenated and the logits are one
float64 matrix product, then a row softmax; no blocking or reordering beyond
that.
"""

import numpy as np


def kept_keys(mask_row: np.ndarray, block: int, N: int) -> np.ndarray:
    """Real key token indices of the kept blocks of one mask row, ascending."""
    cols = np.nonzero(mask_row)[0]
    if len(cols) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(j * block, min((j + 1) * block, N)) for j in cols])


def softmax_rows(logits: np.ndarray):
    """Row softmax probabilities and natural-log LSE of a float64 matrix."""
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    return e / z, (m + np.log(z))[:, 0]


def block_sparse_attention(q, k, v, mask: np.ndarray, block: int, scale: float,
                           query_blocks=None):
    """out [B, H, N, D] and lse [B, H, N] (float64) for the rows of ``query_blocks``.

    q, k, v are float64 arrays [B, H, N, D].  ``mask`` is the boolean block mask
    [nb, nb] shared by every batch and head.  ``query_blocks`` restricts the
    computation to some block rows (the other outputs are left as NaN).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, N, _ = q.shape
    nb = mask.shape[0]
    out = np.full((B, H, N, v.shape[-1]), np.nan)
    lse = np.full((B, H, N), np.nan)
    rows = range(nb) if query_blocks is None else query_blocks
    for i in rows:
        r0, r1 = i * block, min((i + 1) * block, N)
        keys = kept_keys(mask[i], block, N)
        for b in range(B):
            for h in range(H):
                if len(keys) == 0:
                    out[b, h, r0:r1] = 0.0
                    lse[b, h, r0:r1] = -np.inf
                    continue
                s = scale * (q[b, h, r0:r1] @ k[b, h, keys].T)
                p, l = softmax_rows(s)
                out[b, h, r0:r1] = p @ v[b, h, keys]
                lse[b, h, r0:r1] = l
    return out, lse


def dense_attention(q, k, v, scale: float, token_mask=None):
    """Textbook softmax attention with an optional boolean [N, N] token mask.

    Written per element on purpose (masked logits set to -inf before the
    softmax) so that tests can compare the block-wise oracle against it.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = scale * np.einsum("bhnd,bhmd->bhnm", q, k)
    if token_mask is not None:
        s = np.where(token_mask[None, None], s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return np.einsum("bhnm,bhmd->bhnd", e / z, v), (m + np.log(z))[..., 0]


def kept_flops(mask: np.ndarray, block: int, N: int, D: int, B: int = 1, H: int = 1) -> int:
    """Effective FLOP of one call: 4 * D * sum over kept (i, j) of real rows * real columns."""
    nb = mask.shape[0]
    sizes = np.array([min((i + 1) * block, N) - i * block for i in range(nb)], dtype=np.int64)
    pairs = int((mask * sizes[:, None] * sizes[None, :]).sum())
    return 4 * D * pairs * B * H
