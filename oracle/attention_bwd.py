"""Oracle: gradients of block-sparse softmax attention (float64).

Test infrastructure only (see the package docstring).

The training uses on the pages need the backward pass of the sparse attention
they describe: Radial attention is adapted to longer videos by LoRA
fine-tuning (the hyper.ai Radial Attention headline), and LinVideo is a
post-training framework (technical summary sections 1-2).  With the forward of
``oracle.attention`` (per query block i, keys K(i) = the real keys of its kept
blocks; S = scale * Q_i K_K(i)^T, P = row softmax of S, O_i = P V_K(i)) and an
output gradient dO, the gradients are the chain rule written out:

    dV_K(i) += P^T dO_i
    dP = dO_i V_K(i)^T,  Delta = rowsum(P * dP)  (= rowsum(dO_i * O_i))
    dS = P * (dP - Delta)
    dQ_i = scale * dS K_K(i),   dK_K(i) += scale * dS^T Q_i

Keys of skipped blocks receive nothing from that query block; a query row
without keys has O = 0 and receives zero gradient.  Per query block the kept
key blocks are gathered and the products are float64 matrix products, in
query-block order.

Reading (``o_dtype="bf16"``): a bf16 training step keeps the forward output as
stored, in bf16, and takes Delta = rowsum(dO * O) from it (the identity with
rowsum(P * dP) holds for the exact O only); the oracle then rounds its own O to
bf16 before that row sum.  ``o_dtype=None`` uses the exact O.
"""

import numpy as np

from .attention import kept_keys, softmax_rows
from .numerics import round_bf16


def block_sparse_attention_backward(q, k, v, do, mask: np.ndarray, block: int, scale: float, o_dtype=None):
    """(dq, dk, dv) float64 [B, H, N, D] for float64 [B, H, N, D] q, k, v, do."""
    q, k, v, do = (np.asarray(t, np.float64) for t in (q, k, v, do))
    B, H, N, _ = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for i in range(mask.shape[0]):
        r0, r1 = i * block, min((i + 1) * block, N)
        keys = kept_keys(mask[i], block, N)
        if len(keys) == 0:
            continue
        for b in range(B):
            for h in range(H):
                qi, kk, vk, doi = q[b, h, r0:r1], k[b, h, keys], v[b, h, keys], do[b, h, r0:r1]
                p, _ = softmax_rows(scale * (qi @ kk.T))
                dv[b, h, keys] += p.T @ doi
                dp = doi @ vk.T
                if o_dtype == "bf16":
                    delta = (doi * round_bf16(p @ vk)).sum(axis=1, keepdims=True)
                else:
                    delta = (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - delta)
                dq[b, h, r0:r1] = scale * (ds @ kk)
                dk[b, h, keys] += scale * (ds.T @ qi)
    return dq, dk, dv


def transpose_csr(row_ptr, col_idx, nb: int):
    """CSR of the transposed block mask: for every key block the query blocks that
    keep it, ascending."""
    row_ptr = np.asarray(row_ptr)
    col_idx = np.asarray(col_idx)
    cols = [[] for _ in range(nb)]
    for i in range(nb):
        for j in col_idx[row_ptr[i]:row_ptr[i + 1]]:
            cols[int(j)].append(i)
    ptr = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int64)
    idx = np.array([i for c in cols for i in c], dtype=np.int64)
    return ptr, idx
