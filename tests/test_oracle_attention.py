"""Pins for the oracle's block-sparse attention (CPU only)."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import mask as om


def _qkv(seed, B, H, N, D, scale=1.0):
    r = np.random.default_rng(seed)
    return [scale * r.standard_normal((B, H, N, D)) for _ in range(3)]


def test_all_kept_equals_library_sdpa():
    """Every block kept -> dense softmax attention (torch SDPA, float64, CPU)."""
    B, H, N, D, b = 1, 2, 70, 16, 16          # ragged tail: 70 = 4*16 + 6
    q, k, v = _qkv(0, B, H, N, D)
    nb = -(-N // b)
    out, _ = oa.block_sparse_attention(q, k, v, np.ones((nb, nb), bool), b, 1 / math.sqrt(D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=1 / math.sqrt(D))
    assert np.abs(out - ref.numpy()).max() < 1e-12


def test_masked_blocks_match_per_element_masking():
    """Block-wise oracle == textbook attention with the expanded token mask (-inf logits)."""
    spec = om.MaskSpec(kind=om.WINDOW_ANCHOR, frames=5, frame_tokens=7, block=4, window=1,
                       anchor_period=3, anchor_step=1, anchor_rows=0)
    m = om.block_mask(spec)
    N, b = spec.N, spec.block
    tok = np.array([[m[i // b, j // b] for j in range(N)] for i in range(N)])
    q, k, v = _qkv(1, 1, 2, N, 8)
    out, lse = oa.block_sparse_attention(q, k, v, m, b, 0.3)
    ref, rlse = oa.dense_attention(q, k, v, 0.3, tok)
    assert np.abs(out - ref).max() < 1e-12 and np.abs(lse - rlse).max() < 1e-12


def test_bruteforce_loops_tiny():
    """Pure-Python per-query loop over the kept keys (no matrix products)."""
    spec = om.MaskSpec(kind=om.RADIAL, frames=3, frame_tokens=5, block=2, radial_w=1)
    m = om.block_mask(spec)
    q, k, v = _qkv(2, 1, 1, spec.N, 3)
    out, lse = oa.block_sparse_attention(q, k, v, m, 2, 0.7)
    for t in range(spec.N):
        keys = [u for u in range(spec.N) if m[t // 2, u // 2]]
        logits = [0.7 * sum(q[0, 0, t, d] * k[0, 0, u, d] for d in range(3)) for u in keys]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        z = sum(w)
        for d in range(3):
            o = sum(wi * v[0, 0, u, d] for wi, u in zip(w, keys)) / z
            assert abs(o - out[0, 0, t, d]) < 1e-12
        assert abs(mx + math.log(z) - lse[0, 0, t]) < 1e-12


def test_rows_sum_to_one_and_constant_values():
    spec = om.MaskSpec(kind=om.RADIAL, frames=4, frame_tokens=9, block=4, radial_w=3)
    m = om.block_mask(spec)
    q, k, _ = _qkv(3, 1, 2, spec.N, 8, scale=3.0)
    ones = np.ones_like(q)
    out, _ = oa.block_sparse_attention(q, k, ones, m, 4, 0.5)
    assert np.abs(out - 1.0).max() < 1e-12                     # V == 1 -> out == 1
    # probabilities: one-hot V columns recover the row sums of P
    N = spec.N
    eye = np.zeros((1, 2, N, N))
    eye[0, :, np.arange(N), np.arange(N)] = 1.0
    p, _ = oa.block_sparse_attention(q, k, eye, m, 4, 0.5)
    assert np.abs(p.sum(-1) - 1.0).max() < 1e-12
    # and P is exactly zero on skipped blocks
    tok = np.array([[m[i // 4, j // 4] for j in range(N)] for i in range(N)])
    assert (p[0][:, ~tok] == 0).all()


def test_masked_out_blocks_contribute_nothing():
    spec = om.MaskSpec(kind=om.WINDOW_ANCHOR, frames=6, frame_tokens=8, block=8, window=1)
    m = om.block_mask(spec)
    q, k, v = _qkv(4, 1, 1, spec.N, 8)
    out, _ = oa.block_sparse_attention(q, k, v, m, 8, 0.4)
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, 40:48] = 1e6                                      # block 5, unseen by rows 0..3
    v2[0, 0, 40:48] = np.nan
    out2, _ = oa.block_sparse_attention(q, k2, v2, m, 8, 0.4)
    assert np.array_equal(out[0, 0, :32], out2[0, 0, :32])


def test_one_dominant_key():
    q, k, v = _qkv(5, 1, 1, 16, 4)
    k[0, 0, 9] = 50.0 * q[0, 0, 3] / np.linalg.norm(q[0, 0, 3])
    out, _ = oa.block_sparse_attention(q, k, v, np.ones((2, 2), bool), 8, 1.0)
    assert np.abs(out[0, 0, 3] - v[0, 0, 9]).max() < 1e-9


def test_lse_is_log_partition():
    q, k, v = _qkv(6, 1, 1, 12, 4)
    m = np.array([[1, 0, 1], [1, 1, 0], [0, 0, 1]], bool)
    _, lse = oa.block_sparse_attention(q, k, v, m, 4, 0.9)
    for t in range(12):
        keys = [u for u in range(12) if m[t // 4, u // 4]]
        s = sum(math.exp(0.9 * float(q[0, 0, t] @ k[0, 0, u])) for u in keys)
        assert abs(math.exp(lse[0, 0, t]) - s) < 1e-9 * s


def test_empty_row():
    q, k, v = _qkv(7, 1, 1, 8, 4)
    m = np.array([[0, 0], [1, 1]], bool)
    out, lse = oa.block_sparse_attention(q, k, v, m, 4, 1.0)
    assert (out[0, 0, :4] == 0).all() and np.isneginf(lse[0, 0, :4]).all()


def test_kept_flops_counts_real_tokens_only():
    m = np.ones((3, 3), bool)
    # N = 20, block 8: sizes 8, 8, 4 -> pairs = 20 * 20
    assert oa.kept_flops(m, 8, 20, 16) == 4 * 16 * 400
    m[2, 2] = False
    assert oa.kept_flops(m, 8, 20, 16) == 4 * 16 * (400 - 16)


@pytest.mark.parametrize("query_blocks", [[0], [2, 5]])
def test_query_block_subset(query_blocks):
    spec = om.MaskSpec(kind=om.RADIAL, frames=4, frame_tokens=6, block=4, radial_w=2)
    m = om.block_mask(spec)
    q, k, v = _qkv(8, 1, 2, spec.N, 4)
    full, _ = oa.block_sparse_attention(q, k, v, m, 4, 0.5)
    part, _ = oa.block_sparse_attention(q, k, v, m, 4, 0.5, query_blocks=query_blocks)
    for i in query_blocks:
        assert np.array_equal(part[:, :, 4 * i:4 * i + 4], full[:, :, 4 * i:4 * i + 4])
