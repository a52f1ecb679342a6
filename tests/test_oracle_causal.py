"""Pins of the causal linear attention and mixed attention oracles (CPU)."""

import numpy as np
import pytest

from oracle import attention as oa
from oracle import linear as ol


def _qkv(B, H, N, D, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, H, N, D)) for _ in range(3))


def test_first_row_is_the_first_value():
    q, k, v = _qkv(1, 2, 9, 5, 0)
    out = ol.causal_linear_attention(q, k, v)
    assert np.allclose(out[:, :, 0], v[:, :, 0], rtol=0, atol=1e-12)


def test_row_n_is_noncausal_attention_over_the_prefix():
    """The causal output of row n equals the non-causal linear attention of the
    first n + 1 tokens at their last row (an independently pinned oracle)."""
    q, k, v = _qkv(2, 1, 11, 4, 1)
    out = ol.causal_linear_attention(q, k, v)
    for n in range(11):
        ref, _, _ = ol.linear_attention(q[:, :, : n + 1], k[:, :, : n + 1], v[:, :, : n + 1])
        assert np.allclose(out[:, :, n], ref[:, :, n], rtol=1e-12, atol=1e-12)


def test_constant_values_and_convex_bounds():
    q, k, _ = _qkv(1, 1, 13, 6, 2)
    v = np.ones((1, 1, 13, 6))
    assert np.allclose(ol.causal_linear_attention(q, k, v), 1.0, atol=1e-12)
    _, _, v = _qkv(1, 1, 13, 6, 3)
    out = ol.causal_linear_attention(q, k, v)
    for n in range(13):  # a convex combination of v_0 .. v_n (phi > 0)
        assert (out[0, 0, n] <= v[0, 0, : n + 1].max(axis=0) + 1e-12).all()
        assert (out[0, 0, n] >= v[0, 0, : n + 1].min(axis=0) - 1e-12).all()


def test_brute_force_loops():
    q, k, v = _qkv(1, 1, 6, 3, 4)

    def phi(x):
        return x + 1.0 if x > 0 else np.exp(x)

    out = ol.causal_linear_attention(q, k, v)
    for n in range(6):
        num = np.zeros(3)
        den = 0.0
        for m in range(n + 1):
            w = sum(phi(q[0, 0, n, d]) * phi(k[0, 0, m, d]) for d in range(3))
            num += w * v[0, 0, m]
            den += w
        assert np.allclose(out[0, 0, n], num / den, rtol=1e-12)


def test_row_subset_matches_full():
    q, k, v = _qkv(1, 2, 20, 4, 5)
    full = ol.causal_linear_attention(q, k, v)
    part = ol.causal_linear_attention(q, k, v, rows=[0, 7, 19])
    assert np.array_equal(part[:, :, [0, 7, 19]], full[:, :, [0, 7, 19]])
    assert np.isnan(part[:, :, 1]).all()


@pytest.mark.parametrize("r", [0.0, 1.0, 0.3])
def test_mixed_endpoints_and_affinity(r):
    q, k, v = _qkv(1, 2, 32, 8, 6)
    mask = np.ones((2, 2), bool)
    soft, _ = oa.block_sparse_attention(q, k, v, mask, 16, 1 / np.sqrt(8))
    dense, _ = oa.dense_attention(q, k, v, 1 / np.sqrt(8))
    lin, _, _ = ol.linear_attention(q, k, v)
    mixed = ol.mixed_attention(soft, lin, r)
    assert np.allclose(mixed, r * dense + (1 - r) * lin, rtol=1e-12, atol=1e-12)
    if r == 1.0:
        assert np.array_equal(mixed, soft)
    if r == 0.0:
        assert np.array_equal(mixed, lin)


@pytest.mark.parametrize("cut", [1, 5, 12])
def test_carried_state_continues_the_sequence(cut):
    """Running the tokens after ``cut`` with the state of the tokens before it
    (taken from the pinned non-causal oracle) gives the causal output of the
    whole sequence on those rows."""
    q, k, v = _qkv(2, 2, 17, 4, 7)
    whole = ol.causal_linear_attention(q, k, v)
    _, S0, z0 = ol.linear_attention(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut])
    tail = ol.causal_linear_attention(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], S0=S0, z0=z0)
    assert np.allclose(tail, whole[:, :, cut:], rtol=1e-12, atol=1e-12)


def test_carried_state_brute_force():
    """A given (S0, z0) enters numerator and denominator as phi(q).S0 and phi(q).z0."""
    q, k, v = _qkv(1, 1, 4, 3, 8)
    r = np.random.default_rng(9)
    S0 = r.random((1, 1, 3, 3)) * 5
    z0 = r.random((1, 1, 3)) * 5 + 0.5

    def phi(x):
        return x + 1.0 if x > 0 else np.exp(x)

    out = ol.causal_linear_attention(q, k, v, S0=S0, z0=z0)
    for n in range(4):
        fq = [phi(q[0, 0, n, d]) for d in range(3)]
        num = np.array([sum(fq[d] * S0[0, 0, d, e] for d in range(3)) for e in range(3)])
        den = sum(fq[d] * z0[0, 0, d] for d in range(3))
        for m in range(n + 1):
            w = sum(fq[d] * phi(k[0, 0, m, d]) for d in range(3))
            num = num + w * v[0, 0, m]
            den += w
        assert np.allclose(out[0, 0, n], num / den, rtol=1e-12)
