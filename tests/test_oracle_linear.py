"""Pins for the oracle's elu+1 linear attention (CPU only)."""

import math

import numpy as np
import torch

from oracle import linear as ol


def _qkv(seed, N, D, H=1):
    r = np.random.default_rng(seed)
    return [r.standard_normal((1, H, N, D)) for _ in range(3)]


def test_phi_matches_library_elu_plus_one():
    x = np.linspace(-6, 6, 1001)
    ref = torch.nn.functional.elu(torch.from_numpy(x), alpha=1.0).numpy() + 1.0
    assert np.abs(ol.phi(x) - ref).max() < 1e-15
    assert (ol.phi(x) > 0).all()


def test_closed_form_equals_quadratic_form():
    """phi(q)^T S / phi(q)^T z == sum_m (phi(q).phi(k_m)) v_m / sum_m phi(q).phi(k_m), by loops."""
    q, k, v = _qkv(0, 9, 5)
    out, S, z = ol.linear_attention(q, k, v)

    def phi1(x):
        return x + 1.0 if x > 0 else math.exp(x)

    for n in range(9):
        w = []
        for m in range(9):
            w.append(sum(phi1(q[0, 0, n, d]) * phi1(k[0, 0, m, d]) for d in range(5)))
        den = sum(w)
        for e in range(5):
            num = sum(w[m] * v[0, 0, m, e] for m in range(9))
            assert abs(num / den - out[0, 0, n, e]) < 1e-12


def test_state_definitions_by_loops():
    q, k, v = _qkv(1, 7, 4)
    _, S, z = ol.linear_attention(q, k, v)
    S2, z2 = ol.linear_state(k[0, 0], v[0, 0])   # the state alone, on one head
    for d in range(4):
        # phi by its branch definition, written out per element
        zd = sum((k[0, 0, n, d] + 1.0) if k[0, 0, n, d] > 0 else math.exp(k[0, 0, n, d]) for n in range(7))
        assert abs(z[0, 0, d] - zd) < 1e-12 and abs(z2[d] - zd) < 1e-12
        for e in range(4):
            sde = sum(((k[0, 0, n, d] + 1.0) if k[0, 0, n, d] > 0 else math.exp(k[0, 0, n, d])) * v[0, 0, n, e]
                      for n in range(7))
            assert abs(S[0, 0, d, e] - sde) < 1e-12 and abs(S2[d, e] - sde) < 1e-12


def test_special_cases():
    q, k, v = _qkv(2, 33, 8, H=2)
    out, _, _ = ol.linear_attention(q, k, np.ones_like(v))
    assert np.abs(out - 1.0).max() < 1e-12                     # V == 1 -> out == 1
    out1, _, _ = ol.linear_attention(q[:, :, :1], k[:, :, :1], v[:, :, :1])
    assert np.abs(out1 - v[:, :, :1]).max() < 1e-12            # one token -> its value
    o, _, _ = ol.linear_attention(q, k, v)
    o3, _, _ = ol.linear_attention(q, k, 3.0 * v)
    assert np.abs(o3 - 3.0 * o).max() < 1e-12                  # linear in V
    # the output is a convex combination of values: inside their per-column range
    assert (o <= v.max(axis=2, keepdims=True) + 1e-12).all()
    assert (o >= v.min(axis=2, keepdims=True) - 1e-12).all()


def test_rows_from_state():
    q, k, v = _qkv(3, 20, 6)
    out, S, z = ol.linear_attention(q, k, v)
    rows = ol.linear_attention_rows(q[0, 0, 5:9], S[0, 0], z[0, 0])
    assert np.abs(rows - out[0, 0, 5:9]).max() < 1e-13
