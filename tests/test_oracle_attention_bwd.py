"""Pins of the block-sparse attention backward oracle (CPU).

The gradients are pinned against torch autograd (float64) through a masked
softmax attention written with torch ops, against central finite differences
of the (independently pinned) forward oracle, and by invariants of softmax
attention that a dropped term, a wrong sign or a transposed operand breaks."""

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import attention_bwd as ob
from oracle import mask as om


def _case(N, D, block, seed, density=0.5, diag=True):
    r = np.random.default_rng(seed)
    q, k, v, do = (r.standard_normal((1, 2, N, D)) for _ in range(4))
    nb = -(-N // block)
    m = r.random((nb, nb)) < density
    if diag:
        np.fill_diagonal(m, True)
    return q, k, v, do, m


@pytest.mark.parametrize("N,D,block,seed", [(50, 8, 16, 0), (64, 4, 16, 1), (37, 6, 8, 2), (96, 16, 32, 3)])
def test_matches_torch_autograd(N, D, block, seed):
    q, k, v, do, m = _case(N, D, block, seed)
    scale = 1.0 / np.sqrt(D)
    tm = np.kron(m, np.ones((block, block), bool))[:N, :N]
    tq, tk, tv = (torch.tensor(t, requires_grad=True) for t in (q, k, v))
    s = scale * tq @ tk.transpose(-1, -2)
    s = s.masked_fill(~torch.tensor(tm), float("-inf"))
    out = torch.softmax(s, dim=-1) @ tv
    (out * torch.tensor(do)).sum().backward()
    dq, dk, dv = ob.block_sparse_attention_backward(q, k, v, do, m, block, scale)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.allclose(mine, ref.numpy(), rtol=1e-11, atol=1e-11)


def test_matches_finite_differences_of_the_forward():
    q, k, v, do, m = _case(40, 5, 8, 4, density=0.4)
    scale = 0.37
    dq, dk, dv = ob.block_sparse_attention_backward(q, k, v, do, m, 8, scale)

    def loss(qq, kk, vv):
        out, _ = oa.block_sparse_attention(qq, kk, vv, m, 8, scale)
        return float((out * do).sum())

    r = np.random.default_rng(5)
    h = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(6):
            idx = (0, int(r.integers(2)), int(r.integers(40)), int(r.integers(5)))
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            args[name][idx] += h
            up = loss(args["q"], args["k"], args["v"])
            args[name][idx] -= 2 * h
            dn = loss(args["q"], args["k"], args["v"])
            assert abs((up - dn) / (2 * h) - grad[idx]) < 1e-6 * max(1.0, abs(grad[idx]))


def test_invariants():
    q, k, v, do, m = _case(64, 8, 16, 6)
    dq, dk, dv = ob.block_sparse_attention_backward(q, k, v, do, m, 16, 0.3)
    # adding one vector to every key of a row's key set shifts its logits by a
    # constant: the key gradients of each query block sum to zero, so all do
    assert np.allclose(dk.sum(axis=2), 0.0, atol=1e-10)
    # probabilities sum to one over the kept keys: value gradients sum to the
    # output gradients of the rows that have keys
    assert np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-10)
    z = ob.block_sparse_attention_backward(q, k, v, np.zeros_like(do), m, 16, 0.3)
    assert all(np.array_equal(t, np.zeros_like(t)) for t in z)
    # identical keys: the softmax does not depend on q
    k1 = np.repeat(k[:, :, :1], 64, axis=2)
    dq1, _, _ = ob.block_sparse_attention_backward(q, k1, v, do, m, 16, 0.3)
    assert np.abs(dq1).max() < 1e-12


def test_rows_without_keys_get_no_gradient_and_skipped_keys_get_none():
    q, k, v, do, m = _case(48, 4, 16, 7, diag=False)
    m[1, :] = False                      # query block 1 has no keys
    m[:, 2] = False                      # key block 2 is kept by nobody
    dq, dk, dv = ob.block_sparse_attention_backward(q, k, v, do, m, 16, 0.5)
    assert np.array_equal(dq[:, :, 16:32], np.zeros_like(dq[:, :, 16:32]))
    assert np.array_equal(dk[:, :, 32:48], np.zeros_like(dk[:, :, 32:48]))
    assert np.array_equal(dv[:, :, 32:48], np.zeros_like(dv[:, :, 32:48]))


def test_transpose_csr():
    r = np.random.default_rng(8)
    m = r.random((9, 9)) < 0.4
    rp, ci = om.to_csr(m)
    tp, ti = ob.transpose_csr(rp, ci, 9)
    tp2, ti2 = om.to_csr(m.T)
    assert np.array_equal(tp, tp2) and np.array_equal(ti, ti2)


def test_stored_bf16_output_changes_only_delta():
    """With Delta taken from the bf16-rounded output, dS changes by -P * eps per
    row (eps = rowsum(dO * (bf16(O) - O))), so dq moves by -scale * eps * (P K),
    dk by -scale * (P * eps)^T Q and dv not at all: checked against the exact
    gradients with P, O and eps formed from the dense masked softmax."""
    from oracle.numerics import round_bf16
    q, k, v, do, m = _case(48, 8, 16, 9, density=1.1)           # every block kept: plain dense attention
    scale = 0.3
    ex = ob.block_sparse_attention_backward(q, k, v, do, m, 16, scale)
    bf = ob.block_sparse_attention_backward(q, k, v, do, m, 16, scale, o_dtype="bf16")
    s = scale * np.einsum("bhnd,bhmd->bhnm", q, k)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    o = p @ v
    eps = (do * (round_bf16(o) - o)).sum(-1, keepdims=True)
    assert np.allclose(bf[0] - ex[0], -scale * eps * (p @ k), rtol=1e-9, atol=1e-12)
    assert np.allclose(bf[1] - ex[1], -scale * np.einsum("bhnm,bhnd->bhmd", p * eps, q), rtol=1e-9, atol=1e-12)
    assert np.array_equal(bf[2], ex[2])
    assert np.abs(eps).max() > 0
