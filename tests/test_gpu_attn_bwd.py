"""GPU block-sparse attention backward vs the oracle.

The transposed CSR is integer (bit-exact).  Gradients are compared with the
float64 oracle on the same bf16 inputs; the GPU backward takes the forward
output and LSE of the GPU forward, as a training step would, and the oracle
takes Delta from its own forward output rounded to bf16 (the stored output).  Bar, derived from the
arithmetic: P and dS enter the MFMA as bf16 (relative rounding 2^-9 per
element) and are summed over hundreds to thousands of keys or queries with
random signs, so the error is a small fraction of the gradient's scale, not of
each element: relative L2 <= 1e-2 and max-abs <= 2e-2 x the largest |reference|
per tensor."""

import math

import numpy as np
import pytest
import torch

from helpers import inputs_f64, parity, to_device, to_f64
from oracle import attention_bwd as ob
from oracle import mask as om
from synth import gen, get_workload

pytestmark = pytest.mark.gpu


def _assert_grad(got, ref, what):
    """Relative L2 <= 1e-2 and max-abs <= 2e-2 x max|ref| per gradient tensor.
    The max-abs bar scales with the tensor: dK and dV reach max|ref| of 7-9
    here, where rounding a stored bf16 value alone is up to 1.8e-2; measured
    max-abs errors are 0.6-2.5e-2 and relative L2 2.3-5.8e-3."""
    ma, rl = parity(got, ref)
    scale = np.abs(ref).max()
    assert np.isfinite(got).all(), what
    assert rl <= 1e-2 and ma <= 2e-2 * scale, f"{what}: max_abs={ma:.3e} (ref max {scale:.3e}) rel_l2={rl:.3e}"


def _run(bsa, wl, params, seed=0, heads=None):
    d = gen.make_qkv(wl)
    r = np.random.default_rng(1000 + seed)
    do_bits = gen.store(r.standard_normal((wl.B, wl.H, wl.N, wl.D)).astype(np.float32), "bf16")
    q, k, v = (to_device(d[n], "bf16") for n in ("q", "k", "v"))
    do = to_device(do_bits, "bf16")
    rp, ci, ro = bsa.build_block_mask(params, with_order=True)
    o, lse = bsa.block_sparse_attn_fwd(q, k, v, rp, ci, 128, None, row_order=ro)
    cp, ri = bsa.transpose_block_mask(rp, ci)
    dq, dk, dv = bsa.block_sparse_attn_bwd(q, k, v, o, do, lse, rp, ci, 128, col_ptr=cp, row_idx=ri)
    torch.cuda.synchronize()
    m = om.block_mask(om.spec_from_params(params))
    qf, kf, vf = inputs_f64(d, "bf16")
    dof = gen.to_f64(do_bits, "bf16")
    hs = slice(None) if heads is None else heads
    rq, rk, rv = ob.block_sparse_attention_backward(qf[:, hs], kf[:, hs], vf[:, hs], dof[:, hs], m, 128,
                                                    1.0 / math.sqrt(wl.D), o_dtype="bf16")
    return (to_f64(dq)[:, hs], to_f64(dk)[:, hs], to_f64(dv)[:, hs]), (rq, rk, rv), (rp, ci, cp, ri, m)


def _lvsa(wl, window=1):
    return dict(kind=1, frames=wl.frames, frame_tokens=wl.P, block=128, window=window,
                anchor_period=2, anchor_step=1, anchor_rows=1, radial_w=0)


@pytest.mark.parametrize("frames,fh,fw,kind", [(4, 10, 13, "lvsa"), (5, 7, 9, "radial"), (3, 8, 16, "all"),
                                               (6, 9, 11, "cols")])
def test_small_against_oracle(gpu_lib, frames, fh, fw, kind):
    wl = gen.scaled(get_workload("lvsa_32k"), H=2, frames=frames, frame_h=fh, frame_w=fw, seed=50 + frames)
    if kind == "lvsa":
        p = _lvsa(wl)
    elif kind == "radial":
        p = dict(kind=2, frames=frames, frame_tokens=wl.P, block=128, window=0, anchor_period=0, anchor_step=0,
                 anchor_rows=0, radial_w=20)
    elif kind == "all":
        p = dict(kind=0, frames=frames, frame_tokens=wl.P, block=128, window=0, anchor_period=0, anchor_step=0,
                 anchor_rows=0, radial_w=0)
    else:  # column-only anchors: an asymmetric mask
        p = dict(_lvsa(wl, window=0), anchor_rows=0, anchor_period=3, anchor_step=0)
    got, ref, _ = _run(gpu_lib, wl, p, seed=frames)
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        _assert_grad(g, r, f"{kind} {name}")


def test_transposed_csr_is_exact(gpu_lib):
    wl = gen.scaled(get_workload("lvsa_32k"), H=1, frames=9, frame_h=11, frame_w=23, seed=61)
    for p in (dict(_lvsa(wl), anchor_rows=0, window=2, anchor_period=4),
              dict(kind=2, frames=9, frame_tokens=wl.P, block=128, window=0, anchor_period=0, anchor_step=0,
                   anchor_rows=0, radial_w=60)):
        rp, ci, _ = gpu_lib.build_block_mask(p, with_order=True)
        cp, ri = gpu_lib.transpose_block_mask(rp, ci)
        torch.cuda.synchronize()
        rph, cih = rp.cpu().numpy(), ci.cpu().numpy()
        tp, ti = ob.transpose_csr(rph, cih[: rph[-1]], len(rph) - 1)
        assert np.array_equal(cp.cpu().numpy(), tp)
        assert np.array_equal(ri.cpu().numpy()[: tp[-1]], ti)


def test_lvsa_32k_head_against_oracle(gpu_lib):
    """The 32,760-token LVSA workload, all 12 heads on the GPU; heads 0 and 7
    against the oracle (every element)."""
    wl = get_workload("lvsa_32k")
    got, ref, _ = _run(gpu_lib, wl, wl.mask_params(1), seed=7, heads=[0, 7])
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        _assert_grad(g, r, f"lvsa_32k {name}")


def test_deterministic(gpu_lib):
    wl = gen.scaled(get_workload("lvsa_32k"), H=2, frames=5, frame_h=12, frame_w=20, seed=62)
    d = gen.make_qkv(wl)
    q, k, v = (to_device(d[n], "bf16") for n in ("q", "k", "v"))
    do = torch.randn_like(q.float()).to(torch.bfloat16)
    rp, ci, ro = gpu_lib.build_block_mask(_lvsa(wl), with_order=True)
    o, lse = gpu_lib.block_sparse_attn_fwd(q, k, v, rp, ci, 128, None, row_order=ro)
    a = gpu_lib.block_sparse_attn_bwd(q, k, v, o, do, lse, rp, ci)
    b = gpu_lib.block_sparse_attn_bwd(q, k, v, o, do, lse, rp, ci)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("B,H,frames,fh,fw", [(2, 1, 2, 5, 10), (2, 3, 1, 1, 7)])
def test_batches_and_single_block(gpu_lib, B, H, frames, fh, fw):
    """Batch > 1 and sequences of one (ragged) block."""
    wl = gen.scaled(get_workload("lvsa_32k"), B=B, H=H, frames=frames, frame_h=fh, frame_w=fw, seed=70 + B + H)
    p = dict(kind=0, frames=frames, frame_tokens=wl.P, block=128, window=0, anchor_period=0, anchor_step=0,
             anchor_rows=0, radial_w=0)
    got, ref, _ = _run(gpu_lib, wl, p, seed=B * 10 + H)
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        _assert_grad(g, r, f"B={B} {name}")
