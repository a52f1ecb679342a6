"""GPU LinVideo mixed attention vs the oracle.

r * (block-sparse softmax attention) + (1 - r) * (elu+1 linear attention), the
two terms taken from their own oracles and blended by the oracle's
``mixed_attention``.  The library writes the softmax output to ``out`` in bf16
and blends it with the linear output in fp32 before the final bf16 rounding."""

import math

import numpy as np
import pytest
import torch

from helpers import assert_parity, inputs_f64, to_device, to_f64
from oracle import attention as oa
from oracle import linear as ol
from oracle import mask as om
from synth import gen, get_workload

pytestmark = pytest.mark.gpu


def _case(bsa, wl, params, r, rows=None):
    d = gen.make_qkv(wl)
    q, k, v = (to_device(d[n], "bf16") for n in ("q", "k", "v"))
    rp, ci, ro = bsa.build_block_mask(params, with_order=True)
    out = bsa.mixed_attn_fwd(q, k, v, r, rp, ci, params["block"], row_order=ro)
    torch.cuda.synchronize()
    qf, kf, vf = inputs_f64(d, "bf16")
    m = om.block_mask(om.spec_from_params(params))
    blocks = None if rows is None else sorted({int(i) // params["block"] for i in rows})
    soft, _ = oa.block_sparse_attention(qf, kf, vf, m, params["block"], 1.0 / math.sqrt(wl.D), blocks)
    lin, _, _ = ol.linear_attention(qf, kf, vf)
    ref = ol.mixed_attention(soft, lin, r)
    got = to_f64(out)
    if rows is not None:
        got, ref = got[:, :, rows], ref[:, :, rows]
    return got, ref


def _lvsa(wl, block=128):
    return dict(kind=1, frames=wl.frames, frame_tokens=wl.P, block=block, window=1,
                anchor_period=2, anchor_step=1, anchor_rows=1, radial_w=0)


@pytest.mark.parametrize("r", [0.0, 0.3, 0.75, 1.0])
def test_blend_weights(gpu_lib, r):
    wl = gen.scaled(get_workload("lvsa_32k"), H=3, frames=4, frame_h=10, frame_w=13, seed=71)
    got, ref = _case(gpu_lib, wl, _lvsa(wl), r)
    assert_parity(got, ref, "bf16", f"mixed r={r}")


@pytest.mark.parametrize("block", [64, 128])
def test_ragged_radial(gpu_lib, block):
    wl = gen.scaled(get_workload("lvsa_32k"), H=2, frames=5, frame_h=7, frame_w=9, seed=72)
    p = dict(kind=2, frames=5, frame_tokens=63, block=block, window=0, anchor_period=0,
             anchor_step=0, anchor_rows=0, radial_w=20)
    got, ref = _case(gpu_lib, wl, p, 0.5)
    assert_parity(got, ref, "bf16", f"mixed radial block={block}")


def test_r_zero_equals_linear_and_r_one_equals_sparse(gpu_lib):
    """The two ends reproduce the separate entry points bit for bit."""
    wl = gen.scaled(get_workload("lvsa_32k"), H=2, frames=3, frame_h=8, frame_w=16, seed=73)
    d = gen.make_qkv(wl)
    q, k, v = (to_device(d[n], "bf16") for n in ("q", "k", "v"))
    p = _lvsa(wl)
    rp, ci, ro = gpu_lib.build_block_mask(p, with_order=True)
    lin = gpu_lib.linear_attn_fwd(q, k, v, return_state=False)
    soft, _ = gpu_lib.block_sparse_attn_fwd(q, k, v, rp, ci, 128, None, row_order=ro)
    m0 = gpu_lib.mixed_attn_fwd(q, k, v, 0.0)
    m1 = gpu_lib.mixed_attn_fwd(q, k, v, 1.0, rp, ci, 128, row_order=ro)
    torch.cuda.synchronize()
    assert torch.equal(m0.view(torch.int16), lin.view(torch.int16))
    assert torch.equal(m1.view(torch.int16), soft.view(torch.int16))


def test_mixed_32k_sampled_rows(gpu_lib):
    """The 32,760-token LVSA workload at r = 0.5 on sampled query rows (every head)."""
    wl = get_workload("lvsa_32k")
    rows = np.sort(np.random.default_rng(74).choice(wl.N, 48, replace=False))
    rows = np.concatenate([rows, [0, wl.N - 1]])
    got, ref = _case(gpu_lib, wl, wl.mask_params(0), 0.5, rows=rows)
    assert_parity(got, ref, "bf16", "mixed 32k")
