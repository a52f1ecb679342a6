"""GPU elu+1 linear attention vs the oracle."""

import numpy as np
import pytest
import torch

from helpers import assert_parity, inputs_f64, parity, to_device, to_f64
from oracle import linear as ol
from synth import gen, get_workload

pytestmark = pytest.mark.gpu


def _run(bsa, d, state=True):
    q, k, v = (to_device(d[n], "bf16") for n in ("q", "k", "v"))
    res = bsa.linear_attn_fwd(q, k, v, return_state=state)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("D,N", [(128, 1000), (64, 1000), (128, 64), (128, 7), (64, 130)])
def test_small_full_compare(gpu_lib, D, N):
    wl = gen.scaled(get_workload("linear_32k"), H=3, D=D, frames=1, frame_h=1, frame_w=N, seed=41)
    d = gen.make_qkv(wl)
    out, S, z = _run(gpu_lib, d)
    q, k, v = inputs_f64(d, "bf16")
    ref, rS, rz = ol.linear_attention(q, k, v)
    assert_parity(to_f64(out), ref, "bf16", f"linear D={D} N={N}")
    _, rel_s = parity(to_f64(S), rS)
    assert rel_s < 1e-2, rel_s                      # phi(K) enters the MFMA as bf16
    _, rel_z = parity(to_f64(z), rz)
    assert rel_z < 1e-5, rel_z                      # z accumulates phi in fp32


@pytest.mark.parametrize("k", [2, 3, 4, 6, 8, 9])
def test_every_copy_ring_remainder(gpu_lib, k):
    """64 heads split the state pass into 8 chunks of k 32-token tiles each
    (N = 256 k - 13, so the last tile is ragged): the state kernel's ring of
    copy stages then runs every loop remainder (k mod 5) and its tail path."""
    N = 256 * k - 13
    wl = gen.scaled(get_workload("linear_32k"), H=64, D=128, frames=1, frame_h=1, frame_w=N, seed=60 + k)
    d = gen.make_qkv(wl)
    out, S, z = _run(gpu_lib, d)
    q, kk, v = inputs_f64(d, "bf16")
    ref, rS, rz = ol.linear_attention(q, kk, v)
    assert_parity(to_f64(out), ref, "bf16", f"linear ring k={k}")
    _, rel_z = parity(to_f64(z), rz)
    assert rel_z < 1e-5, rel_z


def test_single_token_gives_its_value(gpu_lib):
    wl = gen.scaled(get_workload("linear_32k"), H=2, frames=1, frame_h=1, frame_w=1, seed=42)
    d = gen.make_qkv(wl)
    out = _run(gpu_lib, d, state=False)
    assert np.abs(to_f64(out) - gen.bf16_bits_to_f64(d["v"])).max() <= 2 ** -7 * np.abs(
        gen.bf16_bits_to_f64(d["v"])).max()


def test_constant_values(gpu_lib):
    wl = gen.scaled(get_workload("linear_32k"), H=2, frames=3, frame_h=10, frame_w=11, seed=43)
    d = dict(gen.make_qkv(wl))
    d["v"] = np.full_like(d["v"], 0x3F80)            # bf16 1.0
    out = _run(gpu_lib, d, state=False)
    assert np.abs(to_f64(out) - 1.0).max() < 1e-2


def test_deterministic(gpu_lib):
    wl = gen.scaled(get_workload("linear_32k"), H=2, frames=2, frame_h=30, frame_w=52, seed=44)
    d = gen.make_qkv(wl)
    a, sa, za = _run(gpu_lib, d)
    b, sb, zb = _run(gpu_lib, d)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(sa, sb) and torch.equal(za, zb)


def test_linear_32k_full(gpu_lib):
    """Every output of the 32,760-token workload (12 heads) against the oracle."""
    wl = get_workload("linear_32k")
    d = gen.make_qkv(wl)
    out, S, z = _run(gpu_lib, d)
    got = to_f64(out)
    for h in range(wl.H):
        q, k, v = (gen.to_f64(d[n][:, h:h + 1], "bf16") for n in ("q", "k", "v"))
        ref, rS, rz = ol.linear_attention(q, k, v)
        assert_parity(got[:, h:h + 1], ref, "bf16", f"linear_32k head {h}")
        assert parity(to_f64(S[:, h:h + 1]), rS)[1] < 1e-2


def test_linear_196k_sampled(gpu_lib):
    """196,560 tokens: full state per head, sampled query rows (first, middle, last tiles)."""
    wl = get_workload("linear_196k")
    d = gen.make_qkv(wl)
    out, S, z = _run(gpu_lib, d)
    rows = np.r_[0:300, 98000:98300, wl.N - 300:wl.N]
    got = to_f64(out[:, :, rows])
    for h in (0, 5, 11):
        k, v = (gen.to_f64(d[n][:, h:h + 1], "bf16") for n in ("k", "v"))
        rS, rz = ol.linear_state(k[0, 0], v[0, 0])
        q = gen.to_f64(d["q"][0, h, rows], "bf16")
        ref = ol.linear_attention_rows(q, rS, rz)
        assert_parity(got[0, h], ref, "bf16", f"linear_196k head {h}")
        assert parity(to_f64(z[0, h]), rz)[1] < 1e-5
