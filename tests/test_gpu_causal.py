"""GPU causal (chunked) elu+1 linear attention vs the oracle.

The oracle writes every output row as its quadratic form over the earlier
tokens (plus a carried state); the GPU path runs state partials, an exclusive
prefix over token splits and a 32-token causal walk per split."""

import numpy as np
import pytest
import torch

from helpers import assert_parity, inputs_f64, parity, to_device, to_f64
from oracle import linear as ol
from synth import gen, get_workload

pytestmark = pytest.mark.gpu


def _wl(H, N, seed):
    return gen.scaled(get_workload("linear_32k"), H=H, D=128, frames=1, frame_h=1, frame_w=N, seed=seed)


def _dev(d):
    return [to_device(d[n], "bf16") for n in ("q", "k", "v")]


@pytest.mark.parametrize("H,N", [(3, 1000), (1, 7), (2, 32), (2, 33), (12, 96), (1, 4100)])
def test_full_compare(gpu_lib, H, N):
    """Every row up to N = 1000 (sampled rows above): N = 4100 with one head
    gives 129 one-step splits; 12 heads at N = 96 one step per split."""
    d = gen.make_qkv(_wl(H, N, 80 + N))
    out, S, z = gpu_lib.causal_linear_attn_fwd(*_dev(d), return_state=True)
    torch.cuda.synchronize()
    q, k, v = inputs_f64(d, "bf16")
    rows = None if N <= 1000 else np.unique(np.concatenate([np.arange(0, 80), np.arange(N - 80, N),
                                                            np.random.default_rng(N).choice(N, 120)]))
    ref = ol.causal_linear_attention(q, k, v, rows=rows)
    got = to_f64(out)
    if rows is not None:
        got, ref = got[:, :, rows], ref[:, :, rows]
    assert_parity(got, ref, "bf16", f"causal H={H} N={N}")
    _, rS, rz = ol.linear_attention(q, k, v)       # the state after the last token
    assert parity(to_f64(S), rS)[1] < 1e-2
    assert parity(to_f64(z), rz)[1] < 1e-5


@pytest.mark.parametrize("N", [2035, 4051, 6074])
def test_every_ring_remainder(gpu_lib, N):
    """8 heads, 32 apply splits of 2, 4 and 6 steps of 32 tokens (every
    remainder of the three-stage ring, two state splits each) and a ragged
    last split of 2, 3 and 4 steps."""
    d = gen.make_qkv(_wl(8, N, 90 + N))
    out = gpu_lib.causal_linear_attn_fwd(*_dev(d))
    torch.cuda.synchronize()
    q, k, v = inputs_f64(d, "bf16")
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(N - 100, N),
                                     np.random.default_rng(N).choice(N, 150)]))
    ref = ol.causal_linear_attention(q, k, v, rows=rows)
    assert_parity(to_f64(out)[:, :, rows], ref[:, :, rows], "bf16", f"causal ring N={N}")


def test_carried_state_matches_one_call(gpu_lib):
    """Two calls with the state carried equal the oracle's whole-sequence causal
    output; the carried state may be updated in place."""
    N, cut, H = 900, 345, 2
    d = gen.make_qkv(_wl(H, N, 95))
    q, k, v = _dev(d)
    S = torch.zeros((1, H, 128, 128), dtype=torch.float32, device="cuda")
    z = torch.zeros((1, H, 128), dtype=torch.float32, device="cuda")
    a = gpu_lib.causal_linear_attn_fwd(q[:, :, :cut].contiguous(), k[:, :, :cut].contiguous(),
                                       v[:, :, :cut].contiguous(), state=(S, z), state_out=(S, z))[0]
    b = gpu_lib.causal_linear_attn_fwd(q[:, :, cut:].contiguous(), k[:, :, cut:].contiguous(),
                                       v[:, :, cut:].contiguous(), state=(S, z), state_out=(S, z))[0]
    torch.cuda.synchronize()
    qf, kf, vf = inputs_f64(d, "bf16")
    ref = ol.causal_linear_attention(qf, kf, vf)
    assert_parity(np.concatenate([to_f64(a), to_f64(b)], axis=2), ref, "bf16", "carried")
    _, rS, rz = ol.linear_attention(qf, kf, vf)
    assert parity(to_f64(S), rS)[1] < 1e-2
    assert parity(to_f64(z), rz)[1] < 1e-5


def test_given_state_against_oracle(gpu_lib):
    """An arbitrary positive carried state (S0, z0) against the oracle's form."""
    N, H = 300, 2
    d = gen.make_qkv(_wl(H, N, 96))
    r = np.random.default_rng(97)
    S0 = r.random((1, H, 128, 128)) * 40.0 - 10.0
    z0 = r.random((1, H, 128)) * 50.0 + 1.0
    S0 = S0.astype(np.float32).astype(np.float64)
    z0 = z0.astype(np.float32).astype(np.float64)
    out = gpu_lib.causal_linear_attn_fwd(*_dev(d), state=(torch.tensor(S0, dtype=torch.float32, device="cuda"),
                                                         torch.tensor(z0, dtype=torch.float32, device="cuda")))
    torch.cuda.synchronize()
    q, k, v = inputs_f64(d, "bf16")
    ref = ol.causal_linear_attention(q, k, v, S0=S0, z0=z0)
    assert_parity(to_f64(out), ref, "bf16", "given state")


def test_first_row_is_its_value_and_constant_values(gpu_lib):
    d = dict(gen.make_qkv(_wl(2, 200, 98)))
    out = gpu_lib.causal_linear_attn_fwd(*_dev(d))
    torch.cuda.synchronize()
    v0 = gen.bf16_bits_to_f64(d["v"])[:, :, 0]
    assert np.abs(to_f64(out)[:, :, 0] - v0).max() <= 2 ** -7 * np.abs(v0).max()
    d["v"] = np.full_like(d["v"], 0x3F80)            # bf16 1.0
    out = gpu_lib.causal_linear_attn_fwd(*_dev(d))
    torch.cuda.synchronize()
    assert np.abs(to_f64(out) - 1.0).max() < 1e-2


def test_strided_layout_and_determinism(gpu_lib):
    """[B, N, H, D] storage viewed as [B, H, N, D]; two runs are bitwise equal."""
    B, N, H = 2, 700, 3
    r = np.random.default_rng(99)
    x = [gen.store(r.standard_normal((B, N, H, 128)).astype(np.float32), "bf16") for _ in range(3)]
    dev = [to_device(t, "bf16").permute(0, 2, 1, 3) for t in x]
    out1 = gpu_lib.causal_linear_attn_fwd(*dev)
    out2 = gpu_lib.causal_linear_attn_fwd(*dev)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    q, k, v = (gen.to_f64(np.ascontiguousarray(t.transpose(0, 2, 1, 3)), "bf16") for t in x)
    rows = np.concatenate([np.arange(0, 50), np.arange(650, 700)])
    ref = ol.causal_linear_attention(q, k, v, rows=rows)
    assert_parity(to_f64(out1)[:, :, rows], ref[:, :, rows], "bf16", "strided")


def test_causal_32k_sampled_rows(gpu_lib):
    """The 32,760-token, 12-head workload: sampled rows of every head, and the
    final state."""
    wl = get_workload("linear_32k")
    d = gen.make_qkv(wl)
    out, S, z = gpu_lib.causal_linear_attn_fwd(*_dev(d), return_state=True)
    torch.cuda.synchronize()
    q, k, v = inputs_f64(d, "bf16")
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 799, 800, 1599, 1600, wl.N - 1],
                                     np.random.default_rng(100).choice(wl.N, 40, replace=False)]))
    ref = ol.causal_linear_attention(q, k, v, rows=rows)
    assert_parity(to_f64(out)[:, :, rows], ref[:, :, rows], "bf16", "causal 32k")
    _, rS, rz = ol.linear_attention(q, k, v)
    assert parity(to_f64(S), rS)[1] < 1e-2
    assert parity(to_f64(z), rz)[1] < 1e-5
