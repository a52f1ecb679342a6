"""GPU latent inter-frame pruning / restoration vs the oracle.

Keep flags, positions, kept indices and counts are integers (bit-exact); the
pruned rows and the restored sequence are copies of bf16 rows (bit-exact)."""

import numpy as np
import pytest
import torch

from oracle import lipar as ol
from synth import gen, get_workload

pytestmark = pytest.mark.gpu


def _bits_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _check(bsa, x_bits, frames, tau, x_dev=None):
    """x_bits: uint16 [B, H, N, D]; compares everything against the oracle."""
    B, H, N, D = x_bits.shape
    x = _bits_to_dev(x_bits) if x_dev is None else x_dev
    keep, cpos, kidx, nk, xp = bsa.lipar_prune(x, frames, tau)
    # a processed pruned sequence: every row doubled (exact in bf16)
    y = xp * 2
    out = torch.full((B, H, N, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    bsa.lipar_restore(y, keep, cpos, frames, out)
    torch.cuda.synchronize()
    keep_h, cpos_h, kidx_h, nk_h = keep.cpu().numpy(), cpos.cpu().numpy(), kidx.cpu().numpy(), nk.cpu().numpy()
    xp_h = xp.view(torch.int16).cpu().numpy().view(np.uint16)
    out_h = out.float().cpu().numpy()
    for r in range(B * H):
        b, h = divmod(r, H)
        xf = gen.to_f64(x_bits[b, h], "bf16")
        k_ref, idx_ref, rows_ref = ol.prune(xf, frames, tau)
        assert np.array_equal(keep_h[r].astype(bool), k_ref), r
        assert nk_h[r] == len(idx_ref)
        assert np.array_equal(kidx_h[r][: nk_h[r]], idx_ref)
        assert np.array_equal(cpos_h[r], np.cumsum(k_ref) - k_ref)
        assert np.array_equal(xp_h[r][: nk_h[r]], x_bits[b, h][idx_ref])
        want = ol.restore(2.0 * rows_ref, k_ref, frames)
        assert np.array_equal(out_h[b, h], want), r
    return keep_h, nk_h


@pytest.mark.parametrize("F,P,D,tau", [(5, 37, 64, 0.3), (3, 700, 8, 0.5), (7, 300, 1536, 0.05),
                                       (2, 64, 4096, 0.1), (1, 50, 16, 0.0), (70, 3, 64, 0.3),
                                       (130, 2, 16, 0.5)])
def test_random_and_video_like(gpu_lib, F, P, D, tau):
    r = np.random.default_rng(F * 1000 + P)
    x = np.empty((2, 2, F * P, D), np.float32)
    for b in range(2):
        for h in range(2):
            base = r.standard_normal((P, D)).astype(np.float32)
            frames = [base]
            for f in range(1, F):
                moving = r.random(P) < 0.3
                step = np.where(moving[:, None], 1.0, 0.01).astype(np.float32)
                frames.append(frames[-1] + step * r.standard_normal((P, D)).astype(np.float32))
            x[b, h] = np.concatenate(frames)
    keep, nk = _check(gpu_lib, gen.store(x, "bf16"), F, tau)
    if F > 1:
        assert 0 < nk.min() and nk.max() < F * P   # both outcomes occur


@pytest.mark.parametrize("tau,expect", [(-1.0, "all"), (float("inf"), "first")])
def test_threshold_extremes(gpu_lib, tau, expect):
    F, P, D = 4, 300, 32
    x = gen.store(np.random.default_rng(5).standard_normal((1, 2, F * P, D)).astype(np.float32), "bf16")
    keep, nk = _check(gpu_lib, x, F, tau)
    assert (nk == F * P).all() if expect == "all" else (nk == P).all()


def test_strided_layout(gpu_lib):
    """[B, N, H, D] storage seen as [B, H, N, D] through strides."""
    F, P, D, B, H = 3, 500, 64, 1, 3
    r = np.random.default_rng(6)
    base = r.standard_normal((B, P, H, D)).astype(np.float32)
    fr = [base + (0.5 if f % 2 else 0.001) * r.standard_normal(base.shape).astype(np.float32) for f in range(F)]
    xbnhd = gen.store(np.concatenate(fr, axis=1), "bf16")          # [B, N, H, D]
    dev = _bits_to_dev(xbnhd).permute(0, 2, 1, 3)                   # [B, H, N, D] view
    _check(gpu_lib, np.ascontiguousarray(xbnhd.transpose(0, 2, 1, 3)), F, 0.1, x_dev=dev)


def test_lipar_32k_full(gpu_lib):
    wl = get_workload("lipar_32k")
    x = gen.make_video(wl)
    keep, nk = _check(gpu_lib, x, wl.frames, wl.lipar_tau)
    assert 0.1 < nk[0] / wl.N < 0.4


def test_preallocated_outputs_reused(gpu_lib):
    """Outputs passed back in are overwritten completely: a second call on other
    data into the same buffers equals a call with fresh buffers."""
    F, P, D = 6, 200, 64
    r = np.random.default_rng(9)
    xs = [_bits_to_dev(gen.store(r.standard_normal((1, 2, F * P, D)).astype(np.float32) * s, "bf16"))
          for s in (1.0, 0.05)]
    outs = gpu_lib.lipar_prune(xs[0], F, 0.3)
    gpu_lib.lipar_prune(xs[1], F, 0.3, outputs=outs)
    fresh = gpu_lib.lipar_prune(xs[1], F, 0.3)
    torch.cuda.synchronize()
    nk = fresh[3].cpu().numpy()
    for i in (0, 1, 3):  # keep, cpos, n_kept: every entry
        assert torch.equal(outs[i], fresh[i])
    for bh in range(2):  # kept_idx and the pruned rows: the first n_kept entries are defined
        assert 0 < nk[bh] < F * P
        assert torch.equal(outs[2][bh, : nk[bh]], fresh[2][bh, : nk[bh]])
        assert torch.equal(outs[4][bh, : nk[bh]], fresh[4][bh, : nk[bh]])
    with pytest.raises(gpu_lib.BsaError):
        gpu_lib.lipar_prune(xs[1], F, 0.3, outputs=outs[:4] + (outs[4][:, :-1],))


def test_threshold_fixtures(gpu_lib):
    """The hand-derived cases at the threshold (a sum exactly at tau * D with far
    apart exponents, and a sum between the float and double products of tau
    and D): frame 1 is not kept, as the oracle's pins fix, and every output
    equals the oracle's."""
    from test_oracle_lipar import threshold_fixtures
    for name, x, tau, kept in threshold_fixtures():
        bits = gen.store(x.reshape(1, 1, 2, 8).astype(np.float32), "bf16")
        keep, _ = _check(gpu_lib, bits, 2, tau)
        assert keep[0].tolist() == [1, int(kept)], name
