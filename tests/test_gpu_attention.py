"""GPU block-sparse attention vs the oracle (element by element), plus invariants."""

import math

import numpy as np
import pytest
import torch

from helpers import assert_parity, inputs_f64, to_device, to_f64
from oracle import attention as oa
from oracle import mask as om
from synth import gen, get_workload

pytestmark = pytest.mark.gpu


def _run(bsa, d, wl, params, scale=None, order=True):
    """Mask + attention as the benchmark launches them (with the mask builder's row schedule)."""
    q, k, v = (to_device(d[n], wl.dtype) for n in ("q", "k", "v"))
    rp, ci, ro = bsa.build_block_mask(params, with_order=True)
    out, lse = bsa.block_sparse_attn_fwd(q, k, v, rp, ci, params["block"], scale,
                                         row_order=ro if order else None)
    torch.cuda.synchronize()
    return out, lse


def _oracle(d, wl, params, scale=None, query_blocks=None):
    q, k, v = inputs_f64(d, wl.dtype)
    m = om.block_mask(om.spec_from_params(params))
    scale = 1.0 / math.sqrt(wl.D) if scale is None else scale
    return oa.block_sparse_attention(q, k, v, m, params["block"], scale, query_blocks)


def _rows(blocks, block, N):
    return np.concatenate([np.arange(i * block, min((i + 1) * block, N)) for i in blocks])


# ---------------------------------------------------------------------------
# fp32
# ---------------------------------------------------------------------------

def test_tiny_fp32_full(gpu_lib):
    wl = get_workload("tiny_fp32")
    d = gen.make_qkv(wl)
    p = wl.mask_params(0)
    out, lse = _run(gpu_lib, d, wl, p)
    ref, rlse = _oracle(d, wl, p)
    assert_parity(to_f64(out), ref, "f32", "tiny fp32 out")
    assert_parity(to_f64(lse), rlse, "f32", "tiny fp32 lse")


@pytest.mark.parametrize("D,block", [(32, 16), (64, 64), (128, 128), (128, 32)])
def test_fp32_ragged_radial(gpu_lib, D, block):
    wl = gen.scaled(get_workload("tiny_fp32"), D=D, frames=5, frame_h=5, frame_w=9, H=3, seed=11)
    d = gen.make_qkv(wl)
    p = dict(kind=2, frames=5, frame_tokens=45, block=block, window=0, anchor_period=0,
             anchor_step=0, anchor_rows=0, radial_w=10)
    out, lse = _run(gpu_lib, d, wl, p)
    ref, rlse = _oracle(d, wl, p)
    assert_parity(to_f64(out), ref, "f32", f"fp32 D={D} block={block}")
    assert_parity(to_f64(lse), rlse, "f32", "lse")


# ---------------------------------------------------------------------------
# bf16, reduced sizes (whole output compared)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("D,block,kind", [(128, 128, 1), (128, 128, 2), (64, 64, 1), (64, 128, 2),
                                           (128, 64, 0)])
def test_bf16_reduced_full_compare(gpu_lib, D, block, kind):
    # 6 frames of 10x20 = 1200 tokens: several tiles per row and a ragged last block
    wl = gen.scaled(get_workload("lvsa_32k"), H=2, D=D, frames=6, frame_h=10, frame_w=20, seed=21)
    d = gen.make_qkv(wl)
    p = dict(kind=kind, frames=6, frame_tokens=200, block=block, window=1, anchor_period=4,
             anchor_step=1, anchor_rows=1, radial_w=60)
    out, lse = _run(gpu_lib, d, wl, p)
    ref, rlse = _oracle(d, wl, p)
    assert_parity(to_f64(out), ref, "bf16", f"bf16 D={D} block={block} kind={kind}")
    assert np.abs(to_f64(lse) - rlse).max() < 1e-3


@pytest.mark.parametrize("D,block", [(128, 128), (64, 64), (64, 128)])
def test_row_order_only_schedules(gpu_lib, D, block):
    """The row schedule changes which workgroup runs a row, never the result: the
    builder's schedule, none, all rows "long", and a random permutation with a
    random long count all give the same bits (outputs start as NaN, so a row
    skipped or written twice by a wrong mapping would show)."""
    wl = gen.scaled(get_workload("lvsa_32k"), H=3, D=D, frames=9, frame_h=10, frame_w=20, seed=23)
    d = gen.make_qkv(wl)
    p = dict(kind=1, frames=9, frame_tokens=200, block=block, window=1, anchor_period=4,
             anchor_step=2, anchor_rows=1, radial_w=0)
    q, k, v = (to_device(d[n], wl.dtype) for n in ("q", "k", "v"))
    rp, ci, ro = gpu_lib.build_block_mask(p, with_order=True)
    nb = rp.numel() - 1
    assert 0 < int(ro[-1]) < nb
    lens = np.diff(rp.cpu().numpy())
    full = np.concatenate([np.argsort(-lens, kind="stable"), [nb]]).astype(np.int32)
    r = np.random.default_rng(5)
    rand = np.concatenate([r.permutation(nb), [r.integers(0, nb + 1)]]).astype(np.int32)
    results = []
    for sched in (ro, None, torch.from_numpy(full).cuda(), torch.from_numpy(rand).cuda()):
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), device=q.device)
        gpu_lib.block_sparse_attn_fwd(q, k, v, rp, ci, block, out=out, lse=lse, row_order=sched)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any() and not torch.isnan(lse).any()
        results.append((out.view(torch.int16).clone(), lse.clone()))
    for o2, l2 in results[1:]:
        assert torch.equal(results[0][0], o2) and torch.equal(results[0][1], l2)


def test_head_major_mapping_covers_every_row(gpu_lib):
    """Past 8 heads of K and V above the 256 MiB last-level cache (here N = 70000,
    D = 128) the launcher deals the rows of one head over the XCDs in launch
    order.  Every row must still be written exactly once with the same bits under
    any row schedule, and sampled rows must match the oracle."""
    wl = gen.scaled(get_workload("lvsa_32k"), H=2, D=128, frames=70, frame_h=25, frame_w=40, seed=41)
    assert 8 * 2 * wl.N * wl.D * 2 > 256 << 20
    d = gen.make_qkv(wl)
    p = dict(kind=1, frames=70, frame_tokens=1000, block=128, window=1, anchor_period=16,
             anchor_step=3, anchor_rows=1, radial_w=0)
    q, k, v = (to_device(d[n], wl.dtype) for n in ("q", "k", "v"))
    rp, ci, ro = gpu_lib.build_block_mask(p, with_order=True)
    nb = rp.numel() - 1
    r = np.random.default_rng(9)
    rand = np.concatenate([r.permutation(nb), [r.integers(0, nb + 1)]]).astype(np.int32)
    results = []
    for sched in (ro, None, torch.from_numpy(rand).cuda()):
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), device=q.device)
        gpu_lib.block_sparse_attn_fwd(q, k, v, rp, ci, 128, out=out, lse=lse, row_order=sched)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any() and not torch.isnan(lse).any()
        results.append((out.view(torch.int16).clone(), lse.clone()))
    for o2, l2 in results[1:]:
        assert torch.equal(results[0][0], o2) and torch.equal(results[0][1], l2)
    blocks = [0, nb // 2, nb - 1]
    ref, _ = _oracle(d, wl, p, query_blocks=blocks)
    rows = _rows(blocks, 128, wl.N)
    got = results[0][0].view(torch.bfloat16).float().cpu().numpy()
    assert_parity(got[:, :, rows], ref[:, :, rows], "bf16", "head-major mapping")


def test_bf16_tiny_sequence_shorter_than_a_block(gpu_lib):
    wl = gen.scaled(get_workload("lvsa_32k"), H=1, frames=1, frame_h=3, frame_w=7, seed=22)
    d = gen.make_qkv(wl)
    p = dict(kind=0, frames=1, frame_tokens=21, block=128, window=0, anchor_period=0,
             anchor_step=0, anchor_rows=0, radial_w=0)
    out, _ = _run(gpu_lib, d, wl, p)
    ref, _ = _oracle(d, wl, p)
    assert_parity(to_f64(out), ref, "bf16", "N=21")


# ---------------------------------------------------------------------------
# bf16 invariants
# ---------------------------------------------------------------------------

def _lvsa_small(seed=31):
    wl = gen.scaled(get_workload("lvsa_32k"), H=2, frames=8, frame_h=10, frame_w=16, seed=seed)
    p = dict(kind=1, frames=8, frame_tokens=160, block=128, window=1, anchor_period=5,
             anchor_step=0, anchor_rows=0, radial_w=0)
    return wl, gen.make_qkv(wl), p


def test_constant_values_give_exact_ones(gpu_lib):
    wl, d, p = _lvsa_small()
    d = dict(d)
    d["v"] = np.full_like(d["v"], 0x3F80)        # bf16 1.0
    out, _ = _run(gpu_lib, d, wl, p)
    assert (to_f64(out) == 1.0).all()


def test_masked_out_blocks_are_never_read(gpu_lib):
    wl, d, p = _lvsa_small()
    rp, ci = gpu_lib.build_block_mask(p)
    rpc, cic = rp.cpu().numpy(), ci.cpu().numpy()
    row = 0
    kept = set(cic[rpc[row]:rpc[row + 1]].tolist())
    skipped = [j for j in range(len(rpc) - 1) if j not in kept]
    assert skipped
    out1, lse1 = _run(gpu_lib, d, wl, p)
    d2 = dict(d)
    for n in ("k", "v"):
        arr = d[n].copy()
        for j in skipped:
            arr[:, :, j * 128:(j + 1) * 128] = 0x7FC0      # NaN in every skipped block
        d2[n] = arr
    out2, lse2 = _run(gpu_lib, d2, wl, p)
    a = out1[:, :, :128].cpu()
    b = out2[:, :, :128].cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(lse1[:, :, :128].cpu(), lse2[:, :, :128].cpu())


def test_deterministic(gpu_lib):
    wl, d, p = _lvsa_small(seed=32)
    a, la = _run(gpu_lib, d, wl, p)
    b, lb = _run(gpu_lib, d, wl, p)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


def test_empty_row_gives_zero_and_neg_inf(gpu_lib):
    wl = gen.scaled(get_workload("lvsa_32k"), H=1, frames=2, frame_h=8, frame_w=16, seed=33)
    d = gen.make_qkv(wl)
    q, k, v = (to_device(d[n], "bf16") for n in ("q", "k", "v"))
    rp = torch.tensor([0, 0, 2], dtype=torch.int32, device="cuda")   # row 0 empty
    ci = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    out, lse = gpu_lib.block_sparse_attn_fwd(q, k, v, rp, ci, 128)
    torch.cuda.synchronize()
    assert (out[:, :, :128].float() == 0).all()
    assert torch.isneginf(lse[:, :, :128]).all()
    ref, _ = oa.block_sparse_attention(*inputs_f64(d, "bf16"), np.array([[0, 0], [1, 1]], bool),
                                       128, 1 / math.sqrt(128))
    assert_parity(to_f64(out)[:, :, 128:], ref[:, :, 128:], "bf16", "row 1")


def test_one_dominant_key(gpu_lib):
    wl, d, p = _lvsa_small(seed=34)
    q = gen.bf16_bits_to_f32(d["q"])
    k = gen.bf16_bits_to_f32(d["k"]).copy()
    k[0, 0, 5] = 40.0 * q[0, 0, 3] / np.linalg.norm(q[0, 0, 3])
    d = dict(d, k=gen.f32_to_bf16_bits(k))
    out, _ = _run(gpu_lib, d, wl, p)
    v = gen.bf16_bits_to_f64(d["v"])
    assert np.abs(to_f64(out)[0, 0, 3] - v[0, 0, 5]).max() < 2e-2


# ---------------------------------------------------------------------------
# bf16 at full workload sizes (sampled rows compared; same launch as the benchmark)
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def lvsa_full():
    wl = get_workload("lvsa_32k")
    return wl, gen.make_qkv(wl)


@pytest.mark.parametrize("step", [0, 1, 2, 3])
def test_lvsa_32k_sampled(gpu_lib, lvsa_full, step):
    wl, d = lvsa_full
    p = wl.mask_params(step)
    out, lse = _run(gpu_lib, d, wl, p)
    out = out[:, [0, 7, 11]].float().cpu().numpy()
    lse = lse[:, [0, 7, 11]].cpu().numpy()
    sub = {n: d[n][:, [0, 7, 11]] for n in ("q", "k", "v")}
    # first, second, an anchor-frame block, a middle block, the last two (ragged) blocks
    anchor_blk = (step * wl.P) // wl.block
    blocks = sorted({0, 1, anchor_blk, 100, wl.nb - 2, wl.nb - 1})
    ref, rlse = _oracle(sub, wl, p, query_blocks=blocks)
    rows = _rows(blocks, wl.block, wl.N)
    assert_parity(out[:, :, rows], ref[:, :, rows], "bf16", f"lvsa step {step}")
    assert np.abs(lse[:, :, rows] - rlse[:, :, rows]).max() < 1e-3


def test_radial_196k_sampled(gpu_lib):
    wl = get_workload("radial_196k")
    d = gen.make_qkv(wl)
    p = wl.mask_params(0)
    out, lse = _run(gpu_lib, d, wl, p)
    out = out.float().cpu().numpy()
    # every head; query blocks at both ends, at frame boundaries and inside the
    # sequence (the Radial band differs with the frame distance)
    blocks = [0, 1, 12, 130, 400, 766, 767, 1000, 1100, 1300, wl.nb - 2, wl.nb - 1]
    ref, _ = _oracle(d, wl, p, query_blocks=blocks)
    rows = _rows(blocks, wl.block, wl.N)
    assert_parity(out[:, :, rows], ref[:, :, rows], "bf16", "radial 196k")
