"""The library's calls under HIP graph capture.

Nothing in the library allocates, frees, synchronises or records a memset, so a
sequence of calls can be captured once and replayed.  A graph of the mask
build, block-sparse attention forward and backward, the SVG-EAR fused call,
k-means with the cluster gather, and linear, causal and mixed linear attention
is replayed several times with eager runs of the same calls in between; every
replay must reproduce the eager outputs bit for bit (the kernels are
deterministic)."""

import numpy as np
import pytest
import torch

from helpers import to_device
from synth import gen, get_workload

pytestmark = pytest.mark.gpu


def test_capture_and_replay(gpu_lib):
    bsa = gpu_lib
    wl = gen.scaled(get_workload("lvsa_32k"), H=2, frames=4, frame_h=10, frame_w=26, seed=90)
    d = gen.make_qkv(wl)
    q, k, v = (to_device(d[n], "bf16") for n in ("q", "k", "v"))
    do = torch.randn_like(q.float()).to(torch.bfloat16)
    p = dict(kind=1, frames=wl.frames, frame_tokens=wl.P, block=128, window=1, anchor_period=2,
             anchor_step=1, anchor_rows=1, radial_w=0)
    nb = bsa.num_blocks(p)
    rp = torch.empty(nb + 1, dtype=torch.int32, device="cuda")
    ci = torch.empty(nb * nb, dtype=torch.int32, device="cuda")
    ro = torch.empty(nb + 1, dtype=torch.int32, device="cuda")
    cp = torch.empty(nb + 1, dtype=torch.int32, device="cuda")
    ri = torch.empty(nb * nb, dtype=torch.int32, device="cuda")
    o, lin, cau, mix = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    bwd_ws = torch.empty(bsa.block_sparse_attn_bwd_workspace(q), dtype=torch.uint8, device="cuda")
    lin_ws = torch.empty(bsa.linear_attn_workspace(q), dtype=torch.uint8, device="cuda")
    cau_ws = torch.empty(bsa.causal_linear_attn_workspace(q), dtype=torch.uint8, device="cuda")
    # SVG-EAR inputs: the token rows grouped by a fixed clustering
    wl2 = gen.scaled(get_workload("svg_ear_32k"), H=2, frames=3, frame_h=20, frame_w=26, n_q_clusters=10,
                     n_k_clusters=40, seed=91)
    g = gen.make_gmm_tokens(wl2)
    gq, gk, gv = (to_device(g[n], "bf16") for n in ("q", "k", "v"))
    init = torch.from_numpy(g["centres_k"]).cuda()
    km_ws = torch.empty(bsa.kmeans_workspace(gk, 40), dtype=torch.uint8, device="cuda")
    cent = torch.empty_like(init)
    labels = torch.empty((2, wl2.N), dtype=torch.int32, device="cuda")
    perm = torch.empty_like(labels)
    off = torch.empty((2, 41), dtype=torch.int32, device="cuda")
    kp = torch.empty_like(gk)
    dc = gen.make_clustered(wl2)
    cq_, ck_, cv_ = (to_device(dc[n], "bf16") for n in ("q", "k", "v"))
    q_off = torch.from_numpy(dc["q_off"]).cuda()
    k_off = torch.from_numpy(dc["k_off"]).cuda()
    svg_out = torch.empty_like(cq_)
    svg_lse = torch.empty(cq_.shape[:3], dtype=torch.float32, device="cuda")

    def run():
        bsa.build_block_mask(p, row_ptr=rp, col_idx=ci, row_order=ro)
        bsa.transpose_block_mask(rp, ci, col_ptr=cp, row_idx=ri)
        bsa.block_sparse_attn_fwd(q, k, v, rp, ci, 128, out=o, lse=lse, row_order=ro)
        bsa.block_sparse_attn_bwd(q, k, v, o, do, lse, rp, ci, 128, col_ptr=cp, row_idx=ri, dq=dq, dk=dk, dv=dv,
                                  workspace=bwd_ws)
        bsa.linear_attn_fwd(q, k, v, out=lin, workspace=lin_ws)
        bsa.causal_linear_attn_fwd(q, k, v, out=cau, workspace=cau_ws)
        bsa.mixed_attn_fwd(q, k, v, 0.5, rp, ci, 128, out=mix, row_order=ro, workspace=lin_ws)
        cent.copy_(init)
        lib = bsa.load()
        bsa._check(lib.bsa_kmeans(bsa._ptr(gk), 0, bsa.ctypes.byref(bsa._shape_of(gk)), 40, 4, bsa._ptr(cent),
                                  bsa._ptr(labels), bsa._ptr(perm), bsa._ptr(off), bsa._ptr(km_ws), km_ws.numel(),
                                  bsa._stream(gk.device)), "bsa_kmeans")
        bsa.gather_rows(gk, perm, out=kp)
        bsa.centroid_compensate(cq_, ck_, cv_, q_off, k_off, wl2.density_ppm, out=svg_out, lse=svg_lse)

    outs = (o, lse, dq, dk, dv, lin, cau, mix, cent, labels, perm, off, kp, svg_out, svg_lse)
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv", "lin", "cau", "mix", "cent", "labels", "perm", "off",
                               "kp", "svg_out", "svg_lse"), outs, ref):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                               b.view(torch.uint8) if b.dtype != torch.int32 else b), f"replay {rep}: {name}"
        run()                      # eager work between replays
        torch.cuda.synchronize()
