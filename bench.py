#!/usr/bin/env python3
"""Benchmark of the block-sparse spatiotemporal attention path on one MI355X.

Workload (default ``lvsa_32k``): batch 1, 12 heads, head_dim 128, a video
latent of 21 frames x 30x52 patches = 32,760 tokens, blocks of 128 tokens,
bf16 Q/K/V (N(0,1) plus a per-frame AR(1) component, seeded).  One step is
one denoising step's worth of the hot path: build the LVSA block mask for
step s (local window +-3 frames, anchor frames every 8th frame rotated by s,
s = step index mod 4) and run block-sparse attention with it.  Inputs are
resident in HBM before the timed region starts.

Reported (one JSON line): effective TFLOP/s over the timed steps, counting
4 * D * (real query rows x real key columns) of kept blocks only; ms per
attention call; the attention kernel's roofline against the bf16 MFMA peak
(kernel time from HIP events on the launch stream); the HBM traffic measured
by rocprofv3 counters when a profile of the current kernel source exists; the
measured read-only HBM rate (bsa_hbm_read_probe over 2 GiB) and the sustained
vendor GEMM rate as references; under "side", the call times of the HBM-bound
rows on their own workloads (linear attention at 32K and 196K tokens, SVG-EAR
routing at 32K, replayed as a captured graph of its three calls) as algorithmic
GB/s against the HBM peak; and the CPU oracle timed on a bounded sample of the
same workload.

Other workloads (``--workload``): radial_196k (Radial mask, 196,560 tokens);
linear_32k / linear_196k (elu+1 linear attention, HBM-bound: reported as
algorithmic GB/s = (read Q, K, V + write O) / call time against 8 TB/s);
causal_linear_32k (causal elu+1 linear attention: state partials, split
prefix and the causal walk, as algorithmic GB/s like the non-causal one);
mixed_32k (LinVideo mixed attention r = 0.5: the LVSA mask of the step, then
one mixed call; effective TFLOP/s over kept blocks plus the linear branch's
4 N D^2 per head); svg_ear_32k (clustered Q/K, centroid compensation at 15%
density: one step is the fused call; routing = centroids + scores + selection
reported as algorithmic GB/s of reading Q, K, V once; compensated attention as
effective TFLOP/s over exact plus virtual keys); kmeans_32k (the token
clustering in front of it: k-means of queries and keys, 10 Lloyd steps each,
rows into cluster order and one tensor back, as effective TFLOP/s of the
distance products); lvsa_32k_bwd (the attention part of a training step on the
LVSA workload: mask, transposed mask, forward and backward, as effective
TFLOP/s counting 4 D per kept pair for the forward and 10 D for the backward's
five products); lipar_32k (latent inter-frame pruning and restoration as
algorithmic GB/s).
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E (published)
KERNEL_SRC = os.path.join(ROOT, "block_sparse_spatiotemporal_build_amd", "csrc", "attn_fwd.hip")
PROFILES = os.path.join(ROOT, "profiles")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="lvsa_32k",
                    choices=["lvsa_32k", "lvsa_32k_bwd", "radial_196k", "linear_32k", "linear_196k", "causal_linear_32k",
                             "mixed_32k", "svg_ear_32k", "kmeans_32k", "lipar_32k"])
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="wall-clock budget of the CPU oracle sample (0 disables it)")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy"],
                    help="copy: run a plain device copy of known size (HBM counter calibration)")
    ap.add_argument("--no-refs", action="store_true",
                    help="skip the measured references (sustained bf16 GEMM, 1 GiB copy)")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the side legs of the default line (linear 32K / 196K and SVG-EAR routing call times)")
    ap.add_argument("--cold-calls", type=int, default=10,
                    help="attention calls timed after a 512 MiB scratch write each (cold caches)")
    return ap.parse_args()


def source_hash(path=KERNEL_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def kept_flops_from_csr(row_ptr, col_idx, N, block, D, B, H) -> int:
    """4 * D * sum over kept (i, j) of real rows(i) * real cols(j), times B * H."""
    import numpy as np
    nb = len(row_ptr) - 1
    sizes = np.minimum(block, N - np.arange(nb) * block).astype(np.int64)
    pairs = 0
    for i in range(nb):
        cols = col_idx[row_ptr[i]:row_ptr[i + 1]]
        pairs += int(sizes[i]) * int(sizes[cols].sum())
    return 4 * D * pairs * B * H


def read_traffic(workload: str, profile: str = "attn_bf16", src: str = KERNEL_SRC):
    """HBM bytes per launch from a committed counter profile taken with this kernel
    source (None when there is none, or the source changed since)."""
    path = os.path.join(PROFILES, f"{profile}_{workload}.hbm_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != source_hash(src):
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _events_ms(fn, calls, warm):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / calls


def measure_gemm_tflops():
    """Sustained dense bf16 matrix rate of this GPU as the vendor GEMM reaches it:
    torch.matmul of two contiguous 8192 x 8192 bf16 matrices, about 0.5 s of
    back-to-back calls after as long a warm-up (the clock settles under load)."""
    import torch
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    ms = _events_ms(lambda: torch.matmul(a, b, out=c), 600, 600)
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def measure_copy_gbs():
    """Read + write GB/s of a plain 1 GiB device copy (the measured HBM ceiling)."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms = _events_ms(lambda: dst.copy_(src), 10, 3)
    return 2 * n / (ms * 1e-3) / 1e9


def measure_read_gbs():
    """Read-only HBM rate: bsa_hbm_read_probe streaming a 2 GiB buffer (eight
    times the last-level cache) once per call, as GB/s of bytes read."""
    import torch
    import block_sparse_spatiotemporal_build_amd as bsa
    n = 2 << 30
    buf = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    ms = _events_ms(lambda: bsa.hbm_read_probe(buf, sink), 10, 3)
    del buf
    return n / (ms * 1e-3) / 1e9


# Warm-up calls of each side leg.  The side legs start after seconds of host
# work (input generation) with the GPU idle, and the HBM-bound calls reach their
# steady speed only after tens of milliseconds of load: linear attention at
# 196,560 tokens runs about 12 % slower over its first 25 calls than after them.
SIDE_WARM = 100


def side_legs(args, read_gbs):
    """Call times of the HBM-bound rows on their own workloads, reported with the
    default line: linear attention at 32,760 and 196,560 tokens (read Q, K, V +
    write O), and the SVG-EAR routing at 32,760 tokens (query centroids, the
    fused key-centroid / score pass and the selection; read Q, K, V once),
    the latter as a replayed HIP graph of its three calls.  Inputs from the
    same seeded recipes as their own bench lines."""
    import numpy as np
    import torch
    import block_sparse_spatiotemporal_build_amd as bsa
    from synth import gen, get_workload
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def entry(ms, algo_bytes):
        gbs = algo_bytes / (ms * 1e-3) / 1e9
        e = {"ms_per_call": round(ms, 4), "algorithmic_bytes": algo_bytes, "gbs": round(gbs, 1),
             "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        if read_gbs:
            e["frac_of_measured_read"] = round(gbs / read_gbs, 4)
        return e

    out = {}
    for name in ("linear_32k", "linear_196k"):
        wl = get_workload(name)
        d = gen.make_qkv(wl)
        q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
        del d
        o = torch.empty_like(q)
        ws = torch.empty(bsa.linear_attn_workspace(q), dtype=torch.uint8, device=dev)
        ms = _events_ms(lambda: bsa.linear_attn_fwd(q, k, v, out=o, workspace=ws), 20, SIDE_WARM)
        out[name] = entry(ms, 4 * wl.B * wl.H * wl.N * wl.D * 2)
        del q, k, v, o, ws
    wl = get_workload("svg_ear_32k")
    d = gen.make_clustered(wl)
    q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
    qo = torch.from_numpy(d["q_off"]).to(dev)
    ko = torch.from_numpy(d["k_off"]).to(dev)
    del d
    scale = 1.0 / math.sqrt(wl.D)
    qc, _, _ = bsa.cluster_centroids(q, k, v, qo, ko, which="query")
    sc, kc, vc = bsa.route_scores(k, v, qo, ko, qc, scale)

    def routing():
        bsa.cluster_centroids(q, k, v, qo, ko, which="query")
        bsa.route_scores(k, v, qo, ko, qc, scale, k_cent=kc, v_cent=vc)
        bsa.route_select(sc, q, qo, ko, wl.density_ppm)

    # The three Python-level calls take more host time than the ~160 us of GPU
    # work they launch, so the routing leg replays them as one captured HIP graph
    # (the library records no allocation, synchronisation or memset); the eager
    # time is reported beside it.
    ms_eager = _events_ms(routing, 20, SIDE_WARM)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        routing()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        routing()
    torch.cuda.synchronize()
    ms = _events_ms(graph.replay, 20, SIDE_WARM)
    out["routing_svg_ear_32k"] = entry(ms, 3 * wl.B * wl.H * wl.N * wl.D * 2)
    out["routing_svg_ear_32k"]["timing"] = "replay of a captured HIP graph of the three calls"
    out["routing_svg_ear_32k"]["ms_per_call_eager"] = round(ms_eager, 4)
    del graph
    return out


def cpu_baseline(wl, d, params, budget_s: float):
    """The oracle, as it stands, on a bounded sample: whole heads, query blocks in order,
    until the wall-clock budget is spent."""
    import numpy as np
    from oracle import attention as oa
    from oracle import mask as om
    from synth import gen
    threads = _oracle_threads()
    m = om.block_mask(om.spec_from_params(params))
    scale = 1.0 / math.sqrt(wl.D)
    sizes = np.minimum(wl.block, wl.N - np.arange(wl.nb) * wl.block)
    flops, done, heads = 0, 0, 0
    dt = 0.0
    for h in range(wl.H):
        q, k, v = (gen.to_f64(d[n][:, h:h + 1], wl.dtype) for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        for i in range(wl.nb):
            oa.block_sparse_attention(q, k, v, m, wl.block, scale, query_blocks=[i])
            flops += 4 * wl.D * int(sizes[i]) * int(sizes[m[i]].sum())
            done += 1
            if dt + time.perf_counter() - t0 >= budget_s:
                break
        dt += time.perf_counter() - t0
        heads += 1
        if dt >= budget_s:
            break
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s (effective, kept blocks)",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {wl.nb * wl.H} query-block rows (heads 0..{heads - 1} in order), "
                      f"mask step 0: {flops / 1e9:.1f} GFLOP in {dt:.1f} s, float64 numpy"}


def _oracle_threads():
    try:
        import threadpoolctl
        return max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity size
        return len(os.sched_getaffinity(0))


def cpu_baseline_linear(wl, d, budget_s: float):
    """The linear-attention oracle on whole heads in order until the budget is spent,
    as algorithmic GB/s (read Q, K, V + write O of the heads done)."""
    from oracle import linear as ol
    from synth import gen
    heads, dt = 0, 0.0
    for h in range(wl.H):
        q, k, v = (gen.to_f64(d[n][:, h:h + 1], wl.dtype) for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        ol.linear_attention(q, k, v)
        dt += time.perf_counter() - t0
        heads += 1
        if dt >= budget_s:
            break
    nbytes = 4 * heads * wl.N * wl.D * 2
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s (read Q, K, V + write O)",
            "cores": int(_oracle_threads()), "kind": "oracle",
            "sample": f"heads 0..{heads - 1} of {wl.H} in order: {dt:.1f} s, float64 numpy"}


def cpu_baseline_svg(wl, d, budget_s: float):
    """The SVG-EAR oracle (centroids, scores, selection, compensated attention of every
    query cluster) on whole heads in order until the budget is spent; ms per call
    extrapolated to all B * H heads."""
    from oracle import svg_ear as oe
    from synth import gen
    scale = 1.0 / math.sqrt(wl.D)
    heads, dt = 0, 0.0
    for r in range(wl.B * wl.H):
        b, h = divmod(r, wl.H)
        q, k, v = (gen.to_f64(d[n][b, h], wl.dtype) for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        oe.svg_ear_head(q, k, v, d["q_off"][r], d["k_off"][r], scale, wl.density_ppm)
        dt += time.perf_counter() - t0
        heads += 1
        if dt >= budget_s:
            break
    ms = dt / heads * wl.B * wl.H * 1e3
    return {"value": round(ms, 1), "unit": "ms per call (extrapolated from the heads done)",
            "cores": int(_oracle_threads()), "kind": "oracle",
            "sample": f"heads 0..{heads - 1} of {wl.B * wl.H} in order, all five steps: {dt:.1f} s, float64 numpy"}


def copy_mode():
    """Plain device-to-device copy of 1 GiB (counter calibration, and the measured
    HBM ceiling that the bandwidth-bound kernels are also compared with)."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    print(json.dumps({"mode": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "ms_per_copy": round(ms, 4), "gbs_read_plus_write": round(2 * n / ms / 1e6, 1)}))


def bench_linear(args, wl):
    """Linear attention: one step = one bsa_linear_attn_fwd call (state, reduce, apply)."""
    import numpy as np
    import torch

    import block_sparse_spatiotemporal_build_amd as bsa
    from synth import gen

    bsa.load()
    dev = torch.device("cuda:0")
    d = gen.make_qkv(wl)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
    d_host = d if args.cpu_seconds > 0 else None
    del d
    out = torch.empty_like(q)
    ws = torch.empty(bsa.linear_attn_workspace(q), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        bsa.linear_attn_fwd(q, k, v, out=out, workspace=ws)
    torch.cuda.synchronize(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        bsa.linear_attn_fwd(q, k, v, out=out, workspace=ws)
        e1.record()
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    algo_bytes = 4 * wl.B * wl.H * wl.N * wl.D * 2
    gbs = algo_bytes / (call_ms * 1e-3) / 1e9
    copy = None if args.no_refs else measure_copy_gbs()
    src = os.path.join(ROOT, "block_sparse_spatiotemporal_build_amd", "csrc", "linear_attn.hip")
    traffic = read_traffic(wl.name, "linear_attn", src)
    result = {
        "metric": "algorithmic HBM GB/s of elu+1 linear attention",
        "value": round(algo_bytes * args.steps / (t1 - t0) / 1e9, 1),
        "unit": "GB/s (read Q, K, V + write O)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4),
        "ms_per_call": round(call_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D,
                   "algorithmic_bytes": algo_bytes},
        "roofline": {"bound": "hbm", "kernel": "linear_attn_fwd (state + reduce + apply)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
        "measured_copy": None if copy is None else {
            "kernel": "1 GiB device copy, read + write", "gbs": round(copy, 1),
            "frac_of_copy": round(gbs / copy, 4)},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_linear(wl, d_host, args.cpu_seconds)
    return result


def cpu_baseline_causal(wl, d, budget_s: float):
    """The causal oracle (one quadratic form per query row, every head at once) on
    uniformly drawn rows, 64 per call, until the budget is spent; the mean time
    per row, times N, gives the whole call's time and so an algorithmic GB/s."""
    import numpy as np
    from oracle import linear as ol
    from synth import gen
    q, k, v = (gen.to_f64(d[n], wl.dtype) for n in ("q", "k", "v"))
    rows = np.random.default_rng(0).permutation(wl.N)
    done, dt = 0, 0.0
    for i in range(0, wl.N, 64):
        t0 = time.perf_counter()
        ol.causal_linear_attention(q, k, v, rows=rows[i:i + 64].tolist())
        dt += time.perf_counter() - t0
        done += len(rows[i:i + 64])
        if dt >= budget_s:
            break
    est_s = dt / done * wl.N
    nbytes = 4 * wl.B * wl.H * wl.N * wl.D * 2
    return {"value": round(nbytes / est_s / 1e9, 4), "unit": "GB/s (read Q, K, V + write O)",
            "cores": int(_oracle_threads()), "kind": "oracle",
            "sample": f"{done} uniformly drawn query rows of {wl.N} (all {wl.B * wl.H} heads each): "
                      f"{dt:.1f} s, extrapolated by N / rows, float64 numpy"}


def bench_causal(args, wl):
    """Causal linear attention: one step = one bsa_causal_linear_attn_fwd call
    (state partials, split prefix, causal walk)."""
    import numpy as np
    import torch

    import block_sparse_spatiotemporal_build_amd as bsa
    from synth import gen

    bsa.load()
    dev = torch.device("cuda:0")
    d = gen.make_qkv(wl)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
    d_host = d if args.cpu_seconds > 0 else None
    del d
    out = torch.empty_like(q)
    ws = torch.empty(bsa.causal_linear_attn_workspace(q), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        bsa.causal_linear_attn_fwd(q, k, v, out=out, workspace=ws)
    torch.cuda.synchronize(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        bsa.causal_linear_attn_fwd(q, k, v, out=out, workspace=ws)
        e1.record()
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    algo_bytes = 4 * wl.B * wl.H * wl.N * wl.D * 2
    gbs = algo_bytes / (call_ms * 1e-3) / 1e9
    copy = None if args.no_refs else measure_copy_gbs()
    src = os.path.join(ROOT, "block_sparse_spatiotemporal_build_amd", "csrc", "linear_attn.hip")
    traffic = read_traffic(wl.name, "causal_linear", src)
    result = {
        "metric": "algorithmic HBM GB/s of causal elu+1 linear attention",
        "value": round(algo_bytes * args.steps / (t1 - t0) / 1e9, 1),
        "unit": "GB/s (read Q, K, V + write O)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4),
        "ms_per_call": round(call_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D,
                   "algorithmic_bytes": algo_bytes},
        "roofline": {"bound": "hbm", "kernel": "causal_linear_attn_fwd (state + prefix + causal walk)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
        "measured_copy": None if copy is None else {
            "kernel": "1 GiB device copy, read + write", "gbs": round(copy, 1),
            "frac_of_copy": round(gbs / copy, 4)},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_causal(wl, d_host, args.cpu_seconds)
    return result


def cpu_baseline_mixed(wl, d, params, budget_s: float):
    """The oracles of both branches on whole heads in order (the linear branch of a
    head, then its block-sparse branch block row by block row, each blended)
    until the budget is spent, as effective TFLOP/s counted like the GPU line."""
    import numpy as np
    from oracle import attention as oa
    from oracle import linear as ol
    from oracle import mask as om
    from synth import gen
    m = om.block_mask(om.spec_from_params(params))
    scale = 1.0 / math.sqrt(wl.D)
    sizes = np.minimum(wl.block, wl.N - np.arange(wl.nb) * wl.block)
    flops, rows_done, dt, heads = 0, 0, 0.0, 0
    for h in range(wl.H):
        q, k, v = (gen.to_f64(d[n][:, h:h + 1], wl.dtype) for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        lin, _, _ = ol.linear_attention(q, k, v)
        flops += 4 * wl.N * wl.D * wl.D
        for i in range(wl.nb):
            soft, _ = oa.block_sparse_attention(q, k, v, m, wl.block, scale, query_blocks=[i])
            r0, r1 = i * wl.block, min((i + 1) * wl.block, wl.N)
            ol.mixed_attention(soft[:, :, r0:r1], lin[:, :, r0:r1], wl.mix_r)
            flops += 4 * wl.D * int(sizes[i]) * int(sizes[m[i]].sum())
            rows_done += 1
            if dt + time.perf_counter() - t0 >= budget_s:
                break
        dt += time.perf_counter() - t0
        heads += 1
        if dt >= budget_s:
            break
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s (effective, kept blocks + linear branch)",
            "cores": int(_oracle_threads()), "kind": "oracle",
            "sample": f"{rows_done} of {wl.nb * wl.H} query-block rows (heads 0..{heads - 1} in order, "
                      f"each head's linear branch included), mask step 0: {flops / 1e9:.1f} GFLOP in {dt:.1f} s, "
                      "float64 numpy"}


def bench_mixed(args, wl):
    """LinVideo mixed attention: one step = the LVSA mask of the step, then one
    bsa_mixed_attn_fwd call (block-sparse branch into o, linear pass blending)."""
    import numpy as np
    import torch

    import block_sparse_spatiotemporal_build_amd as bsa
    from synth import gen

    bsa.load()
    dev = torch.device("cuda:0")
    d = gen.make_qkv(wl)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
    params = [wl.mask_params(s) for s in wl.anchor_steps]
    nb = wl.nb
    rp = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(nb * nb, dtype=torch.int32, device=dev)
    ro = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty(bsa.linear_attn_workspace(q), dtype=torch.uint8, device=dev)
    lin_flops = 4 * wl.B * wl.H * wl.N * wl.D * wl.D     # S = phi(K)^T V and phi(Q) S
    flops = []
    for p in params:
        bsa.build_block_mask(p, row_ptr=rp, col_idx=ci)
        r = rp.cpu().numpy()
        c = ci[: int(r[-1])].cpu().numpy()
        flops.append(kept_flops_from_csr(r, c, wl.N, wl.block, wl.D, wl.B, wl.H) + lin_flops)

    def step(i, evs=None):
        bsa.build_block_mask(params[i % len(params)], row_ptr=rp, col_idx=ci, row_order=ro)
        if evs is not None:
            evs[0].record()
        bsa.mixed_attn_fwd(q, k, v, wl.mix_r, rp, ci, wl.block, out=out, row_order=ro, workspace=ws)
        if evs is not None:
            evs[1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    call_ms = [e[0].elapsed_time(e[1]) for e in evs]
    step_flops = [flops[i % len(flops)] for i in range(args.steps)]
    achieved = float(np.mean(step_flops)) / (float(np.mean(call_ms)) * 1e-3) / 1e12
    d_host = d if args.cpu_seconds > 0 else None
    result = {
        "metric": "effective TFLOP/s of LinVideo mixed attention (r = 0.5) at 32K video tokens",
        "value": round(sum(step_flops) / (t1 - t0) / 1e12, 3),
        "unit": "TFLOP/s (kept blocks + linear branch; mask build + mixed call per step)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4),
        "ms_per_call": round(float(np.mean(call_ms)), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D, "r": wl.mix_r,
                   "mask": "window +-3 frames, anchor every 8th frame rotated by step s=0..3, rows+cols",
                   "gflop_per_call": [round(f / 1e9, 2) for f in flops]},
        "roofline": {"bound": "mfma", "kernel": "mixed_attn_fwd (block-sparse + linear with blend)",
                     "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None},
    }
    if d_host is not None:
        result["cpu_baseline"] = cpu_baseline_mixed(wl, d_host, params[0], args.cpu_seconds)
    return result


def cpu_baseline_kmeans(wl, d, budget_s: float):
    """The k-means oracle (keys, then queries, of whole heads in order, all Lloyd
    steps) until the budget is spent, as TFLOP/s of the distance products."""
    from oracle import kmeans as ok
    from synth import gen
    flops, dt, done = 0, 0.0, []
    for r in range(wl.B * wl.H):
        b, h = divmod(r, wl.H)
        for name, C in (("k", wl.n_k_clusters), ("q", wl.n_q_clusters)):
            x = gen.to_f64(d[name][b, h], wl.dtype)
            t0 = time.perf_counter()
            lab, _ = ok.lloyd(x, d["centres_" + name][r].astype("float64"), wl.kmeans_iters)
            ok.cluster_order(lab, C)
            dt += time.perf_counter() - t0
            flops += 2 * wl.N * C * wl.D * (wl.kmeans_iters + 1)
            done.append(f"{name}{r}")
            if dt >= budget_s:
                break
        if dt >= budget_s:
            break
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s (distance products)",
            "cores": int(_oracle_threads()), "kind": "oracle",
            "sample": f"k-means of {', '.join(done)} (tensor, head) in order: {dt:.1f} s, float64 numpy"}


def bench_kmeans(args, wl):
    """Token clustering: one step = k-means of Q (Cq) and K (Ck), 10 Lloyd steps
    each, Q, K, V gathered into cluster order and one output-sized tensor
    scattered back to token order."""
    import numpy as np
    import torch

    import block_sparse_spatiotemporal_build_amd as bsa
    from synth import gen

    bsa.load()
    dev = torch.device("cuda:0")
    d = gen.make_gmm_tokens(wl)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
    Cq, Ck, T = wl.n_q_clusters, wl.n_k_clusters, wl.kmeans_iters
    init_q = torch.from_numpy(d["centres_q"]).to(dev)
    init_k = torch.from_numpy(d["centres_k"]).to(dev)
    ws_q = torch.empty(bsa.kmeans_workspace(q, Cq), dtype=torch.uint8, device=dev)
    ws_k = torch.empty(bsa.kmeans_workspace(k, Ck), dtype=torch.uint8, device=dev)
    qp, kp, vp, ob = (torch.empty_like(q) for _ in range(4))

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        _, _, perm_k, _ = bsa.kmeans(k, Ck, T, init_k, workspace=ws_k)
        if evs is not None:
            evs[1].record()
        _, _, perm_q, _ = bsa.kmeans(q, Cq, T, init_q, workspace=ws_q)
        if evs is not None:
            evs[2].record()
        bsa.gather_rows(q, perm_q, out=qp)
        bsa.gather_rows(k, perm_k, out=kp)
        bsa.gather_rows(v, perm_k, out=vp)
        bsa.scatter_rows(qp, perm_q, out=ob)
        if evs is not None:
            evs[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    k_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    q_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    p_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    bh = wl.B * wl.H
    fl_k = 2 * bh * wl.N * Ck * wl.D * (T + 1)
    fl_q = 2 * bh * wl.N * Cq * wl.D * (T + 1)
    achieved = fl_k / (k_ms * 1e-3) / 1e12
    perm_bytes = 4 * 2 * bh * wl.N * wl.D * 2           # three gathers and one scatter, read + write
    d_host = d if args.cpu_seconds > 0 else None
    result = {
        "metric": "effective TFLOP/s of SVG-EAR token clustering (k-means distance products) at 32K tokens",
        "value": round((fl_k + fl_q) * args.steps / (t1 - t0) / 1e12, 3),
        "unit": "TFLOP/s (2 N C D per assignment; k-means of Q and K, 10 steps each, plus permutes, per step)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4),
        "ms_kmeans_keys": round(k_ms, 4), "ms_kmeans_queries": round(q_ms, 4),
        "ms_permute": round(p_ms, 4),
        "permute_gbs": round(perm_bytes / (p_ms * 1e-3) / 1e9, 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D, "Cq": Cq, "Ck": Ck,
                   "lloyd_steps": T},
        "roofline": {"bound": "mfma", "kernel": "bsa_kmeans of the keys (assign + scan + place + update launches)",
                     "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None},
    }
    if d_host is not None:
        result["cpu_baseline"] = cpu_baseline_kmeans(wl, d_host, args.cpu_seconds)
    return result


def cpu_baseline_bwd(wl, d, do, params, budget_s: float):
    """The backward oracle on whole heads in order until the budget is spent, as
    effective TFLOP/s (10 D per kept pair)."""
    import numpy as np
    from oracle import attention_bwd as ob
    from oracle import mask as om
    from synth import gen
    m = om.block_mask(om.spec_from_params(params))
    sizes = np.minimum(wl.block, wl.N - np.arange(wl.nb) * wl.block)
    pairs = int((m * sizes[:, None] * sizes[None, :]).sum())
    heads, dt = 0, 0.0
    for h in range(wl.H):
        q, k, v = (gen.to_f64(d[n][:, h:h + 1], wl.dtype) for n in ("q", "k", "v"))
        g = gen.to_f64(do[:, h:h + 1], wl.dtype)
        t0 = time.perf_counter()
        ob.block_sparse_attention_backward(q, k, v, g, m, wl.block, 1.0 / math.sqrt(wl.D), o_dtype="bf16")
        dt += time.perf_counter() - t0
        heads += 1
        if dt >= budget_s:
            break
    return {"value": round(10 * wl.D * pairs * heads / dt / 1e12, 6),
            "unit": "TFLOP/s (effective, 10 D per kept pair)", "cores": int(_oracle_threads()),
            "kind": "oracle", "sample": f"heads 0..{heads - 1} of {wl.H} in order, mask step 0: {dt:.1f} s, "
                                        "float64 numpy"}


def bench_bwd(args, wl):
    """Attention part of a training step: one step = the LVSA mask of step s, its
    transpose, the forward (output and LSE) and the backward."""
    import numpy as np
    import torch

    import block_sparse_spatiotemporal_build_amd as bsa
    from synth import gen

    bsa.load()
    dev = torch.device("cuda:0")
    d = gen.make_qkv(wl)
    do_bits = gen.store(gen.normal_f32((wl.seed, 9, 0, 0, 9), (wl.B, wl.H, wl.N, wl.D)), wl.dtype)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = up(d["q"]), up(d["k"]), up(d["v"]), up(do_bits)
    params = [wl.mask_params(s) for s in wl.anchor_steps]
    nb = wl.nb
    rp = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(nb * nb, dtype=torch.int32, device=dev)
    ro = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    cp = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    ri = torch.empty(nb * nb, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(bsa.block_sparse_attn_bwd_workspace(q), dtype=torch.uint8, device=dev)
    pairs = []
    for p in params:
        bsa.build_block_mask(p, row_ptr=rp, col_idx=ci)
        r = rp.cpu().numpy()
        c = ci[: int(r[-1])].cpu().numpy()
        pairs.append(kept_flops_from_csr(r, c, wl.N, wl.block, wl.D, wl.B, wl.H) // (4 * wl.D))

    def step(i, evs=None):
        bsa.build_block_mask(params[i % len(params)], row_ptr=rp, col_idx=ci, row_order=ro)
        bsa.transpose_block_mask(rp, ci, col_ptr=cp, row_idx=ri)
        if evs is not None:
            evs[0].record()
        bsa.block_sparse_attn_fwd(q, k, v, rp, ci, wl.block, out=o, lse=lse, row_order=ro)
        if evs is not None:
            evs[1].record()
        bsa.block_sparse_attn_bwd(q, k, v, o, do, lse, rp, ci, wl.block, col_ptr=cp, row_idx=ri,
                                  dq=dq, dk=dk, dv=dv, workspace=ws)
        if evs is not None:
            evs[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    step_pairs = [pairs[i % len(pairs)] for i in range(args.steps)]
    bwd_tf = 10 * wl.D * float(np.mean(step_pairs)) / (bwd_ms * 1e-3) / 1e12
    result = {
        "metric": "effective TFLOP/s of the LVSA attention training step (forward + backward) at 32K tokens",
        "value": round(14 * wl.D * sum(step_pairs) / (t1 - t0) / 1e12, 3),
        "unit": "TFLOP/s (4 D per kept pair forward + 10 D backward; mask, transpose, fwd, bwd per step)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4),
        "ms_forward": round(fwd_ms, 4), "ms_backward": round(bwd_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D, "block": wl.block,
                   "mask": "window +-3 frames, anchor every 8th frame rotated by step s=0..3, rows+cols"},
        "roofline": {"bound": "mfma", "kernel": "block_sparse_attn_bwd (dq and dkdv launches)",
                     "achieved": round(bwd_tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(bwd_tf / BF16_PEAK_TFLOPS, 4), "traffic": None},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_bwd(wl, d, do_bits, params[0], args.cpu_seconds)
    return result


def bench_lipar(args, wl):
    """Latent inter-frame pruning + restoration: one step = bsa_lipar_prune of the
    sequence, then bsa_lipar_restore of the pruned rows back to full length."""
    import numpy as np
    import torch

    import block_sparse_spatiotemporal_build_amd as bsa
    from synth import gen

    bsa.load()
    dev = torch.device("cuda:0")
    xb = gen.make_video(wl)
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).to(dev)
    out = torch.empty_like(x)
    outs = bsa.lipar_prune(x, wl.frames, wl.lipar_tau)
    keep, cpos, kidx, nk, xp = outs

    def step():
        bsa.lipar_prune(x, wl.frames, wl.lipar_tau, outputs=outs)
        bsa.lipar_restore(xp, keep, cpos, wl.frames, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    # the timed steps carry no events (a step is short next to the host cost of
    # recording them); the prune / restore split comes from a second, evented pass
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in evs:
        e[0].record()
        bsa.lipar_prune(x, wl.frames, wl.lipar_tau, outputs=outs)
        e[1].record()
        bsa.lipar_restore(xp, keep, cpos, wl.frames, out)
        e[2].record()
    torch.cuda.synchronize(dev)
    prune_ms = float(np.median([a[0].elapsed_time(a[1]) for a in evs]))
    restore_ms = float(np.median([a[1].elapsed_time(a[2]) for a in evs]))
    n_kept = int(nk.sum().item())
    rows = wl.B * wl.H * wl.N
    row_b = wl.D * 2
    prune_bytes = rows * row_b + n_kept * row_b + rows * (1 + 4) + n_kept * 4
    restore_bytes = n_kept * row_b + rows * row_b + rows * (1 + 4)
    algo = prune_bytes + restore_bytes
    gbs = algo / ((prune_ms + restore_ms) * 1e-3) / 1e9
    copy = None if args.no_refs else measure_copy_gbs()
    result = {
        "metric": "algorithmic HBM GB/s of latent inter-frame pruning + restoration",
        "value": round(algo * args.steps / (t1 - t0) / 1e9, 1),
        "unit": "GB/s (read tokens, write kept rows, read kept rows, write tokens, flags and positions)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4),
        "ms_split": {"prune": round(prune_ms, 4), "restore": round(restore_ms, 4)},
        "kept_fraction": round(n_kept / rows, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D, "frames": wl.frames,
                   "tau": wl.lipar_tau, "algorithmic_bytes": algo},
        "roofline": {"bound": "hbm", "kernel": "lipar prune (flag, count, scan, compact) + restore",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "measured_copy": None if copy is None else {
            "kernel": "1 GiB device copy, read + write", "gbs": round(copy, 1),
            "frac_of_copy": round(gbs / copy, 4)},
    }
    if args.cpu_seconds > 0:
        from oracle import lipar as olp
        t = time.perf_counter()
        done = 0
        while True:
            xf = gen.to_f64(xb[0, 0], "bf16")
            kk, idx, y = olp.prune(xf, wl.frames, wl.lipar_tau)
            olp.restore(y, kk, wl.frames)
            done += 1
            if time.perf_counter() - t >= min(args.cpu_seconds, 5.0):
                break
        dt = time.perf_counter() - t
        result["cpu_baseline"] = {"value": round(done * algo / (wl.B * wl.H) / dt / 1e9, 4),
                                  "unit": result["unit"], "cores": int(_oracle_threads()), "kind": "oracle",
                                  "sample": f"{done} full sequence(s) (prune + restore): {dt:.1f} s, float64 numpy"}
    return result


def bench_svg(args, wl):
    """Centroid compensation: one step = one bsa_centroid_compensate call."""
    import numpy as np
    import torch

    import block_sparse_spatiotemporal_build_amd as bsa
    from synth import gen

    bsa.load()
    dev = torch.device("cuda:0")
    d = gen.make_clustered(wl)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
    qo = torch.from_numpy(d["q_off"]).to(dev)
    ko = torch.from_numpy(d["k_off"]).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    res = bsa.centroid_compensate(q, k, v, qo, ko, wl.density_ppm, out=out, lse=lse)
    rrow, rcol = res[2], res[3]
    scale = 1.0 / math.sqrt(wl.D)

    def fused():
        bsa.centroid_compensate(q, k, v, qo, ko, wl.density_ppm, out=out, lse=lse, rrow=rrow, rcol=rcol)

    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        fused()
        e1.record()
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    # per-step split through the step entry points, which run the fused call's
    # kernels (query centroids; the probe, which also averages the key
    # clusters, and the scores; the selection, whose call rebuilds the score
    # histograms the fused call reuses; the compensated attention)
    qc, _, _ = bsa.cluster_centroids(q, k, v, qo, ko, which="query")
    sc, kc, vc = bsa.route_scores(k, v, qo, ko, qc, scale)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    split = []
    for _ in range(max(3, args.steps // 4)):
        marks[0].record()
        bsa.cluster_centroids(q, k, v, qo, ko, which="query")
        marks[1].record()
        bsa.route_scores(k, v, qo, ko, qc, scale, k_cent=kc, v_cent=vc)
        marks[2].record()
        r2, c2 = bsa.route_select(sc, q, qo, ko, wl.density_ppm)
        marks[3].record()
        bsa.compensated_attn_fwd(q, k, v, qo, ko, r2, c2, kc, vc, scale, out=out, return_lse=False)
        marks[4].record()
        torch.cuda.synchronize(dev)
        split.append([marks[i].elapsed_time(marks[i + 1]) for i in range(4)])
    cent_ms, score_ms, sel_ms, attn_ms = (float(x) for x in np.median(np.array(split), axis=0))

    # effective FLOP of the compensated attention: exact keys of kept clusters + virtual keys
    rr, rc = rrow.cpu().numpy(), rcol.cpu().numpy()
    qon, kon = d["q_off"], d["k_off"]
    pairs = 0
    for r in range(wl.B * wl.H):
        nk = np.diff(kon[r]).astype(np.int64)
        nq = np.diff(qon[r]).astype(np.int64)
        for a in range(wl.n_q_clusters):
            cols = rc[r][rr[r][a]:rr[r][a + 1]]
            exact = int(nk[cols].sum())
            virt = int((nk > 0).sum()) - len(cols)
            pairs += int(nq[a]) * (exact + virt)
    attn_flop = 4 * wl.D * pairs
    route_bytes = 3 * wl.B * wl.H * wl.N * wl.D * 2
    route_ms = cent_ms + score_ms + sel_ms
    achieved = attn_flop / (attn_ms * 1e-3) / 1e12
    route_gbs = route_bytes / (route_ms * 1e-3) / 1e9
    copy = None if args.no_refs else measure_copy_gbs()
    gemm = None if args.no_refs else measure_gemm_tflops()
    src = os.path.join(ROOT, "block_sparse_spatiotemporal_build_amd", "csrc", "svg_ear.hip")
    result = {
        "metric": "ms per centroid-compensated attention call (routing + attention)",
        "value": round(call_ms, 4), "unit": "ms", "higher_is_better": False,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 4),
        "ms_split": {"centroids": round(cent_ms, 4), "route_scores": round(score_ms, 4),
                     "route_select": round(sel_ms, 4), "compensated_attn": round(attn_ms, 4)},
        "routing_gbs": round(route_gbs, 1),
        "routing_frac_of_hbm": round(route_gbs / HBM_PEAK_GBS, 4),
        "routing_frac_of_copy": None if copy is None else round(route_gbs / copy, 4),
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D,
                   "Cq": wl.n_q_clusters, "Ck": wl.n_k_clusters, "density_ppm": wl.density_ppm,
                   "attn_gflop": round(attn_flop / 1e9, 2), "routing_bytes": route_bytes},
        "roofline": {"bound": "mfma", "kernel": "comp_attn_d128_kernel", "achieved": round(achieved, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": read_traffic(wl.name, "comp_attn", src)},
        "measured_copy": None if copy is None else {"kernel": "1 GiB device copy, read + write",
                                                    "gbs": round(copy, 1)},
        "measured_peak": None if gemm is None else {
            "kernel": "sustained bf16 GEMM 8192^3 (torch.matmul)", "tflops": round(gemm, 1),
            "attn_frac_of_measured": round(achieved / gemm, 4)},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_svg(wl, d, args.cpu_seconds)
    return result


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the path has no multi-GPU part; heads would be sharded with no exchange.", file=sys.stderr)
        sys.exit(2)
    if args.mode == "copy":
        copy_mode()
        return

    import numpy as np
    import torch

    import block_sparse_spatiotemporal_build_amd as bsa
    from synth import gen, get_workload

    wl = get_workload(args.workload)
    if wl.op == "causal":
        print(json.dumps(bench_causal(args, wl)), flush=True)
        return
    if wl.op == "mixed":
        print(json.dumps(bench_mixed(args, wl)), flush=True)
        return
    if wl.op == "kmeans":
        print(json.dumps(bench_kmeans(args, wl)), flush=True)
        return
    if wl.op == "bwd":
        print(json.dumps(bench_bwd(args, wl)), flush=True)
        return
    if wl.values == "iid":
        print(json.dumps(bench_linear(args, wl)), flush=True)
        return
    if wl.values == "gmm":
        print(json.dumps(bench_svg(args, wl)), flush=True)
        return
    if wl.values == "video":
        print(json.dumps(bench_lipar(args, wl)), flush=True)
        return
    bsa.load()
    dev = torch.device("cuda:0")
    d = gen.make_qkv(wl)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
    steps_cycle = list(wl.anchor_steps) if wl.mask_kind == 1 else [0]
    params = [wl.mask_params(s) for s in steps_cycle]
    nb = wl.nb
    rp = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(nb * nb, dtype=torch.int32, device=dev)
    ro = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    # effective FLOP of each step's mask (from the device CSR)
    flops = []
    for p in params:
        bsa.build_block_mask(p, row_ptr=rp, col_idx=ci)
        r = rp.cpu().numpy()
        c = ci[: int(r[-1])].cpu().numpy()
        flops.append(kept_flops_from_csr(r, c, wl.N, wl.block, wl.D, wl.B, wl.H))

    def step(i, evs=None):
        p = params[i % len(params)]
        if evs is not None:
            evs[0].record()
        bsa.build_block_mask(p, row_ptr=rp, col_idx=ci, row_order=ro)
        if evs is not None:
            evs[1].record()
        bsa.block_sparse_attn_fwd(q, k, v, rp, ci, wl.block, out=out, lse=lse, row_order=ro)
        if evs is not None:
            evs[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()

    total_s = t1 - t0
    step_flops = [flops[i % len(flops)] for i in range(args.steps)]
    attn_ms = [evs[i][1].elapsed_time(evs[i][2]) for i in range(args.steps)]
    mask_ms = [evs[i][0].elapsed_time(evs[i][1]) for i in range(args.steps)]
    attn_avg_ms = float(np.mean(attn_ms))
    achieved = float(np.mean(step_flops)) / (attn_avg_ms * 1e-3) / 1e12
    traffic = read_traffic(wl.name)

    # cold caches: a 512 MiB scratch write before each timed attention call
    cold_ms = []
    if args.cold_calls > 0:
        scratch = torch.empty(128 << 20, dtype=torch.float32, device=dev)
        for i in range(args.cold_calls):
            p = params[i % len(params)]
            bsa.build_block_mask(p, row_ptr=rp, col_idx=ci, row_order=ro)
            scratch.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bsa.block_sparse_attn_fwd(q, k, v, rp, ci, wl.block, out=out, lse=lse, row_order=ro)
            e1.record()
            torch.cuda.synchronize(dev)
            cold_ms.append(e0.elapsed_time(e1))
        del scratch

    result = {
        "metric": "ms/attn call and effective TFLOP/s at 32K video tokens; % of bf16 MFMA peak",
        "value": round(sum(step_flops) / total_s / 1e12, 3),
        "unit": "TFLOP/s (effective, kept blocks; mask build + attention per step)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_s * 1e3 / args.steps, 4),
        "ms_per_attn_call": round(attn_avg_ms, 4),
        "ms_per_attn_call_median": round(float(np.median(attn_ms)), 4),
        "ms_per_attn_call_p10_p90": [round(float(np.percentile(attn_ms, 10)), 4),
                                     round(float(np.percentile(attn_ms, 90)), 4)],
        "ms_per_attn_call_cold_median": round(float(np.median(cold_ms)), 4) if cold_ms else None,
        "ms_per_mask_build": round(float(np.mean(mask_ms)), 4),
        "pct_of_bf16_mfma_peak": round(100 * achieved / BF16_PEAK_TFLOPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D,
                   "frames": wl.frames, "frame_hw": [wl.frame_h, wl.frame_w], "block": wl.block,
                   "mask": ("window +-3 frames, anchor every 8th frame rotated by step s=0..3, rows+cols"
                            if wl.mask_kind == 1 else f"radial W={wl.radial_w}"),
                   "gflop_per_call": [round(f / 1e9, 2) for f in flops]},
        "roofline": {"bound": "mfma", "kernel": "attn_bf16_d128_kernel",
                     "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": traffic},
    }
    read_gbs = None if args.no_refs else measure_read_gbs()
    if read_gbs is not None:
        result["measured_hbm_read"] = {"kernel": "bsa_hbm_read_probe, 2 GiB read once per call",
                                       "gbs": round(read_gbs, 1), "frac_of_peak": round(read_gbs / HBM_PEAK_GBS, 4)}
    if not args.no_side and wl.name == "lvsa_32k":
        result["side"] = side_legs(args, read_gbs)
    # The GEMM reference (about 1.2 s of full-power matrix work) runs after the
    # other measurements so that the clock state it leaves behind does not
    # carry into them.
    gemm = None if args.no_refs else measure_gemm_tflops()
    if gemm is not None:
        result["measured_peak"] = {"kernel": "sustained bf16 GEMM 8192^3 (torch.matmul)",
                                   "tflops": round(gemm, 1),
                                   "attn_frac_of_measured": round(achieved / gemm, 4)}
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(wl, d, params[0], args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
