"""The no-allocation linear attention entry point (bsa_linear_attn_fwd_noalloc)
against the workspace entry point (bsa_linear_attn_fwd), both called through the
C ABI on the same inputs.

The two share kernels and launch plan, so the outputs, S and z must agree to
the bf16 parity bar (max-abs 2e-2, relative L2 1e-2; S and z relative L2 1e-5)
and are in fact bitwise equal.  Several calls in a row, each smaller than the
one before, check that what an earlier call left in the shared scratch does
not leak into a later one."""

import ctypes

import numpy as np
import pytest
import torch

from helpers import assert_parity, parity, to_device, to_f64
from synth import gen, get_workload

pytestmark = pytest.mark.gpu


def _inputs(H, N, D, seed):
    wl = gen.scaled(get_workload("linear_32k"), H=H, D=D, frames=1, frame_h=1, frame_w=N, seed=seed)
    d = gen.make_qkv(wl)
    return [to_device(d[n], "bf16") for n in ("q", "k", "v")]


def _with_workspace(bsa, q, k, v):
    lib = bsa.load()
    shape = bsa._shape_of(q)
    B, H, N, D = q.shape
    out = torch.full_like(q, float("nan"))
    S = torch.full((B, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    z = torch.full((B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(int(lib.bsa_linear_attn_workspace(ctypes.byref(shape))), dtype=torch.uint8, device="cuda")
    st = lib.bsa_linear_attn_fwd(bsa._ptr(q), bsa._ptr(k), bsa._ptr(v), bsa._ptr(out), 0, ctypes.byref(shape),
                                 bsa._ptr(S), bsa._ptr(z), bsa._ptr(ws), ws.numel(), bsa._stream(q.device))
    assert st == 0, lib.bsa_last_error()
    return out, S, z


def _no_alloc(bsa, q, k, v):
    lib = bsa.load()
    shape = bsa._shape_of(q)
    B, H, N, D = q.shape
    out = torch.full_like(q, float("nan"))
    S = torch.full((B, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    z = torch.full((B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.bsa_linear_attn_fwd_noalloc(bsa._ptr(q), bsa._ptr(k), bsa._ptr(v), bsa._ptr(out), 0,
                                         ctypes.byref(shape), bsa._ptr(S), bsa._ptr(z), bsa._stream(q.device))
    assert st == 0, lib.bsa_last_error()
    return out, S, z


def test_no_alloc_matches_workspace_call_on_shrinking_calls(gpu_lib):
    # 12 heads of 32,760 tokens (the benchmark shape, 33 MiB of scratch), then
    # smaller and smaller shapes, then a head_dim-64 shape (the general kernels)
    cases = [(12, 32760, 128, 71), (3, 1000, 128, 72), (2, 257, 128, 73), (2, 130, 64, 74)]
    for H, N, D, seed in cases:
        q, k, v = _inputs(H, N, D, seed)
        ref = _with_workspace(gpu_lib, q, k, v)
        got = _no_alloc(gpu_lib, q, k, v)
        torch.cuda.synchronize()
        what = f"H={H} N={N} D={D}"
        assert_parity(to_f64(got[0]), to_f64(ref[0]), "bf16", what)
        for g, r in zip(got[1:], ref[1:]):
            assert np.isfinite(to_f64(g)).all(), what
            assert parity(to_f64(g), to_f64(r))[1] <= 1e-5, what
        for g, r in zip(got, ref):
            assert torch.equal(g, r), what          # same kernels and plan: bitwise equal


def test_no_alloc_repeated_call_is_stable(gpu_lib):
    """The same call twice on the shared scratch gives the same bits."""
    q, k, v = _inputs(4, 2000, 128, 75)
    a = _no_alloc(gpu_lib, q, k, v)
    b = _no_alloc(gpu_lib, q, k, v)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_no_alloc_rejects_a_shape_beyond_its_scratch(gpu_lib):
    lib = gpu_lib.load()
    q = torch.empty((1, 600, 1000, 128), dtype=torch.bfloat16, device="cuda")
    shape = gpu_lib._shape_of(q)
    need = int(lib.bsa_linear_attn_workspace(ctypes.byref(shape)))
    assert need > int(lib.bsa_linear_attn_noalloc_max_scratch())
    st = lib.bsa_linear_attn_fwd_noalloc(gpu_lib._ptr(q), gpu_lib._ptr(q), gpu_lib._ptr(q), gpu_lib._ptr(q), 0,
                                         ctypes.byref(shape), None, None, gpu_lib._stream(q.device))
    assert st == 2 and b"scratch" in lib.bsa_last_error()
