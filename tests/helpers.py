"""Shared test helpers: moving stored inputs to the device and parity metrics."""

import numpy as np
import torch

from synth import gen

# Parity bars: bf16 outputs max-abs 2e-2 and relative L2 1e-2; fp32 outputs 1e-5 for both.
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-5, 1e-5)}


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Stored tensor (uint16 bf16 bits or float32) -> torch device tensor of that dtype."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def parity(got: np.ndarray, ref: np.ndarray):
    """(max-abs error, relative L2 error) over all elements."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = got - ref
    return float(np.abs(err).max()), float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))


def assert_parity(got, ref, dtype: str, what: str = ""):
    ma, rl = parity(got, ref)
    tol_abs, tol_rel = TOL[dtype]
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert ma <= tol_abs and rl <= tol_rel, f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e} (tol {tol_abs}, {tol_rel})"
    return ma, rl


def inputs_f64(d: dict, dtype: str):
    return [gen.to_f64(d[n], dtype) for n in ("q", "k", "v")]
