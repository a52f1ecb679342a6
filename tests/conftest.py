import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_mask_fixture(name):
    """Read a hand-derived block-mask fixture: returns (params dict, bool matrix)."""
    import numpy as np
    params, rows = None, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("params"):
                params = {k: int(v) for k, v in (t.split("=") for t in line.split()[1:])}
            else:
                rows.append([c == "1" for c in line])
    return params, np.array(rows, dtype=bool)


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; skips when no GPU is present."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_spatiotemporal_build_amd as bsa
    bsa.load()
    return bsa
