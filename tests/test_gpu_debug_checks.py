"""BSA_DEBUG on the device outputs: the mask and route CSRs the kernels write
pass the host checker after every call of the debug mode (and the results are
unchanged by it)."""

import math
import os

import numpy as np
import pytest
import torch

from helpers import to_device
from synth import gen, get_workload

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_env():
    old = os.environ.get("BSA_DEBUG")
    os.environ["BSA_DEBUG"] = "1"
    yield
    if old is None:
        os.environ.pop("BSA_DEBUG", None)
    else:
        os.environ["BSA_DEBUG"] = old


def test_mask_builds_pass_the_debug_check(gpu_lib, debug_env):
    bsa = gpu_lib
    for name in ("lvsa_32k", "radial_196k"):
        wl = get_workload(name)
        steps = wl.anchor_steps if wl.mask_kind == 1 else (0,)
        for s in steps:
            rp, ci = bsa.build_block_mask(wl.mask_params(s), device=torch.device("cuda:0"))
            torch.cuda.synchronize()
            assert int(rp[0]) == 0


def test_routing_passes_the_debug_check(gpu_lib, debug_env):
    bsa = gpu_lib
    wl = get_workload("svg_ear_32k")
    d = gen.make_clustered(wl)
    q, k, v = (to_device(d[n], "bf16") for n in ("q", "k", "v"))
    qo = torch.from_numpy(d["q_off"]).cuda()
    ko = torch.from_numpy(d["k_off"]).cuda()
    out, lse, rrow, rcol = bsa.centroid_compensate(q, k, v, qo, ko, wl.density_ppm)
    torch.cuda.synchronize()
    os.environ.pop("BSA_DEBUG")
    out2, lse2, rrow2, rcol2 = bsa.centroid_compensate(q, k, v, qo, ko, wl.density_ppm)
    torch.cuda.synchronize()
    assert torch.equal(rrow, rrow2)
    # each head's route columns: only the row_ptr[Cq] leading entries are written
    rr, c1, c2 = rrow.cpu().numpy(), rcol.cpu().numpy(), rcol2.cpu().numpy()
    for h in range(rr.shape[0]):
        n = int(rr[h][-1])
        assert np.array_equal(c1[h][:n], c2[h][:n]), h
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
