"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments
on the host before touching the device (CPU only: no kernel is launched)."""

import ctypes
import os
import re

import pytest

import block_sparse_spatiotemporal_build_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(bsa_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bsa.LIB_PATH):
        pytest.fail("libbsa.so is not built (run __graft_entry__.build())")
    return bsa.load()


def test_every_declared_symbol_is_exported(lib):
    declared = _declared()
    assert len(declared) >= 5
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(bsa.exported_names())


def _desc(**kw):
    p = dict(kind=1, frames=4, frame_tokens=64, block=64, window=1, anchor_period=8,
             anchor_step=0, anchor_rows=1, radial_w=0)
    p.update(kw)
    return bsa.mask_desc(p)


def test_num_blocks(lib):
    assert lib.bsa_mask_num_blocks(ctypes.byref(_desc())) == 4
    assert lib.bsa_mask_num_blocks(ctypes.byref(_desc(frames=21, frame_tokens=1560, block=128))) == 256
    assert lib.bsa_mask_num_blocks(ctypes.byref(_desc(block=0))) == -1
    assert lib.bsa_mask_num_blocks(None) == -1


@pytest.mark.parametrize("bad", [dict(kind=7), dict(frames=0), dict(block=0), dict(block=5000),
                                 dict(window=-1), dict(anchor_period=-2), dict(radial_w=-1),
                                 dict(frames=100000, frame_tokens=100000)])
def test_mask_rejects_bad_descriptions(lib, bad):
    st = lib.bsa_build_block_mask(ctypes.byref(_desc(**bad)), ctypes.c_void_p(16), ctypes.c_void_p(16),
                                  1 << 40, None, None)
    assert st == 1, lib.bsa_last_error()
    assert lib.bsa_last_error().decode()


def test_mask_rejects_small_capacity_and_null(lib):
    d = _desc()
    assert lib.bsa_build_block_mask(ctypes.byref(d), ctypes.c_void_p(16), ctypes.c_void_p(16), 15, None, None) == 3
    assert b"col_capacity" in lib.bsa_last_error()
    assert lib.bsa_build_block_mask(ctypes.byref(d), None, ctypes.c_void_p(16), 16, None, None) == 1


def _shape(B=1, H=2, N=256, D=64, sn=None):
    sn = D if sn is None else sn
    return bsa.Shape(B, H, N, D, H * N * sn, N * sn, sn)


def _attn(lib, dtype=0, shape=None, block=64, scale=0.125, ptr=4096, rp=4096):
    shape = shape or _shape()
    p = ctypes.c_void_p(ptr)
    return lib.bsa_block_sparse_attn_fwd(p, p, p, p, None, dtype, ctypes.byref(shape),
                                         ctypes.c_void_p(rp), ctypes.c_void_p(rp), None, block,
                                         ctypes.c_float(scale), None)


def test_attention_argument_checks(lib):
    assert _attn(lib, dtype=5) == 1
    assert _attn(lib, shape=_shape(D=48)) == 2                  # bf16 needs D in {64, 128}
    assert _attn(lib, block=32) == 2                            # bf16 needs block in {64, 128}
    assert _attn(lib, dtype=1, block=48) == 2
    assert _attn(lib, shape=_shape(N=0)) == 1
    assert _attn(lib, shape=_shape(D=64, sn=60)) == 1           # stride_n < D
    assert _attn(lib, shape=_shape(D=64, sn=68)) == 1           # 136-byte rows: not 16-byte multiple
    assert _attn(lib, ptr=4098) == 1                            # misaligned tensor
    assert _attn(lib, ptr=0) == 1
    assert _attn(lib, rp=0) == 1
    assert _attn(lib, scale=0.0) == 1
    assert _attn(lib, scale=-0.125) == 1                        # a negative scale is rejected
    assert _attn(lib, dtype=1, scale=-0.125) == 1
    assert _attn(lib, scale=float("inf")) == 1
    assert _attn(lib, scale=float("nan")) == 1
    assert b"bsa_block_sparse_attn_fwd" in lib.bsa_last_error()


def test_status_strings(lib):
    for s in range(6):
        assert lib.bsa_status_string(s)
    assert lib.bsa_status_string(99) == b"unknown status"


def test_workspace_queries_do_not_crash_and_are_aligned(lib):
    """The host-side plans behind the workspace queries (a stale second copy of a
    plan struct once made these overrun the caller's stack)."""
    for N in (1, 7, 1000, 32760, 196560):
        for H in (1, 2, 12):
            sh = _shape(B=1, H=H, N=N, D=128)
            lw = lib.bsa_linear_attn_workspace(ctypes.byref(sh))
            assert lw > 0 and lw % 256 == 0
            assert lw >= H * 128 * 128 * 2 + H * 128 * 4      # S^T (bf16) and z at least
            for Cq, Ck in ((8, 20), (100, 500), (150, 40)):
                rw = lib.bsa_route_scores_workspace(ctypes.byref(sh), Cq, Ck)
                assert rw > 0 and rw % 256 == 0
                assert rw >= 2 * H * Cq * Ck * 4                # e and m of every block at least
                fw = lib.bsa_centroid_compensate_workspace(ctypes.byref(sh), Cq, Ck)
                assert fw >= rw + H * Cq * Ck * 4               # plus the scores


def test_each_struct_is_defined_once_in_the_native_sources():
    """Host plan structs cross translation units by value: one definition only."""
    csrc = os.path.join(ROOT, "block_sparse_spatiotemporal_build_amd", "csrc")
    seen = {}
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            for name in re.findall(r"^\s*struct\s+(\w+)\s*\{", open(os.path.join(csrc, f)).read(), flags=re.M):
                assert name not in seen, f"struct {name} defined in {seen[name]} and {f}"
                seen[name] = f


def _lipar(lib, shape, frames=4, tau=0.1, ptr=4096):
    p = ctypes.c_void_p(ptr)
    return lib.bsa_lipar_prune(p, 0, ctypes.byref(shape), frames, ctypes.c_float(tau), p, p, p, p, p, None)


def test_lipar_argument_checks(lib):
    ok = _shape(B=1, H=2, N=256, D=64)
    assert _lipar(lib, _shape(D=60)) == 1                        # 120-byte rows: not 16-byte multiple
    assert _lipar(lib, _shape(D=68, sn=72)) == 2                 # D not a multiple of 8
    assert _lipar(lib, _shape(D=4104)) == 2                      # D > 4096
    assert _lipar(lib, ok, frames=3) == 1                        # 3 does not divide 256
    assert _lipar(lib, ok, frames=0) == 1
    assert _lipar(lib, ok, tau=float("nan")) == 1
    assert _lipar(lib, ok, ptr=4098) == 1                        # misaligned tensor
    assert b"bsa_lipar_prune" in lib.bsa_last_error()
    p = ctypes.c_void_p(4096)
    assert lib.bsa_lipar_restore(p, 0, ctypes.byref(ok), 3, p, p, p, None) == 1
    assert lib.bsa_lipar_restore(p, 1, ctypes.byref(ok), 4, p, p, p, None) == 2   # fp32 not implemented


def _mixed(lib, shape, r=0.5, block=128, ws=1 << 30, ptr=4096, mask=4096, scale=0.1):
    p, m = ctypes.c_void_p(ptr), ctypes.c_void_p(mask)
    return lib.bsa_mixed_attn_fwd(p, p, p, p, 0, ctypes.byref(shape), m, m, None, block, ctypes.c_float(scale),
                                  ctypes.c_float(r), ctypes.c_void_p(1 << 20), ws, None)


def test_mixed_attention_argument_checks(lib):
    ok = _shape(B=1, H=2, N=1000, D=128)
    assert _mixed(lib, ok, r=-0.1) == 1
    assert _mixed(lib, ok, r=1.5) == 1
    assert _mixed(lib, ok, r=float("nan")) == 1
    assert _mixed(lib, ok, scale=-0.1) == 1
    assert _mixed(lib, _shape(B=1, H=2, N=1000, D=64)) == 2      # D = 128 only
    assert _mixed(lib, ok, block=32) == 2
    assert _mixed(lib, ok, mask=0) == 1                           # softmax term needs the mask
    assert _mixed(lib, ok, ws=16) == 4                            # linear term needs the workspace
    assert _mixed(lib, ok, ptr=4098) == 1
    assert b"bsa_mixed_attn_fwd" in lib.bsa_last_error()


def _causal(lib, shape, ws=1 << 30, ptr=4096, s_in=None, z_in=None, s_out=None):
    p = ctypes.c_void_p(ptr)
    return lib.bsa_causal_linear_attn_fwd(p, p, p, p, 0, ctypes.byref(shape), s_in, z_in, s_out, None,
                                          ctypes.c_void_p(1 << 20), ws, None)


def test_causal_linear_argument_checks(lib):
    ok = _shape(B=1, H=2, N=1000, D=128)
    assert _causal(lib, _shape(B=1, H=2, N=1000, D=64)) == 2      # D = 128 only
    assert lib.bsa_causal_linear_attn_workspace(ctypes.byref(_shape(D=64))) == 0
    assert _causal(lib, ok, ws=16) == 4
    assert _causal(lib, ok, ptr=4098) == 1
    assert _causal(lib, ok, s_in=ctypes.c_void_p(4096)) == 1        # S_in without z_in
    assert _causal(lib, ok, s_in=ctypes.c_void_p(4096), z_in=ctypes.c_void_p(4100)) == 1   # misaligned z_in
    assert _causal(lib, ok, s_out=ctypes.c_void_p(4104)) == 1
    assert b"bsa_causal_linear_attn_fwd" in lib.bsa_last_error()
    p = ctypes.c_void_p(4096)
    assert lib.bsa_causal_linear_attn_fwd(p, p, p, p, 1, ctypes.byref(ok), None, None, None, None, p,
                                          1 << 30, None) == 2       # fp32 not implemented


def test_causal_workspace_plan(lib):
    for N, H in ((1, 1), (7, 2), (1000, 3), (32760, 12), (196560, 12), (4100, 1)):
        sh = _shape(B=1, H=H, N=N, D=128)
        w = lib.bsa_causal_linear_attn_workspace(ctypes.byref(sh))
        assert w > 0 and w % 256 == 0
        tiles = -(-N // 32)
        splits = w // (H * (128 * 128 + 128) * 4)              # about 512 / H state splits
        assert 1 <= splits <= max(2 * 256 // H, 1) + 1 and splits <= tiles


def test_kmeans_and_row_permute_argument_checks(lib):
    p = ctypes.c_void_p(4096)
    ok_ = _shape(B=1, H=2, N=1000, D=128)

    def km(shape=ok_, C=10, iters=3, dtype=0, ws=1 << 30, ptr=p):
        return lib.bsa_kmeans(ptr, dtype, ctypes.byref(shape), C, iters, p, p, None, None,
                              ctypes.c_void_p(1 << 20), ws, None)

    assert km(shape=_shape(D=64)) == 2
    assert km(C=0) == 1 and km(C=1025) == 1
    assert km(iters=-1) == 1
    assert km(dtype=1) == 2
    assert km(ws=16) == 4
    assert km(ptr=ctypes.c_void_p(4098)) == 1
    assert lib.bsa_kmeans_workspace(ctypes.byref(ok_), 0) == 0
    assert lib.bsa_kmeans_workspace(ctypes.byref(ok_), 500) > 0
    assert lib.bsa_gather_rows(p, 0, ctypes.byref(_shape(D=4, sn=8)), p, ctypes.c_void_p(8192), None) == 1
    assert lib.bsa_gather_rows(p, 0, ctypes.byref(ok_), p, p, None) == 1          # in place
    assert lib.bsa_scatter_rows(p, 7, ctypes.byref(ok_), p, ctypes.c_void_p(8192), None) == 1
    assert b"bsa_scatter_rows" in lib.bsa_last_error()


def test_attention_backward_argument_checks(lib):
    p = ctypes.c_void_p(4096)
    ok_ = _shape(B=1, H=2, N=1000, D=128)

    def bwd(shape=ok_, block=128, dtype=0, ws=1 << 30, scale=0.1, ptr=p):
        return lib.bsa_block_sparse_attn_bwd(ptr, p, p, p, p, p, dtype, ctypes.byref(shape), p, p, p, p, block,
                                             ctypes.c_float(scale), p, p, p, ctypes.c_void_p(1 << 20), ws, None)

    assert bwd(shape=_shape(D=64)) == 2
    assert bwd(block=64) == 2
    assert bwd(dtype=1) == 2
    assert bwd(scale=float("inf")) == 1
    assert bwd(scale=-0.1) == 1
    assert bwd(ws=16) == 4
    assert bwd(ptr=ctypes.c_void_p(4098)) == 1
    assert b"bsa_block_sparse_attn_bwd" in lib.bsa_last_error()
    assert lib.bsa_transpose_block_mask(p, p, 10, p, p, 99, None) == 3          # capacity < nb * nb
    assert lib.bsa_transpose_block_mask(p, p, 0, p, p, 99, None) == 1


def test_route_budget_is_exact_up_to_the_largest_sequence(lib):
    """floor(N * N * ppm / 10^6) with no overflow: N * N * ppm needs 82 bits at
    N = 2^31 - 1 and ppm = 10^6 (the 64-bit product wrapped from N of about 3M)."""
    for N in (0, 1, 32760, 196560, 3_037_000, 3_100_000, 7_800_000, 50_000_000, 2**31 - 1):
        for ppm in (0, 1, 150_000, 999_999, 1_000_000):
            assert lib.bsa_route_budget(N, ppm) == N * N * ppm // 1_000_000, (N, ppm)
    assert lib.bsa_route_budget(32760, 150_000) == 160_982_640
    assert lib.bsa_route_budget(-1, 10) == -1
    assert lib.bsa_route_budget(10, 1_000_001) == -1
    assert lib.bsa_route_budget(10, -1) == -1


def test_linear_no_alloc_argument_checks(lib):
    """Validation of the no-allocation linear attention runs before any HIP call:
    bad arguments and shapes whose workspace exceeds the library's scratch are
    rejected with no device present."""
    p = ctypes.c_void_p(4096)
    assert lib.bsa_linear_attn_noalloc_max_scratch() == 40 << 20

    def call(shape, dtype=0, ptr=p):
        return lib.bsa_linear_attn_fwd_noalloc(ptr, p, p, p, dtype, ctypes.byref(shape), None, None, None)

    big = _shape(B=1, H=600, N=1000, D=128)
    assert lib.bsa_linear_attn_workspace(ctypes.byref(big)) > 40 << 20
    assert call(big) == 2
    assert b"scratch" in lib.bsa_last_error()
    assert call(_shape(B=1, H=12, N=32760, D=96)) == 2           # D in {64, 128}
    assert call(_shape(B=1, H=2, N=100, D=128), dtype=1) == 2
    assert call(_shape(B=1, H=2, N=100, D=128), ptr=ctypes.c_void_p(4098)) == 1
    assert call(_shape(B=1, H=2, N=0, D=128)) == 1
    # the benchmark shape fits
    assert lib.bsa_linear_attn_workspace(ctypes.byref(_shape(B=1, H=12, N=196560, D=128))) <= 40 << 20


def test_cluster_centroids_output_choice(lib):
    """bsa_cluster_centroids computes the query set, the key set or both; the
    argument checks run before any HIP call."""
    p = ctypes.c_void_p(4096)
    sh = _shape(B=1, H=2, N=1000, D=128)

    def cc(qc, kc, vc, q=p):
        return lib.bsa_cluster_centroids(q, p, p, 0, ctypes.byref(sh), p, 10, p, 20, qc, kc, vc, None)

    assert cc(None, None, None) == 1                         # nothing asked for
    assert cc(None, p, None) == 1                            # k_cent without v_cent
    assert cc(p, None, None, q=None) == 1                    # query centroids need q
    assert cc(p, None, None, q=ctypes.c_void_p(4098)) == 1   # misaligned q
    assert b"bsa_cluster_centroids" in lib.bsa_last_error()


def test_fused_compensation_argument_checks(lib):
    p = ctypes.c_void_p(4096)
    sh = _shape(B=1, H=2, N=1000, D=128)

    def fused(use_given=0, ppm=150000, ws=1 << 30):
        return lib.bsa_centroid_compensate(p, p, p, p, None, 0, ctypes.byref(sh), p, 10, p, 20, ppm, use_given,
                                           ctypes.c_float(0.1), p, p, None, ctypes.c_void_p(1 << 20), ws, None)

    assert fused(use_given=2) == 1
    assert fused(ppm=-1) == 1
    assert fused(ws=16) == 4
    assert b"bsa_centroid_compensate" in lib.bsa_last_error()
    need = lib.bsa_centroid_compensate_workspace(ctypes.byref(sh), 10, 20)
    assert need % 256 == 0 and need >= lib.bsa_route_scores_workspace(ctypes.byref(sh), 10, 20)
    assert lib.bsa_route_select_workspace(ctypes.byref(sh), 10, 20) >= 2 * 8 * 2048 * 8   # cost histograms
