"""Checks of the seeded input generators (CPU only)."""

import numpy as np

from synth import gen, get_workload


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 0.0, 3.0e38], np.float32)
    b = gen.f32_to_bf16_bits(x)
    y = gen.bf16_bits_to_f32(b)
    assert y[0] == 1.0
    assert y[1] == 1.0                       # halfway -> even (mantissa 0)
    assert y[2] == 1.0 + 2 ** -7             # 1.5 ulp -> up to the even neighbour
    assert y[3] == -2.5 and y[4] == 0.0
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    rb = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(r))
    assert np.abs(rb - r).max() <= np.abs(r).max() * 2 ** -8


def test_streams_are_per_slice_and_repeatable():
    wl = gen.scaled(get_workload("lvsa_32k"), H=3, frames=4, frame_h=4, frame_w=5)
    a = gen.make_qkv(wl)
    b = gen.make_qkv(wl, heads=[2])
    assert np.array_equal(a["k"][:, 2:3], b["k"])
    assert not np.array_equal(a["q"][:, 0], a["q"][:, 1])


def test_ar1_frame_component_statistics():
    g = gen.ar1_frame_component((9, 9), 4000, 64, 0.9).astype(np.float64)
    lag1 = (g[1:] * g[:-1]).mean() / (g * g).mean()
    assert abs(lag1 - 0.9) < 0.03
    assert abs(g.var() - 1.0) < 0.15


def test_ar1_tokens_variance_and_frame_correlation():
    wl = gen.scaled(get_workload("lvsa_32k"), H=1, frames=6, frame_h=10, frame_w=10)
    x = gen.to_f64(gen.make_qkv(wl)["q"][0, 0], "bf16").reshape(6, 100, wl.D)
    assert abs(x.mean()) < 0.3 and abs(x.var() - 2.0) < 0.5
    fm = x.mean(axis=1)                       # per-frame mean estimates g_f
    c = (fm[1:] * fm[:-1]).sum() / np.sqrt((fm[1:] ** 2).sum() * (fm[:-1] ** 2).sum())
    assert c > 0.5


def test_clustered_recipe_offsets_and_permutation():
    wl = gen.scaled(get_workload("svg_ear_32k"), H=1, frames=2, frame_h=10, frame_w=20,
                    n_q_clusters=8, n_k_clusters=12, kmeans_iters=3)
    d = gen.make_clustered(wl)
    assert d["q_off"][0, -1] == wl.N and d["k_off"][0, -1] == wl.N
    assert (np.diff(d["q_off"][0]) >= 0).all() and (np.diff(d["k_off"][0]) >= 0).all()
    assert sorted(d["perm_q"][0]) == list(range(wl.N))
    # tokens of one query cluster are closer to their own mean than to others' (on average)
    q = gen.to_f64(d["q"][0, 0], "bf16")
    off = d["q_off"][0]
    cents = np.array([q[off[a]:off[a + 1]].mean(0) for a in range(8) if off[a + 1] > off[a]])
    assert len(cents) > 1
