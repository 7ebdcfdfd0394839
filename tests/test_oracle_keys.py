"""Pins for oracle.keys and oracle.layout."""
import json
import os

import numpy as np
import pytest

from kv_cache_compression_quantize_amd import inputs
from oracle import codebook as cb
from oracle import keys, layout, rotation

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _params(d, w, m, layer=0):
    g, s = inputs.layer_gaussians(layer, d, m)
    pi = rotation.rotation_fp32(g)
    s32 = s.astype(np.float32)
    if w > 0:
        c, t = cb.codebook_fp32(d, w)
    else:
        c, t = np.zeros(0, np.float32), np.zeros(0, np.float32)
    return pi, s32, c, t


def test_index_is_nearest_centroid():
    # boundary count == brute-force nearest centroid (Lloyd-Max cells are Voronoi cells)
    d, w = 128, 2
    pi, s, c, t = _params(d, w, d)
    x = np.random.default_rng(0).standard_normal((500, d))
    qk = keys.quantize_keys(x, pi, s, c, t, w)
    near = np.argmin(np.abs(qk.y[:, :, None] - c.astype(np.float64)[None, None, :]), axis=2)
    ok = ~keys.index_window(qk.y, t, 1e-12)
    np.testing.assert_array_equal(qk.idx[ok], near[ok])


@pytest.mark.parametrize("w", [0, 1, 2, 3])
def test_power_of_two_scale_invariance(w):
    d, m = 64, 128
    pi, s, c, t = _params(d, w, m) if w > 0 else _params(d, 0, m)
    if w > 0:
        c, t = cb.codebook_fp32(d, w)
    x = np.random.default_rng(1).standard_normal((50, d))
    a = keys.quantize_keys(x, pi, s, c, t, w)
    for e in (-7, 3, 20):
        b = keys.quantize_keys(x * 2.0 ** e, pi, s, c, t, w)
        np.testing.assert_array_equal(a.idx, b.idx)
        np.testing.assert_array_equal(a.bits, b.bits)
        np.testing.assert_array_equal(a.norm * 2.0 ** e, b.norm)
        np.testing.assert_array_equal(a.rnorm * 2.0 ** e, b.rnorm)


def test_zero_key():
    d, w = 128, 2
    pi, s, c, t = _params(d, w, d)
    x = np.zeros((2, d))
    x[1, 5] = 1.0
    qk = keys.quantize_keys(x, pi, s, c, t, w)
    assert qk.norm[0] == 0.0 and qk.rnorm[0] == 0.0
    assert np.all(qk.bits[0])
    assert np.all(qk.idx[0] == int(np.sum(t < 0)))
    k_hat = keys.dequantize_keys(qk.idx, qk.bits, qk.norm, qk.rnorm, pi, s, c, w)
    assert np.all(k_hat[0] == 0.0)


def test_residual_norm_in_rotated_space():
    # Pi orthogonal => ||x - n Pi^T c|| == n ||y - c[idx]||  (independent of how r is formed)
    d, w = 128, 3
    pi, s, c, t = _params(d, w, d)
    x = np.random.default_rng(2).standard_normal((300, d)) * 3.0
    qk = keys.quantize_keys(x, pi, s, c, t, w)
    alt = qk.norm * np.linalg.norm(qk.y - c.astype(np.float64)[qk.idx], axis=1)
    np.testing.assert_allclose(qk.rnorm, alt, rtol=2e-6)


def test_pure_qjl_mode_signs_of_sketch():
    # A-QJL: no rotation, no codebook; signs of S x, stored norm is ||x||
    d, m = 128, 192
    _, s, _, _ = _params(d, 0, m)
    x = np.random.default_rng(3).standard_normal((40, d))
    qk = keys.quantize_keys(x, None, s, np.zeros(0), np.zeros(0), 0)
    np.testing.assert_array_equal(qk.bits, (x @ s.astype(np.float64).T) >= 0)
    np.testing.assert_allclose(qk.rnorm, np.linalg.norm(x, axis=1))


@pytest.mark.parametrize("d,w", [(128, 1), (128, 2), (128, 3)])
def test_distortion_matches_codebook_mse(d, w):
    # E||u - Pi^T c[idx]||^2 over random unit keys == d * MSE of the codebook
    pi, s, c, t = _params(d, w, d)
    x = np.random.default_rng(4).standard_normal((6000, d))
    qk = keys.quantize_keys(x, pi, s, c, t, w)
    u = x / qk.norm[:, None]
    rec = c.astype(np.float64)[qk.idx] @ pi.astype(np.float64)
    emp = np.mean(np.sum((u - rec) ** 2, axis=1))
    c64, t64, _ = cb.lloyd_max(d, w)
    theory = d * cb.distortion(d, c64, t64)
    assert abs(emp - theory) < 0.02 * theory


def test_golden_layouts():
    with open(os.path.join(GOLDEN, "layout_example.json")) as f:
        g = json.load(f)
    e = g["key_codes_d32_w2"]
    idx = np.zeros((1, e["d"]), dtype=np.int64)
    for k, v in e["idx_nonzero"].items():
        idx[0, int(k)] = v
    assert layout.pack_code_planes(idx, 2)[0].tobytes().hex() == e["row_hex"]
    e = g["signs_m64"]
    bits = np.zeros((1, 64), dtype=bool)
    bits[0, e["set"]] = True
    assert layout.pack_bits(bits)[0].tobytes().hex() == e["row_hex"]
    for key, vb in (("value_codes_d32_vb2", 2), ("value_codes_d32_vb4", 4)):
        e = g[key]
        codes = np.zeros((32, 32), dtype=np.int64)
        for t, ch, v in e["codes_nonzero"]:
            codes[t, ch] = v
        out = layout.pack_value_codes(codes, vb).reshape(-1)
        assert out.size == e["block_bytes"]
        assert {str(i): int(x) for i, x in enumerate(out) if x} == e["bytes_nonzero"]


def test_pack_roundtrip():
    rng = np.random.default_rng(5)
    for d, w in ((128, 2), (256, 3), (64, 1)):
        idx = rng.integers(0, 1 << w, size=(7, d))
        np.testing.assert_array_equal(layout.unpack_code_planes(layout.pack_code_planes(idx, w), d, w), idx)
    for k in (64, 192, 512):
        bits = rng.random((9, k)) < 0.5
        np.testing.assert_array_equal(layout.unpack_bits(layout.pack_bits(bits), k), bits)
    for vb in (2, 4):
        for T in (32, 77, 130):
            codes = rng.integers(0, 1 << vb, size=(T, 128))
            packed = layout.pack_value_codes(codes, vb)
            assert packed.shape == ((T + 31) // 32 * 32, 128 * vb // 8)
            np.testing.assert_array_equal(layout.unpack_value_codes(packed, T, 128, vb), codes)


def test_bit_budget_and_compression_ratio():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        fig = json.load(f)
    budget = fig["turboquant_bit_budget"]["value"]
    # 3-bit keys = (b-1) Lloyd-Max bits + 1 QJL bit per coordinate, m == d
    d = 128
    rb = layout.row_bytes(d, w=2, m=d)
    assert 8 * (rb["key_codes"] + rb["key_signs"]) / d == budget["key_bits_total"]
    assert 8 * rb["val_codes"] / d == budget["value_bits"]
    # compression at head_dim 256 with 3-bit keys / 2-bit values, fp32 side information
    ratio = fig["turboquant_compression_ratio_d256"]
    rb = layout.row_bytes(256, w=2, m=256)
    total = sum(rb.values())
    assert round(2 * 2 * 256 / total, 2) == ratio["value"]


def test_aqjl_layer_group_sketch_dims():
    # A-QJL article, section 实际部署与使用: 4 groups split at layers 8, 16, 24 with k = 512/384/256/192
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["aqjl_layer_groups"]["value"]
    w = inputs.WORKLOADS["aqjl_32layer_gqa32x8_b16_t32k"]
    bounds = [0] + fig["layer_group_boundaries"] + [32]
    for g, k in enumerate(fig["sketch_dims"]):
        for layer in range(bounds[g], bounds[g + 1]):
            assert w.sketch_dim(layer) == k


@pytest.mark.parametrize("d,w", [(128, 2), (256, 3)])
def test_codebook_still_fits_under_a_randomized_hadamard_rotation(d, w):
    # the Lloyd-Max codebook is designed for Haar-rotated coordinates; under a
    # randomised Hadamard rotation (NexusQuant stage 4) the coordinates are only
    # approximately that law, so re-check the distortion: isotropic keys stay
    # within 3 % of the codebook's MSE; keys dominated by 4 outlier channels x10
    # (whose rotated coordinates are close to a few discrete values, not the
    # Beta law) must not be worse than it
    _, s, c, t = _params(d, w, d)
    g, _ = inputs.layer_gaussians(0, d, d)
    pi = rotation.randomized_hadamard_fp32(g)
    c64, t64, _ = cb.lloyd_max(d, w)
    theory = d * cb.distortion(d, c64, t64)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6000, d))
    xo = x.copy()
    xo[:, [3, 40, 77, 101]] *= 10.0
    emp = []
    for keys_ in (x, xo):
        qk = keys.quantize_keys(keys_, pi, s, c, t, w)
        u = keys_ / qk.norm[:, None]
        rec = c.astype(np.float64)[qk.idx] @ pi.astype(np.float64)
        emp.append(np.mean(np.sum((u - rec) ** 2, axis=1)))
    assert abs(emp[0] - theory) < 0.03 * theory, (emp, theory)
    assert emp[1] < 1.03 * theory, (emp, theory)
