"""Pins for oracle.values (min-max grouped value codec)."""
import json
import os

import numpy as np
import pytest

from oracle import values

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fig():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("vb", [2, 4])
def test_nearest_level_and_error_bound(vb):
    v = np.random.default_rng(0).standard_normal((400, 128)).astype(np.float32)
    codes, scale, vmin = values.quantize_values(v, vb)
    v_hat = values.dequantize_values(codes, scale, vmin)
    s = np.repeat(scale.astype(np.float64), 32, axis=1)
    mn = np.repeat(vmin.astype(np.float64), 32, axis=1)
    # brute force: the code is the nearest of the 2**vb levels (away from rounding midpoints)
    levels = np.arange(1 << vb)[None, None, :] * s[:, :, None] + mn[:, :, None]
    near = np.argmin(np.abs(v.astype(np.float64)[:, :, None] - levels), axis=2)
    ok = ~values.code_window(v, scale, vmin, eps=1e-4)
    np.testing.assert_array_equal(codes[ok], near[ok])
    assert np.all(np.abs(v - v_hat) <= s / 2 * (1 + 1e-5) + 1e-7)
    # the group minimum is reconstructed exactly (code 0), the maximum by the top code
    g = v.reshape(400, 4, 32)
    np.testing.assert_array_equal(g.min(axis=2), vmin)
    top = codes.reshape(400, 4, 32)[np.arange(400)[:, None], np.arange(4)[None, :], g.argmax(axis=2)]
    assert np.all(top == (1 << vb) - 1)


def test_constant_group():
    v = np.zeros((2, 64), np.float32)
    v[0, :32] = 1.5
    v[1] = -2.0
    codes, scale, vmin = values.quantize_values(v, 2)
    assert np.all(codes == 0) and np.all(scale == 0)
    np.testing.assert_array_equal(values.dequantize_values(codes, scale, vmin), v)


def test_round_half_even_in_fp32():
    # group values 0, 1.5, 3 -> scale 1, t = 1.5 exactly -> rint -> 2 (half to even); 0.5 -> 0
    v = np.zeros((1, 32), np.float32)
    v[0, 1] = 1.5
    v[0, 2] = 3.0
    v[0, 3] = 0.5
    v[0, 4] = 2.5
    codes, scale, vmin = values.quantize_values(v, 2)
    assert scale[0, 0] == 1.0
    assert list(codes[0, :5]) == [0, 2, 3, 0, 2]


@pytest.mark.parametrize("vb", [2, 4])
def test_cosine_similarity_matches_page(vb):
    # TurboQuant article section 七: cos_sim ~0.94 for 2-bit values, 0.997 for 4-bit.
    page = _fig()["turboquant_value_cos_sim"]["value"][str(vb)]
    v = np.random.default_rng(1).standard_normal((4000, 128)).astype(np.float32)
    v_hat = values.dequantize_values(*values.quantize_values(v, vb))
    cos = np.sum(v * v_hat, axis=1) / (np.linalg.norm(v, axis=1) * np.linalg.norm(v_hat, axis=1))
    assert abs(np.mean(cos) - page) < (0.012 if vb == 2 else 0.002), np.mean(cos)
