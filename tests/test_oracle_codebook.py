"""Pins for oracle.codebook: closed forms, textbook limits, invariants."""
import json
import os

import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import codebook as cb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _max_table():
    with open(os.path.join(GOLDEN, "max1960_gaussian.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_d3_is_uniform_quantiser(bits):
    # f_3 is uniform on [-1, 1] (Archimedes), so Lloyd-Max is the uniform quantiser:
    # centroids -1 + (2k+1)/L, and d*MSE = d * (2/L)^2 / 12.
    L = 1 << bits
    c, t, _ = cb.lloyd_max(3, bits)
    expect = -1.0 + (2.0 * np.arange(L) + 1.0) / L
    np.testing.assert_allclose(c, expect, atol=1e-14)
    np.testing.assert_allclose(t, 0.5 * (expect[:-1] + expect[1:]), atol=1e-14)
    D = cb.distortion(3, c, t)
    assert abs(3 * D - 3 * (2.0 / L) ** 2 / 12.0) < 1e-12


@pytest.mark.parametrize("d", [3, 4, 5, 8, 16, 64, 128, 256])
def test_one_bit_closed_form(d):
    # 1 bit: cells are t<0 and t>0, centroid = +-E|T| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)).
    c, t, _ = cb.lloyd_max(d, 1)
    e_abs = np.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / np.sqrt(np.pi)
    np.testing.assert_allclose(c, [-e_abs, e_abs], rtol=1e-13)
    assert t[0] == 0.0


def test_one_bit_value_d128():
    c, _, _ = cb.lloyd_max(128, 1)
    assert abs(c[1] - 0.0706616) < 5e-7


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_large_d_limit_is_max_gaussian_table(bits):
    # sqrt(d) * T -> N(0, 1): the codebook scaled by sqrt(d) tends to Max's Gaussian quantiser.
    tab = _max_table()[str(bits)]
    d = 1 << 16
    c, t, _ = cb.lloyd_max(d, bits, tol=1e-13)
    L = 1 << bits
    pos = np.sqrt(d) * c[L // 2:]
    np.testing.assert_allclose(pos, tab["levels"], atol=6e-4)
    thr = np.sqrt(d) * t[L // 2 - 1:]
    np.testing.assert_allclose(thr, tab["thresholds"], atol=6e-4)
    assert abs(d * cb.distortion(d, c, t) - tab["mse"]) < 2e-4


def test_distortion_scales_as_quarter_per_bit():
    # TurboQuant article section 一: distortion scales as 1/4^b.  High-resolution theory gives
    # 4^b * MSE_b -> Panter-Dite constant (sqrt(3) pi / 2 for the Gaussian limit), from below.
    d = 4096
    scaled = []
    for bits in range(1, 6):
        c, t, _ = cb.lloyd_max(d, bits, tol=1e-13)
        scaled.append((4.0 ** bits) * d * cb.distortion(d, c, t))
    scaled = np.array(scaled)
    assert np.all(np.diff(scaled) > 0)
    pd = _max_table()["panter_dite_constant"]["value"]
    assert scaled[-1] < pd and pd - scaled[-1] < 0.2
    ratios = scaled[:-1] / scaled[1:] * 4.0          # MSE_b / MSE_{b+1}
    assert np.all((ratios > 2.8) & (ratios < 4.0))


@pytest.mark.parametrize("d,bits", [(128, 2), (128, 3), (256, 3), (7, 2)])
def test_fixed_point_by_quadrature(d, bits):
    # Both Lloyd conditions, re-checked with plain adaptive quadrature of t f and f
    # (independent of the closed-form moment and the incomplete beta used by the solver).
    c, t, _ = cb.lloyd_max(d, bits)
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-16)
    edges = np.concatenate(([-1.0], t, [1.0]))
    for k in range(len(c)):
        m0, _ = integrate.quad(lambda x: cb.pdf(x, d), edges[k], edges[k + 1], epsabs=1e-14, epsrel=1e-13, limit=200)
        m1, _ = integrate.quad(lambda x: x * cb.pdf(x, d), edges[k], edges[k + 1], epsabs=1e-15, epsrel=1e-13, limit=200)
        assert abs(m1 / m0 - c[k]) < 1e-11 * max(1.0, abs(c[k]) * np.sqrt(d))


@pytest.mark.parametrize("d,bits", [(128, 2), (256, 3), (16, 3)])
def test_symmetry_and_unique_fixed_point(d, bits):
    c, t, _ = cb.lloyd_max(d, bits)
    np.testing.assert_array_equal(c, -c[::-1])
    assert t[len(t) // 2] == 0.0
    # f_d is log-concave (d >= 3): any start reaches the same fixed point, even unsymmetrised.
    rng = np.random.default_rng(0)
    init = np.sort(rng.uniform(-0.5, 0.3, size=1 << bits))
    c2, _, _ = cb.lloyd_max(d, bits, init=init, symmetric=False)
    np.testing.assert_allclose(c2, c, atol=1e-12)


def test_density_is_sphere_coordinate():
    # Monte Carlo: one coordinate of a uniform point on S^{d-1} follows cdf(., d).
    rng = np.random.default_rng(1)
    for d in (3, 8, 128):
        g = rng.standard_normal((40000, d))
        u = g[:, 0] / np.linalg.norm(g, axis=1)
        res = stats.kstest(u, lambda x: cb.cdf(x, d))
        assert res.pvalue > 1e-3, (d, res)
    # and it integrates to one, with variance 1/d
    for d in (3, 8, 128):
        tot, _ = integrate.quad(lambda x: cb.pdf(x, d), -1, 1, points=[0.0])
        var, _ = integrate.quad(lambda x: x * x * cb.pdf(x, d), -1, 1, points=[0.0])
        assert abs(tot - 1) < 1e-10 and abs(var - 1.0 / d) < 1e-10


def test_codebook_fp32_values_d128():
    c, t = cb.codebook_fp32(128, 2)
    assert c.dtype == np.float32 and t.dtype == np.float32
    # sqrt(128) c = +-0.45245, +-1.50519 (exact sphere density; the Gaussian limit is 0.4528, 1.510)
    np.testing.assert_allclose(np.sqrt(128) * c.astype(np.float64), [-1.50519, -0.45245, 0.45245, 1.50519], atol=2e-5)
