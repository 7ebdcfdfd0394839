"""Pins for oracle.rotation: orthogonality, Haar distribution, special cases."""
import json
import os

import numpy as np
import pytest
from scipy import linalg as sla
from scipy import stats

from kv_cache_compression_quantize_amd import inputs
from oracle import codebook as cb
from oracle import rotation

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_fp32_rotation_is_orthogonal():
    for layer, d in ((0, 128), (3, 128), (0, 256)):
        g, _ = inputs.layer_gaussians(layer, d, d)
        pi = rotation.rotation_fp32(g).astype(np.float64)
        err = np.max(np.abs(pi.T @ pi - np.eye(d)))
        assert err <= 1e-6, err
        assert abs(abs(np.linalg.det(pi)) - 1.0) < 1e-4


def test_storage_size_matches_page():
    # TurboQuant article section 二: a 128x128 rotation is 64 KB -> 4 bytes per entry (fp32).
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        fig = json.load(f)["turboquant_rotation_storage"]
    g, _ = inputs.layer_gaussians(0, 128, 128)
    pi = rotation.rotation_fp32(g)
    assert list(pi.shape) == fig["shape"] and pi.nbytes == fig["value_bytes"]


def test_upper_triangular_input_gives_identity():
    # G = R with positive diagonal is its own QR factor: Q = I.
    rng = np.random.default_rng(0)
    r = np.triu(rng.standard_normal((16, 16)))
    np.fill_diagonal(r, np.abs(np.diag(r)) + 0.5)
    np.testing.assert_allclose(rotation.rotation_from_gaussian(r), np.eye(16), atol=1e-14)
    # a negative diagonal entry flips the sign of Q's column, then the sign fix undoes it
    r2 = r.copy()
    r2[:, 3] *= -1
    q = rotation.rotation_from_gaussian(r2)
    np.testing.assert_allclose(np.abs(q), np.eye(16), atol=1e-14)


def test_haar_rotation_of_fixed_vector_is_uniform_on_sphere():
    # For Haar Pi and a fixed unit u, Pi u is uniform on the sphere: its first coordinate
    # follows the sphere-coordinate law, and E[y_j^2] = 1/d.
    d = 6
    rng = np.random.default_rng(7)
    u = np.zeros(d)
    u[0] = 1.0
    ys = []
    for _ in range(6000):
        pi = rotation.rotation_from_gaussian(rng.standard_normal((d, d)))
        ys.append(pi @ u)
    ys = np.array(ys)
    for j in range(d):
        assert stats.kstest(ys[:, j], lambda x: cb.cdf(x, d)).pvalue > 1e-3
    np.testing.assert_allclose(np.mean(ys ** 2, axis=0), 1.0 / d, atol=0.012)


def test_layer_seeds_differ_and_repeat():
    g0, s0 = inputs.layer_gaussians(0, 128, 128)
    g0b, s0b = inputs.layer_gaussians(0, 128, 128)
    g1, _ = inputs.layer_gaussians(1, 128, 128)
    np.testing.assert_array_equal(g0, g0b)
    np.testing.assert_array_equal(s0, s0b)
    assert not np.allclose(g0, g1)
    assert inputs.layer_seed(0) == 42 and inputs.layer_seed(5) == 77


# ---------------------------------------------------------------- randomised Hadamard


@pytest.mark.parametrize("d", [1, 2, 4, 64, 128, 256])
def test_sylvester_matches_library(d):
    np.testing.assert_array_equal(rotation.sylvester_hadamard(d), sla.hadamard(d))


def test_sylvester_small_textbook():
    np.testing.assert_array_equal(rotation.sylvester_hadamard(2), [[1, 1], [1, -1]])
    with pytest.raises(ValueError):
        rotation.sylvester_hadamard(96)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_randomized_hadamard_is_orthogonal_and_a_fast_transform(d):
    g, _ = inputs.layer_gaussians(3, d, d)
    pi = rotation.randomized_hadamard(g)
    np.testing.assert_allclose(pi @ pi.T, np.eye(d), atol=1e-13)
    # Pi x = FWHT(D x) / sqrt(d): the explicit matrix against the butterfly recursion
    x = np.random.default_rng(d).standard_normal((7, d))
    s = rotation.hadamard_signs(g)
    np.testing.assert_allclose(x @ pi.T, rotation.fwht(x * s) / np.sqrt(d), rtol=1e-12, atol=1e-13)
    # the signs are random: about half of them flip
    assert 0.3 * d < np.sum(s < 0) < 0.7 * d


def test_hadamard_spreads_an_outlier_channel():
    # NexusQuant stage 4: the energy of a single channel is spread evenly over all d
    d = 128
    g, _ = inputs.layer_gaussians(0, d, d)
    pi = rotation.randomized_hadamard(g)
    e = np.zeros(d)
    e[17] = 10.0
    np.testing.assert_allclose(np.abs(pi @ e), 10.0 / np.sqrt(d), rtol=1e-13)
