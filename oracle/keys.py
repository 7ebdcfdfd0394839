"""Key quantisation (oracle, float64).

TurboQuant article §二 (three-stage pipeline) and §五 (quantize() returns the
MSE indices, QJL sign bytes, residual norm and original norm):

1. store n = ||x||, move x / n onto the unit sphere, rotate: y = Pi (x / n);
2. Lloyd-Max: each coordinate gets the index of its cell, found by comparing
   y_j with the decision boundaries (w = b - 1 bits per coordinate);
3. reconstruct x~ = n * Pi^T c[idx], residual r = x - x~, project it through
   the Gaussian matrix S, keep only the signs (one bit per sketch row), and
   store gamma = ||r||.

For pure QJL keys (A-QJL article, section "QJL：量化Johnson-Lindenstrauss变换";
w = 0) there is no rotation and no codebook: r = x, the signs are sign(S x)
and only ||x|| is stored.

Readings where the pages are silent (listed in the design notes):
* the residual lives in the original space and gamma = ||r|| at full scale;
* an index counts the boundaries strictly below y_j (a tie takes the lower cell);
* a zero projection S r = 0 stores bit 1 (+1); a zero key has n = 0, y = 0,
  r = 0, gamma = 0 and every sign bit 1.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import layout


@dataclass
class QuantizedKeys:
    idx: np.ndarray        # [N, d] int64 Lloyd-Max indices (w > 0)
    bits: np.ndarray       # [N, m] bool, True = non-negative projection
    norm: np.ndarray       # [N] float64, ||x||
    rnorm: np.ndarray      # [N] float64, ||r|| (== norm for w == 0)
    y: np.ndarray          # [N, d] float64 rotated unit-sphere coordinates (diagnostic)
    z: np.ndarray          # [N, m] float64 projections S r (diagnostic)

    def packed(self, w: int, side_f16: bool = False):
        """The cache rows: (codes, signs, norm, residual norm), the norms as
        stored (fp32, or half with the half side-information option)."""
        codes = layout.pack_code_planes(self.idx, w)
        signs = layout.pack_bits(self.bits)
        return (codes, signs, layout.stored_side(self.norm, side_f16),
                layout.stored_side(self.rnorm, side_f16))


def quantize_keys(x, rotation, sketch, centroids, boundaries, w: int) -> QuantizedKeys:
    """Quantise keys x [N, d] (values exactly as the device sees them).

    rotation [d, d] (y = Pi x), sketch [m, d], centroids [2**w], boundaries
    [2**w - 1] are the stored fp32 parameters; everything is evaluated in
    float64 from them.
    """
    x = np.asarray(x, dtype=np.float64)
    S = np.asarray(sketch, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=1))
    N, d = x.shape
    if w == 0:
        r = x
        idx = np.zeros((N, d), dtype=np.int64)
        y = np.zeros((N, d))
        gamma = n.copy()
    else:
        Pi = np.asarray(rotation, dtype=np.float64)
        c = np.asarray(centroids, dtype=np.float64)
        t = np.asarray(boundaries, dtype=np.float64)
        safe = np.where(n > 0, n, 1.0)
        u = np.where((n > 0)[:, None], x / safe[:, None], 0.0)
        y = u @ Pi.T                                   # y = Pi u, row form
        idx = np.sum(y[:, :, None] > t[None, None, :], axis=2).astype(np.int64)
        x_tilde = n[:, None] * (c[idx] @ Pi)           # n * Pi^T c[idx], row form
        r = x - x_tilde
        gamma = np.sqrt(np.sum(r * r, axis=1))
    z = r @ S.T                                        # S r, row form
    bits = z >= 0.0
    return QuantizedKeys(idx=idx, bits=bits, norm=n, rnorm=gamma, y=y, z=z)


def dequantize_keys(idx, bits, norm, rnorm, rotation, sketch, centroids, w: int):
    """k^ = n Pi^T c[idx] + sqrt(pi/2)/m * gamma * S^T (2 bits - 1)  (float64).

    TurboQuant article §五: the inner-product estimate is
    <y, x~_mse> + ||r|| sqrt(pi/2)/d <S^T signs, y>; with m sketch rows the
    constant is sqrt(pi/2)/m (m == d for TurboQuant keys, m == k for A-QJL).
    For w == 0 the first term is absent and gamma is the key norm.
    """
    S = np.asarray(sketch, dtype=np.float64)
    m = S.shape[0]
    signs = np.where(np.asarray(bits, dtype=bool), 1.0, -1.0)
    qjl = (np.sqrt(np.pi / 2.0) / m) * np.asarray(rnorm, dtype=np.float64)[:, None] * (signs @ S)
    if w == 0:
        return qjl
    Pi = np.asarray(rotation, dtype=np.float64)
    c = np.asarray(centroids, dtype=np.float64)
    mse = np.asarray(norm, dtype=np.float64)[:, None] * (c[np.asarray(idx)] @ Pi)
    return mse + qjl


def index_window(y, boundaries, eps: float = 1e-5):
    """Coordinates within eps of a decision boundary (unit-sphere units)."""
    t = np.asarray(boundaries, dtype=np.float64)
    if t.size == 0:
        return np.zeros_like(np.asarray(y), dtype=bool)
    return np.min(np.abs(np.asarray(y)[..., None] - t), axis=-1) < eps


def sign_window(z, rnorm, eps: float = 1e-5):
    """Sketch rows whose projection is within eps * ||r|| of zero."""
    return np.abs(np.asarray(z)) < eps * np.asarray(rnorm)[:, None]
