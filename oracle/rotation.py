"""Random orthogonal rotation (oracle, float64).

TurboQuant article §二, step "归一化 + 随机旋转": the rotation matrix is made
by a QR decomposition of a random matrix (one fixed seed per layer; §六 gives
seed = 42 + 7 * layer).  The article does not say how the signs of the QR
factors are fixed; here the columns of Q are multiplied by sign(diag R), which
makes the result Haar-distributed (Mezzadri 2007), and the rotation acts as
y = Pi @ x.

The Gaussian matrix itself is an input (drawn by the seeded input module).
"""
from __future__ import annotations

import numpy as np


def rotation_from_gaussian(g: np.ndarray) -> np.ndarray:
    """Haar orthogonal matrix Q * diag(sign(diag R)) from G = Q R (float64)."""
    g = np.asarray(g, dtype=np.float64)
    q, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return q * s[None, :]


def rotation_fp32(g: np.ndarray) -> np.ndarray:
    """The rotation as stored and handed to both sides (fp32, row-major, y = Pi x)."""
    return rotation_from_gaussian(g).astype(np.float32)
