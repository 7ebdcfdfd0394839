"""Random orthogonal rotation (oracle, float64).

TurboQuant article §二, the normalise-and-rotate step: the rotation matrix is made
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


# ---------------------------------------------------------------- structured

def sylvester_hadamard(d: int) -> np.ndarray:
    """The d x d Hadamard matrix of Sylvester's construction (entries +-1),
    H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]]; d a power of two."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_signs(g: np.ndarray) -> np.ndarray:
    """The random sign flips D of a randomised Hadamard rotation: the signs of
    the first row of the layer's d x d Gaussian draw (+1 for >= 0)."""
    g = np.asarray(g, dtype=np.float64)
    return np.where(g[0] >= 0.0, 1.0, -1.0)


def randomized_hadamard(g: np.ndarray) -> np.ndarray:
    """NexusQuant article, stage 4 (the Hadamard rotation): Pi = H D / sqrt(d),
    an orthogonal rotation that spreads every coordinate's energy over all d
    (float64)."""
    s = hadamard_signs(g)
    d = s.shape[0]
    return sylvester_hadamard(d) * s[None, :] / np.sqrt(d)


def randomized_hadamard_fp32(g: np.ndarray) -> np.ndarray:
    """The randomised Hadamard rotation as stored and handed to both sides (fp32, y = Pi x)."""
    return randomized_hadamard(g).astype(np.float32)


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis (float64):
    log2(d) stages of butterflies (a + b, a - b) on pairs 2^s apart."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a + b, a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y
