"""Value quantisation (oracle).

TurboQuant article, component table (the value row: grouped conventional
min-max at 2 bits per dimension) and §七 (kv_cache.py: value group
quantisation and bit packing).
The article fixes only "min-max", "group" and the bit width.  Reading used on
both sides:

* a group is `group` (32) contiguous channels of one token;
* zero point = group minimum, scale = (max - min) / (2**vb - 1);
* code = clamp(round_half_even((v - min) / scale), 0, 2**vb - 1), and
  code = 0 when scale == 0;
* the code decision is made in IEEE fp32 (subtract, divide, round), the
  precision the stored scale and minimum have; it is emulated here with
  numpy float32 arithmetic, which is IEEE round-to-nearest-even per operation;
* dequantisation: v^ = code * scale + min, evaluated in float64 from the
  stored scale and min (fp32, or their halves with the half side-information
  option, layout.stored_side; the codes are decided from the fp32 numbers
  either way).
"""
from __future__ import annotations

import numpy as np


def quantize_values(v, vb: int = 2, group: int = 32):
    """v [N, d] float32 -> (codes [N, d] int64, scale [N, d/group] f32, vmin [N, d/group] f32)."""
    v = np.asarray(v, dtype=np.float32)
    N, d = v.shape
    assert d % group == 0
    g = v.reshape(N, d // group, group)
    vmin = g.min(axis=2)
    vmax = g.max(axis=2)
    levels = np.float32((1 << vb) - 1)
    scale = (vmax - vmin) / levels                       # fp32 subtract, fp32 divide
    diff = g - vmin[:, :, None]                          # fp32 subtract
    with np.errstate(divide="ignore", invalid="ignore"):
        t = diff / scale[:, :, None]                     # fp32 divide
    code = np.rint(t)                                    # half to even
    code = np.where(scale[:, :, None] > 0, code, 0.0)
    code = np.clip(code, 0, (1 << vb) - 1).astype(np.int64)
    return code.reshape(N, d), scale.astype(np.float32), vmin.astype(np.float32)


def dequantize_values(codes, scale, vmin, group: int = 32):
    codes = np.asarray(codes, dtype=np.float64)
    N, d = codes.shape
    s = np.repeat(np.asarray(scale, dtype=np.float64), group, axis=1)
    mn = np.repeat(np.asarray(vmin, dtype=np.float64), group, axis=1)
    return codes * s + mn


def code_window(v, scale, vmin, group: int = 32, eps: float = 1e-5):
    """Elements whose (v - min) / scale lies within eps of a rounding midpoint
    (in code units, float64)."""
    v = np.asarray(v, dtype=np.float64)
    N, d = v.shape
    s = np.repeat(np.asarray(scale, dtype=np.float64), group, axis=1)
    mn = np.repeat(np.asarray(vmin, dtype=np.float64), group, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s > 0, (v - mn) / s, 0.0)
    frac = t - np.floor(t)
    return np.abs(frac - 0.5) < eps
