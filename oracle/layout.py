"""Bit layouts of the compressed cache rows (oracle).

TurboQuant article §二 says the d sign bits of the QJL sketch are packed into
d/8 bytes, and §五 that quantize() returns four bit-packed things per key
(MSE indices, QJL sign bytes, residual norm, original norm); the value codes
are bit-packed too (§七, kv_cache.py).  The exact bit order is not given;
the reading used on both sides is:

* key codes, one row of w*d/8 bytes per token: w bit-planes one after the
  other, plane p holding bit p of every coordinate's index; inside a plane,
  coordinate j is bit (j % 8) of byte j // 8 (LSB first);
* key signs, one row of m/8 bytes per token, sketch row i at bit (i % 8)
  of byte i // 8, bit = 1 for a non-negative projection;
* value codes, one row of d*vb/8 bytes per token, LSB-first bitstream:
  channel j occupies bits [vb*j, vb*j + vb) of the little-endian row;
* norms, value scales and value minima are fp32.
"""
from __future__ import annotations

import numpy as np


def pack_bits(bits: np.ndarray) -> np.ndarray:
    """[N, k] booleans -> [N, k/8] uint8, element i at bit i%8 of byte i//8."""
    bits = np.asarray(bits, dtype=bool)
    assert bits.shape[-1] % 8 == 0
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack_bits(packed: np.ndarray, k: int) -> np.ndarray:
    return np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=-1, count=k,
                         bitorder="little").astype(bool)


def pack_code_planes(idx: np.ndarray, w: int) -> np.ndarray:
    """[N, d] integer indices in [0, 2**w) -> [N, w*d/8] uint8 (plane-major)."""
    idx = np.asarray(idx, dtype=np.int64)
    if w == 0:
        return np.zeros(idx.shape[:-1] + (0,), dtype=np.uint8)
    planes = [pack_bits((idx >> p) & 1) for p in range(w)]
    return np.concatenate(planes, axis=-1)


def unpack_code_planes(rows: np.ndarray, d: int, w: int) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.uint8)
    nb = d // 8
    idx = np.zeros(rows.shape[:-1] + (d,), dtype=np.int64)
    for p in range(w):
        idx |= unpack_bits(rows[..., p * nb:(p + 1) * nb], d).astype(np.int64) << p
    return idx


def pack_value_codes(codes: np.ndarray, vb: int) -> np.ndarray:
    """[N, d] codes in [0, 2**vb) -> [N, d*vb/8] uint8, LSB-first bitstream."""
    codes = np.asarray(codes, dtype=np.int64)
    n, d = codes.shape[:-1], codes.shape[-1]
    bits = np.zeros(n + (d * vb,), dtype=bool)
    for b in range(vb):
        bits[..., b::vb] = (codes >> b) & 1
    return pack_bits(bits)


def unpack_value_codes(rows: np.ndarray, d: int, vb: int) -> np.ndarray:
    bits = unpack_bits(rows, d * vb).astype(np.int64)
    codes = np.zeros(bits.shape[:-1] + (d,), dtype=np.int64)
    for b in range(vb):
        codes |= bits[..., b::vb] << b
    return codes


def row_bytes(d: int, w: int, m: int, vb: int = 2, group: int = 32) -> dict:
    """Bytes one token of one KV head occupies in each cache plane."""
    return {
        "key_codes": w * d // 8,
        "key_signs": m // 8,
        "key_norm": 4,
        "key_rnorm": 4 if w > 0 else 0,
        "val_codes": d * vb // 8,
        "val_scale": 4 * (d // group),
        "val_min": 4 * (d // group),
    }
