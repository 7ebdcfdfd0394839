"""Bit layouts of the compressed cache rows (oracle).

TurboQuant article §二 says the d sign bits of the QJL sketch are packed into
d/8 bytes, and §五 that quantize() returns four bit-packed things per key
(MSE indices, QJL sign bytes, residual norm, original norm); the value codes
are bit-packed too (§七, kv_cache.py).  The bit order is not given.  The
reading used on both sides (chosen so a decoder turns 4 bits into 4 operand
bytes with one shift and one mask, and gets one value code per token of a
32-token block from one 32-bit word):

* bit rows (key signs, and each key index plane): 32-bit little-endian words
  of 32 consecutive elements; element j = 4 i + k of a word (i in 0..7,
  k in 0..3) is bit 8 k + i, i.e. byte k holds the elements with j % 4 == k;
* key codes, one row of w*d/8 bytes per token: w such bit rows one after the
  other, plane p holding bit p of every coordinate's index;
* key signs, one row of m/8 bytes per token, bit 1 = non-negative projection;
* value codes, in blocks of 32 tokens (32 * d * vb / 8 bytes per block): for
  channel group g (32 channels), column n (0..15), half h (0..1) -- channel
  32 g + 16 h + n -- and token T = 4 i + r of the block (r in 0..3, i in 0..7):
    vb = 2: 32-bit word (16 g + n) * 4 + r, bit 8 h + 16 (i & 1) + 2 (i >> 1);
    vb = 4: 32-bit word ((16 g + n) * 4 + r) * 2 + h, bit 16 (i & 1) + 4 (i >> 1);
* norms, value scales and value minima are fp32, one row per token; with the
  half side-information option (the bytes-for-precision knob beside the
  head_dim 256 compression figure of §一's Paper Validation table) they are
  IEEE halves instead, see stored_side.
"""
from __future__ import annotations

import numpy as np


def pack_bits(bits: np.ndarray) -> np.ndarray:
    """[N, k] booleans (k % 32 == 0) -> [N, k/8] uint8 in the word layout above."""
    bits = np.asarray(bits, dtype=bool)
    n, k = bits.shape[:-1], bits.shape[-1]
    assert k % 32 == 0
    w = bits.reshape(n + (k // 32, 8, 4))          # [.., word, i, k]
    w = np.swapaxes(w, -1, -2)                     # [.., word, k, i]
    by = np.packbits(w, axis=-1, bitorder="little")[..., 0]   # byte k: bit i = element 4 i + k
    return by.reshape(n + (k // 8,))


def unpack_bits(packed: np.ndarray, k: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[:-1]
    by = packed.reshape(n + (k // 32, 4, 1))
    w = np.unpackbits(by, axis=-1, count=8, bitorder="little").astype(bool)   # [.., word, k, i]
    return np.swapaxes(w, -1, -2).reshape(n + (k,))


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


def _value_bit_positions(d: int, vb: int):
    """(word index, bit offset) of every (token-in-block, channel) pair: two [32, d] arrays."""
    t = np.arange(32)[:, None]
    ch = np.arange(d)[None, :]
    g, rem = ch // 32, ch % 32
    h, n = rem // 16, rem % 16
    i, r = t // 4, t % 4
    if vb == 2:
        word = (16 * g + n) * 4 + r
        bit = 8 * h + 16 * (i & 1) + 2 * (i >> 1)
    elif vb == 4:
        word = ((16 * g + n) * 4 + r) * 2 + h
        bit = 16 * (i & 1) + 4 * (i >> 1)
    else:
        raise ValueError("value bits must be 2 or 4")
    return np.broadcast_to(word, (32, d)), np.broadcast_to(bit, (32, d))


def pack_value_codes(codes: np.ndarray, vb: int) -> np.ndarray:
    """[T, d] codes in [0, 2**vb) -> [ceil(T/32) * 32, d*vb/8] uint8 rows of 32-token blocks
    (tokens past T are zero)."""
    codes = np.asarray(codes, dtype=np.int64)
    T, d = codes.shape
    nblk = (T + 31) // 32
    padded = np.zeros((nblk * 32, d), dtype=np.int64)
    padded[:T] = codes
    word, bit = _value_bit_positions(d, vb)
    words = np.zeros((nblk, 32 * d * vb // 32), dtype=np.uint64)
    blk = padded.reshape(nblk, 32, d)
    vals = blk.astype(np.uint64) << bit.astype(np.uint64)[None]
    for b in range(nblk):
        np.bitwise_or.at(words[b], word.reshape(-1), vals[b].reshape(-1))
    out = words.astype("<u4").view(np.uint8).reshape(nblk * 32, d * vb // 8)
    return out


def unpack_value_codes(rows: np.ndarray, T: int, d: int, vb: int) -> np.ndarray:
    """Inverse of pack_value_codes for the first T tokens."""
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.uint8))
    nblk = (T + 31) // 32
    words = rows[: nblk * 32].reshape(nblk, -1).view("<u4").astype(np.int64)
    word, bit = _value_bit_positions(d, vb)
    codes = (words[:, word] >> bit[None]) & ((1 << vb) - 1)
    return codes.reshape(nblk * 32, d)[:T]


def row_bytes(d: int, w: int, m: int, vb: int = 2, group: int = 32, side_f16: bool = False) -> dict:
    """Bytes one token of one KV head occupies in each cache plane (side
    information 4 bytes a number, 2 with the half option)."""
    e = 2 if side_f16 else 4
    return {
        "key_codes": w * d // 8,
        "key_signs": m // 8,
        "key_norm": e,
        "key_rnorm": e if w > 0 else 0,
        "val_codes": d * vb // 8,
        "val_scale": e * (d // group),
        "val_min": e * (d // group),
    }


HALF_MAX = 65504.0   # largest finite IEEE half: (2 - 2^-10) * 2^15


def stored_side(x, side_f16: bool = False) -> np.ndarray:
    """What the cache holds for side information x (the key norm and residual
    norm that §五's quantize() keeps beside the bits, the value scale and
    minimum of §七): the fp32 value; with the half option, that fp32 value
    rounded to the nearest IEEE half, ties to the even significand, a finite
    value past the half range saturating to +-HALF_MAX (a reading: the pages
    give no half format; saturation keeps every stored number finite).
    Returned in the stored type (float32 or float16).

    The codes (indices, sign bits, value codes) never depend on this rounding:
    they are decided from the unrounded numbers on both sides."""
    x32 = np.asarray(x, dtype=np.float32)
    if not side_f16:
        return x32
    big = (np.abs(x32) > np.float32(HALF_MAX)) & np.isfinite(x32)
    x32 = np.where(big, np.copysign(np.float32(HALF_MAX), x32), x32)
    return x32.astype(np.float16)
