"""Pins of the oracle's half side-information reading (oracle.layout.stored_side,
row_bytes with side_f16) against what IEEE 754 and arithmetic fix:

* the nearest-half rounding is checked by brute force over the whole grid of
  finite halves (nearest by distance, a tie going to the even significand),
  on every midpoint between neighbouring halves (exactly representable in
  fp32, so every tie of the format is exercised) and on fp32 numbers drawn
  over the whole exponent range, with the saturation of the reading past
  65504;
* the layout: at head_dim 256, 3-bit keys and 2-bit values a token of one KV
  head takes 232 bytes with fp32 side information, which is the TurboQuant
  article's 4.41x against bf16 K and V (§一, Paper Validation table), and
  196 bytes with halves: 1024 / 196 = 5.22x.
"""
import json
import os

import numpy as np

from oracle import layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# every finite non-negative half, ascending: codes 0x0000 .. 0x7BFF
GRID_CODES = np.arange(0x7C00, dtype=np.uint16)
GRID = GRID_CODES.view(np.float16).astype(np.float64)


def _nearest_half_by_search(x):
    """The nearest finite half to each float x by search over GRID (ties to the
    even code, i.e. even significand), saturating past the largest half."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    i = np.clip(np.searchsorted(GRID, a), 1, GRID.size - 1)
    lo, hi = GRID[i - 1], GRID[i]
    take_hi = (hi - a < a - lo) | ((hi - a == a - lo) & (GRID_CODES[i] % 2 == 0))
    r = np.where(take_hi, hi, lo)
    r = np.where(a >= GRID[-1], GRID[-1], r)
    return np.copysign(r, x)


def test_grid_is_the_half_format():
    assert GRID[0] == 0.0 and GRID[1] == 2.0 ** -24            # smallest subnormal
    assert GRID[0x0400] == 2.0 ** -14                           # smallest normal
    assert GRID[-1] == layout.HALF_MAX == (2 - 2 ** -10) * 2 ** 15
    assert np.all(np.diff(GRID) > 0)


def test_every_midpoint_ties_to_even():
    mid = (GRID[:-1] + GRID[1:]) / 2
    assert np.all(mid.astype(np.float32).astype(np.float64) == mid)   # exact in fp32
    for sign in (1.0, -1.0):
        got = layout.stored_side(sign * mid, True).astype(np.float64)
        np.testing.assert_array_equal(got, _nearest_half_by_search(sign * mid))
    # spot values: 1 + 2^-11 sits halfway between 1 and 1 + 2^-10 -> 1 (even);
    # 1 + 3 * 2^-11 halfway between 1 + 2^-10 and 1 + 2^-9 -> 1 + 2^-9 (even)
    assert float(layout.stored_side(1 + 2.0 ** -11, True)) == 1.0
    assert float(layout.stored_side(1 + 3 * 2.0 ** -11, True)) == 1 + 2.0 ** -9
    assert float(layout.stored_side(2.0 ** -25, True)) == 0.0                 # tie with 0 -> 0
    assert float(layout.stored_side(3 * 2.0 ** -25, True)) == 2.0 ** -23      # tie -> even code 2


def test_random_fp32_over_every_exponent():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 0x7F800000, size=400_000, dtype=np.int64).astype(np.uint32)
    x = bits.view(np.float32).astype(np.float64)
    x = np.concatenate([x, -x, rng.standard_normal(100_000) * 10.0 ** rng.uniform(-9, 7, 100_000)])
    x32 = x.astype(np.float32).astype(np.float64)
    got = layout.stored_side(x32, True)
    assert got.dtype == np.float16
    np.testing.assert_array_equal(got.astype(np.float64), _nearest_half_by_search(x32))


def test_saturation_and_specials():
    s = lambda v: float(layout.stored_side(np.float32(v), True))
    assert s(65504.0) == 65504.0
    assert s(65519.0) == 65504.0           # nearer to 65504 than to 2^16
    assert s(65520.0) == 65504.0           # would round to infinity: saturates
    assert s(1e30) == 65504.0 and s(-1e30) == -65504.0
    assert s(np.inf) == np.inf and s(-np.inf) == -np.inf
    assert np.isnan(s(np.nan))
    assert s(-0.0) == 0.0 and np.signbit(s(-0.0))
    # without the option the stored number is the fp32 one
    x = np.array([1 + 2.0 ** -20, 1e30], np.float64)
    assert layout.stored_side(x, False).dtype == np.float32
    np.testing.assert_array_equal(layout.stored_side(x, False), x.astype(np.float32))


def test_half_side_layout_is_5_22x_at_head_dim_256():
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["turboquant_compression_ratio_d256"]
    bf16_kv = 2 * 2 * 256                  # K and V of one token, bf16
    full = sum(layout.row_bytes(256, w=2, m=256).values())
    half = sum(layout.row_bytes(256, w=2, m=256, side_f16=True).values())
    assert full == 232 and round(bf16_kv / full, 2) == fig["value"] == 4.41
    # codes and signs unchanged; 2 norms + 8 scales + 8 minima at 2 bytes instead of 4
    assert full - half == 2 * (2 + 2 * 256 // 32)
    assert half == 196 and round(bf16_kv / half, 2) == 5.22
    for name in ("key_codes", "key_signs", "val_codes"):
        assert layout.row_bytes(256, 2, 256)[name] == layout.row_bytes(256, 2, 256, side_f16=True)[name]
