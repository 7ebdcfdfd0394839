"""The value kernel forms scale = fl((max - min) / L), L = 2^vb - 1, without a
divide: q0 = x * fl(1/L), r = fma(-q0, L, x), q = fma(r, fl(1/L), q0).  This
checks, in exact integer arithmetic, that q equals the correctly rounded
quotient for every fp32 significand (x in [1, 2)); a power-of-two exponent
carries over unchanged while every step stays a normal number, which the kernel
ensures by taking the IEEE divide for x outside [1e-28, 1e28]."""
import numpy as np
import pytest


def _bitlen(p):
    # exact for 0 < p < 2^53
    return np.frexp(p.astype(np.float64))[1].astype(np.int64)


def _round24(p, e):
    """Round the positive integers p * 2^e to 24 significant bits, ties to even:
    (significand in [2^23, 2^24), exponent)."""
    shift = _bitlen(p) - 24
    assert shift.min() >= 1
    q = p >> shift
    rem = p & ((np.int64(1) << shift) - 1)
    half = np.int64(1) << (shift - 1)
    q = q + ((rem > half) | ((rem == half) & (q & 1 == 1))).astype(np.int64)
    carry = q == (1 << 24)
    q = np.where(carry, q >> 1, q)
    return q, e + shift + carry.astype(np.int64)


def _split(f):
    m, e = np.frexp(np.float64(f))
    return np.int64(m * 2.0**24), np.int64(e - 24)


@pytest.mark.parametrize("levels", [3, 15])
def test_constant_divide_is_correctly_rounded(levels):
    Z, ez = _split(np.float32(1.0) / np.float32(levels))          # fl(1/L) = Z 2^ez
    for lo in range(1 << 23, 1 << 24, 1 << 21):
        X = np.arange(lo, lo + (1 << 21), dtype=np.int64)          # x = X 2^-23
        # q0 = RN(x z)
        Q0, e0 = _round24(X * Z, np.full_like(X, ez - 23))
        # r = x - L q0, exact; it must be an fp32 value for the fma residual to be exact
        E = np.minimum(-23, e0)
        R = (X << (-23 - E)) - levels * (Q0 << (e0 - E))
        assert np.all(np.abs(R) < (1 << 24))
        # q = RN(q0 + r z)
        F = np.minimum(e0, E + ez)
        S = (Q0 << (e0 - F)) + R * Z * (np.int64(1) << (E + ez - F))
        assert S.min() > 0 and S.max() < (1 << 53)
        Q, eq = _round24(S, F)
        # correctly rounded x / L: X 2^26 / L = N + rem / L, rounded with the remainder
        N, rem = np.divmod(X << 26, levels)
        shift = _bitlen(N) - 24
        Qr = N >> shift
        low = (N & ((np.int64(1) << shift) - 1)) * levels + rem     # discarded part, times L
        half = (np.int64(1) << (shift - 1)) * levels
        Qr = Qr + ((low > half) | ((low == half) & (Qr & 1 == 1))).astype(np.int64)
        er = shift - 23 - 26
        carry = Qr == (1 << 24)
        Qr = np.where(carry, Qr >> 1, Qr)
        er = er + carry.astype(np.int64)
        np.testing.assert_array_equal(Q, Qr)
        np.testing.assert_array_equal(eq, er)


def test_model_matches_float32_on_samples():
    # the integer model above agrees with numpy's own fp32 arithmetic where no fma is needed
    rng = np.random.default_rng(5)
    x = (1.0 + rng.random(1000)).astype(np.float32)
    for levels in (3, 15):
        ref = x / np.float32(levels)
        X = (x.astype(np.float64) * 2.0**23).astype(np.int64)
        N, rem = np.divmod(X << 26, levels)
        assert np.all(np.abs(N * 2.0**-49 - ref.astype(np.float64)) <= ref.astype(np.float64) * 2.0**-23)
