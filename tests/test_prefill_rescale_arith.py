"""CPU checks of the fp32 arithmetic behind the prefill kernel's conversion-free
W-group rescale (32-key groups): every step is replayed in exact rational
arithmetic with IEEE single rounding, on random and extreme operands.

The kernel starts each PV MFMA's int32 accumulator at the bit pattern of
M = 1.5 * 2^23 and reads the result as fp32, cuts sW to 22 significant bits,
and folds the two groups of a 64-key tile into O as
    t = fma(sW1, x1, fma(sW0, x0, -S)),  S = fl(P0 + P1),  P_g = M * sW_g,
keeping the residual d = P0 + P1 - S (Fast2Sum) per row.  The claims:
  * bits(0x4B400000 + acc) read as fp32 is exactly M + acc for every
    |acc| <= 32 * 127^2;
  * M * sW_g is exact once sW_g has 22 significant bits;
  * d is exact, so t - d = sW0 acc0 + sW1 acc1 up to the roundings of the
    two fmas, which are bounded by half an ulp of |P1| plus half an ulp of
    the true result.
"""
from fractions import Fraction

import numpy as np

M = 12582912.0
ACC_MAX = 32 * 127 * 127


def f32(x):
    return np.float32(x)


def round_f32(q: Fraction) -> np.float32:
    """Exact rational -> nearest fp32, ties to even (normal range)."""
    a = np.float32(float(q))          # within one fp32 ulp of q
    lo, hi = a, a
    while Fraction(float(lo)) > q:
        lo = np.nextafter(lo, np.float32(-np.inf))
    while Fraction(float(hi)) < q:
        hi = np.nextafter(hi, np.float32(np.inf))
    if lo == hi:
        return lo
    dl, dh = q - Fraction(float(lo)), Fraction(float(hi)) - q
    if dl != dh:
        return lo if dl < dh else hi
    return lo if (lo.view(np.uint32) & 1) == 0 else hi


def fma32(a, b, c) -> np.float32:
    return round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def cut22(x: np.float32) -> np.float32:
    return (np.asarray(x, np.float32).view(np.uint32) & np.uint32(0xFFFFFFFC)).view(np.float32)


def ulp(x: float) -> Fraction:
    x = np.float32(abs(x))
    return Fraction(float(np.nextafter(x, np.float32(np.inf)))) - Fraction(float(x))


def test_bias_bits_read_as_float_are_exact():
    accs = np.array([0, 1, -1, 2, -2, 12345, -54321, ACC_MAX, -ACC_MAX, 2**21, -(2**21)],
                    np.int64)
    rng = np.random.default_rng(1)
    accs = np.concatenate([accs, rng.integers(-ACC_MAX, ACC_MAX + 1, 2000)])
    bits = (np.int64(0x4B400000) + accs).astype(np.uint32)
    vals = bits.view(np.float32).astype(np.float64)
    assert np.array_equal(vals, M + accs.astype(np.float64))


def test_magic_times_cut_scale_is_exact():
    rng = np.random.default_rng(2)
    sw = np.concatenate([
        rng.uniform(1e-9, 1.0, 3000).astype(np.float32),
        (rng.uniform(0, 1, 200) * 2.0 ** rng.integers(-120, 20, 200)).astype(np.float32),
        np.array([0.0, np.finfo(np.float32).tiny, 1.0, 0.99999994], np.float32)])
    for s in sw:
        c = cut22(s)
        assert abs(Fraction(float(c)) - Fraction(float(s))) <= Fraction(float(s)) / 2**21
        p = f32(np.float32(M) * c)
        assert Fraction(float(p)) == Fraction(M) * Fraction(float(c)), (s, c, p)


def test_fold_of_two_groups():
    rng = np.random.default_rng(3)
    worst = Fraction(0)
    for trial in range(3000):
        # scales of the two groups of one row: W max / 127 with p~ <= 2^8
        # and V scales ~ 3/127, sometimes an empty (zero) group
        sw = [cut22(f32(rng.uniform(0, 256) * rng.uniform(0.5, 8) / 127 / 127)) for _ in range(2)]
        if trial % 7 == 0:
            sw[1] = np.float32(0.0)
        if trial % 11 == 0:
            sw[0] = np.float32(0.0)
        acc = [int(rng.integers(-ACC_MAX, ACC_MAX + 1)) for _ in range(2)]
        x = [np.uint32(0x4B400000 + a).view(np.float32) for a in acc]
        p0, p1 = f32(np.float32(M) * sw[0]), f32(np.float32(M) * sw[1])
        ph, pl = max(p0, p1), min(p0, p1)
        S = f32(ph + pl)
        d = f32(pl - f32(S - ph))
        # Fast2Sum: d is the exact rounding error of S
        assert Fraction(float(S)) + Fraction(float(d)) == Fraction(float(p0)) + Fraction(float(p1))
        t = fma32(sw[1], x[1], fma32(sw[0], x[0], -S))
        exact = Fraction(float(sw[0])) * acc[0] + Fraction(float(sw[1])) * acc[1]
        err = abs(Fraction(float(t)) - Fraction(float(d)) - exact)
        inner = Fraction(float(sw[0])) * acc[0] - Fraction(float(p1)) + Fraction(float(d))
        bound = ulp(float(inner)) / 2 + ulp(float(exact + Fraction(float(d)))) / 2
        assert err <= bound, (trial, sw, acc, float(err), float(bound))
        # in units of the larger group scale the error stays at about one
        # unit of a single Wq * Vq product
        smax = max(Fraction(float(sw[0])), Fraction(float(sw[1])))
        if smax > 0:
            worst = max(worst, err / smax)
    assert worst <= 1, float(worst)


def test_planted_mistakes_are_caught():
    """The same checks fail for an uncut scale (inexact M * sW) and for a
    bias outside the binade."""
    s = np.float32(0.1234567)
    assert (np.asarray(s).view(np.uint32) & 3) != 0
    p = f32(np.float32(M) * s)
    assert Fraction(float(p)) != Fraction(M) * Fraction(float(s))
    acc = 2**22 + 5                                  # beyond what the binade holds
    v = np.uint32(0x4B400000 + acc).view(np.float32)
    assert float(v) != M + acc
