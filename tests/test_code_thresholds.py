"""The quantize kernel computes a 2-bit code without a division: with
d = fl32(x - m) and an fp16 scale s, code = [d > 0.5 s] + [d >= 1.5 s] +
[d > 2.5 s] in fp32 (the products are exact). This checks that identity
against the oracle's definition of the code (divide in fp32, round half to
even, clip): exhaustively over fp16 inputs, on exact ties, and for fp32
differences next to every rounding boundary."""
import numpy as np
import pytest

from oracle import ott_oracle as O

F16, F32, F64 = np.float16, np.float32, np.float64


def _thr_of_d(d, s):
    """The kernel's rule on fp32 differences d."""
    s32 = F32(s)
    if not s32 > 0:
        return np.zeros(np.shape(d), np.uint8)
    t1, t2, t3 = F32(0.5) * s32, F32(1.5) * s32, F32(2.5) * s32
    return ((d > t1).astype(np.uint8) + (d >= t2) + (d > t3)).astype(np.uint8)


def codes_by_thresholds(v, lo, s):
    d = np.asarray(v, F16).astype(F32) - F32(lo)
    return _thr_of_d(d, s)


ALL_F16 = np.arange(1 << 16, dtype=np.uint16).view(F16)
ALL_F16 = ALL_F16[np.isfinite(ALL_F16)]


def _pairs(n, seed):
    rng = np.random.default_rng(seed)
    lo = rng.choice(ALL_F16, n)
    s = np.abs(rng.choice(ALL_F16, n))
    # scales of realistic size too: (max - min) / 3 of typical groups
    s[: n // 2] = (rng.uniform(1e-3, 40.0, n // 2)).astype(F16)
    return lo, s


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_thresholds_equal_division_for_every_fp16_input(seed):
    lo, s = _pairs(60, seed)
    for l, sc in zip(lo, s):
        # every finite fp16 value at or above the minimum (members never lie below it)
        v = ALL_F16[ALL_F16.astype(F32) >= F32(l)]
        assert np.array_equal(codes_by_thresholds(v, l, sc), O.codes_of(v, l, sc)), (l, sc)


def test_thresholds_on_exact_ties():
    """Values whose quotient lands exactly on 0.5, 1.5, 2.5 (ties to even) and
    one fp32 ulp either side."""
    for sc in [F16(1.0), F16(0.25), F16(3.0), F16(0.1), F16(7.5), F16(6.1e-5)]:
        for lo in [F16(0.0), F16(-2.0), F16(1.5)]:
            for k in (0.5, 1.5, 2.5):
                x = F16(F32(lo) + F32(k) * F32(sc))
                v = np.array([x, np.nextafter(x, F16(np.inf)), np.nextafter(x, F16(-np.inf))], F16)
                v = v[v.astype(F32) >= F32(lo)]
                assert np.array_equal(codes_by_thresholds(v, lo, sc), O.codes_of(v, lo, sc)), (sc, lo, k)


def _codes_of_d(d, s):
    """The oracle's rounding applied to an fp32 difference d directly."""
    y = d.astype(F32) / F32(s)
    return np.clip(np.rint(y), 0, 3).astype(np.uint8)


def test_thresholds_for_any_fp32_difference():
    """fp32 differences within 64 ulps of every rounding boundary, where the
    fp32 division rounds across or onto the boundary."""
    rng = np.random.default_rng(5)
    scales = np.concatenate([rng.uniform(1e-4, 60.0, 300).astype(F16),
                             np.array([1, 0.25, 3, 0.1, 6.1e-5, 1000], F16)])
    steps = np.arange(-64, 65)
    for sc in scales:
        for k in (0.5, 1.5, 2.5):
            c = F32(F64(sc) * k)
            bits = c.view(np.uint32).astype(np.int64) + steps
            d = bits.astype(np.uint32).view(F32)
            assert np.array_equal(_thr_of_d(d, sc), _codes_of_d(d, sc)), (sc, k)


def test_zero_scale_gives_code_zero():
    v = ALL_F16[:1000]
    assert not codes_by_thresholds(v, F16(0), F16(0)).any()
