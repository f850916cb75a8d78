"""Pins for the oracle's scalar arithmetic: exp/sigmoid, E4M3 and bf16.

None of these checks re-types the oracle's formulas: exp is held to libm's
double exp, E4M3 to a nearest-codebook search and to torch's float8 cast,
bf16 to torch's cast, and all of them to hand-worked cases."""
import numpy as np
import pytest
import torch

import oracle
from checks import bf16_to_f32, bits_from_f32, f32_from_bits, f32_ulp, golden_lines


# ---------------------------------------------------------------- exp ----

def _sweep(lo: float, hi: float, n: int) -> np.ndarray:
    """About n fp32 values covering [lo, hi] by stepping through bit patterns."""
    parts = []
    for a, b in ((0.0, hi), (0.0, -lo)):
        ua, ub = int(bits_from_f32([a])[0]), int(bits_from_f32([b])[0])
        step = max(1, (ub - ua) // (n // 2))
        u = np.arange(ua, ub + 1, step, dtype=np.uint32)
        v = f32_from_bits(u)
        parts.append(v if (a, b) == (0.0, hi) else -v)
    x = np.unique(np.concatenate(parts + [np.float32([lo, hi])]))
    return x[(x >= lo) & (x <= hi)]


# fp32's own range of the exponential, found from the mathematics in double
# precision (not from the oracle): the first fp32 x whose e^x exceeds the
# largest finite float, and the first whose e^x is at least the smallest
# normal float 2^-126.
def _first_f32_above(v: float, strict: bool) -> np.float32:
    f = np.float32(v)
    if float(f) < v or (strict and float(f) == v):
        f = np.nextafter(f, np.float32(np.inf))
    return f


X_OVF = _first_f32_above(np.log(np.float64(np.finfo(np.float32).max)), strict=True)
X_NORM = _first_f32_above(np.log(np.float64(2.0) ** -126), strict=False)


def _edge(x0: np.float32, n: int) -> np.ndarray:
    """The n fp32 values below x0 and x0 with the n - 1 above it."""
    u = int(bits_from_f32([abs(x0)])[0])
    v = f32_from_bits(np.arange(u - n, u + n, dtype=np.uint32))
    return v if x0 > 0 else -v


def test_expf_range_ends_are_fp32s():
    # the whole polynomial path: n = rint(x log2 e) reaches 128 just below
    # the overflow end and -126 at the normal end
    assert float(X_OVF) == 88.72283935546875
    assert float(X_NORM) == -87.33654022216797
    with np.errstate(over="ignore"):
        assert np.float32(np.exp(np.float64(X_OVF))) == np.inf
        assert np.isfinite(np.float32(np.exp(np.float64(np.nextafter(X_OVF, np.float32(0))))))
    assert np.exp(np.float64(X_NORM)) >= 2.0 ** -126
    assert np.exp(np.float64(np.nextafter(X_NORM, np.float32(-np.inf)))) < 2.0 ** -126


def test_expf_within_2ulp_of_double_exp():
    top = np.nextafter(X_OVF, np.float32(0))
    x = np.concatenate([_sweep(float(X_NORM), float(top), 4_000_000),
                        _edge(X_OVF, 1 << 16), _edge(X_NORM, 1 << 16)])
    x = x[(x >= X_NORM) & (x < X_OVF)]
    got = oracle.expf(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    err = np.abs(got - ref) / f32_ulp(ref)
    assert err.max() <= 2.0, (x[np.argmax(err)], err.max())
    assert np.all(got >= 2.0 ** -126) and np.all(np.isfinite(got))   # normal results only
    # dense around 0, where the reduction does nothing
    x = np.linspace(-1, 1, 200_001, dtype=np.float32)
    err = np.abs(oracle.expf(x) - np.exp(x.astype(np.float64))) / f32_ulp(np.exp(x.astype(np.float64)))
    assert err.max() <= 2.0


def test_expf_zero_and_inf_exactly_outside_the_normal_range():
    # +inf exactly where e^x rounds to +inf in fp32; 0 exactly where e^x is
    # below the smallest normal (the stated reading: no subnormal results)
    x = np.concatenate([_sweep(-110.0, 110.0, 400_000), _edge(X_OVF, 4096), _edge(X_NORM, 4096),
                        np.float32([np.inf, -np.inf, 1e30, -1e30])])
    got = oracle.expf(x)
    with np.errstate(over="ignore"):
        ref = np.exp(x.astype(np.float64))
        assert np.array_equal(np.isinf(got), np.float32(ref) == np.inf)
    assert np.array_equal(got == 0.0, ref < 2.0 ** -126)


def test_expf_monotone_and_special_values():
    x = np.sort(np.concatenate([_sweep(-100.0, 100.0, 1_000_000), _edge(X_OVF, 2048), _edge(X_NORM, 2048)]))
    y = oracle.expf(x)
    assert np.all(y[1:] >= y[:-1])   # (+inf >= +inf holds; a difference would be NaN)
    assert oracle.expf(np.float32([0.0]))[0] == 1.0
    assert np.isnan(oracle.expf(np.float32([np.nan]))[0])
    assert oracle.expf(np.float32([-np.inf]))[0] == 0.0 and oracle.expf(np.float32([np.inf]))[0] == np.inf


def test_oracle_cutoffs_equal_the_mathematical_ones():
    assert oracle.lib().orc_expf_hi() == X_OVF
    assert oracle.lib().orc_expf_lo() == X_NORM


def test_sigmoid_range_monotone_and_accuracy():
    x = np.sort(np.concatenate([_sweep(-100.0, 100.0, 1_000_000), _edge(-X_OVF, 4096), _edge(X_NORM, 4096)]))
    s = oracle.sigmoid(x)
    assert np.all(s >= 0) and np.all(s <= 1)
    assert np.all(np.diff(s.astype(np.float64)) >= 0)
    assert oracle.sigmoid(np.float32([0.0]))[0] == 0.5
    # within 3 ulp of the double sigmoid wherever fp32's e^-x is finite,
    # including the subnormal results of 1 / (1 + e^-x) below x = -87.34
    # (an ulp there is 2^-149)
    fin = x > -X_OVF
    ref = 1.0 / (1.0 + np.exp(-x[fin].astype(np.float64)))
    err = np.abs(s[fin] - ref) / f32_ulp(ref)
    assert err.max() <= 3.0, (x[fin][np.argmax(err)], err.max())
    assert np.any(s[fin] < 2.0 ** -126)   # the subnormal results are reached
    # below -88.7228 fp32's e^-x is +inf, and 1 / (1 + inf) is 0
    assert np.all(s[~fin] == 0.0)


# --------------------------------------------------------------- E4M3 ----

def _codebook():
    """All non-negative finite E4M3 codes and their values, from the OFP8
    definition of the format."""
    codes = np.arange(0x7F, dtype=np.int64)     # 0x00..0x7E (0x7F is NaN)
    e, m = codes >> 3, codes & 7
    vals = np.where(e == 0, m * 2.0 ** -9, (8 + m) * 2.0 ** (e - 10.0))
    return codes, vals


def _nearest_code(v: np.ndarray) -> np.ndarray:
    codes, vals = _codebook()
    a = np.abs(v.astype(np.float64))
    hi = np.clip(np.searchsorted(vals, a), 1, len(vals) - 1)
    lo = hi - 1
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(codes[lo] % 2 == 0, lo, hi)))
    c = codes[pick]
    c = np.where(a >= 448.0, 0x7E, c)
    sign = (bits_from_f32(v) >> 31).astype(np.int64)
    return (c | (sign << 7)).astype(np.uint8)


def test_e4m3_golden_cases():
    n = 0
    for line in golden_lines("e4m3_cases.txt"):
        val, code = line.split()[:2]
        v = np.float32(float.fromhex(val))
        assert oracle.e4m3_from_f32(np.float32([v]))[0] == int(code, 16), (val, code)
        n += 1
    assert n >= 20


def test_e4m3_decode_matches_torch():
    c = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f32(c)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("scale", [1.0, 0.5, 3.0, 448.0 / 3.0, 448.0 / 0.7, 17.25, 2.0 ** -5, 1e4])
def test_e4m3_is_nearest_codebook_value_for_all_bf16(scale):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(over="ignore", invalid="ignore"):
        v = bf16_to_f32(b) * np.float32(scale)
    v = v[~np.isnan(v)]
    got = oracle.e4m3_from_f32(v)
    assert np.array_equal(got, _nearest_code(v))


def test_e4m3_matches_torch_cast_in_range():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = f32_from_bits(u)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    v = np.concatenate([v, np.linspace(-448, 448, 100_001, dtype=np.float32)])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_from_f32(v), ref)


# --------------------------------------------------------------- bf16 ----

def test_bf16_golden_cases():
    n = 0
    for line in golden_lines("bf16_cases.txt"):
        src, dst = line.split()[:2]
        v = f32_from_bits([int(src, 16)])
        assert oracle.bf16_from_f32(v)[0] == int(dst, 16), (src, dst)
        n += 1
    assert n >= 10


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = f32_from_bits(u)
    v = v[~np.isnan(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_from_f32(v), ref)
