"""Pins for the oracle's format codecs.

Expected values come from outside the oracle: torch's own casts (library
routines), brute-force nearest-code search over every code point, exact
rational arithmetic, and the formats' published definitions.
"""
import numpy as np
import pytest
import torch

from tests import ref_exact as R

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FINITE_BF16 = ALL_BF16[((ALL_BF16 >> 7) & 0xFF) != 0xFF]


def _bf16_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------- bf16 --
def test_bf16_decode_every_pattern(orc):
    for b in FINITE_BF16[::7]:
        assert orc.lib().oracle_bf16_to_double(int(b)) == float(R.bf16_value(int(b)))
    assert np.isinf(orc.lib().oracle_bf16_to_double(0x7F80))
    assert np.isnan(orc.lib().oracle_bf16_to_double(0x7FC1))


def test_bf16_encode_matches_torch_on_fp32_patterns(orc):
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    # include every bf16 midpoint pattern and its fp32 neighbours
    mids = ((FINITE_BF16.astype(np.uint32) << 16) | 0x8000)
    extra = np.concatenate([mids, mids + 1, mids - 1]).view(np.float32)
    f = np.concatenate([f, extra[np.isfinite(extra)], np.float32([0.0, -0.0, 3.3895314e38, 1e-45])])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_from_double(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_encode_doubles_by_nearest_search(orc):
    """Doubles that are not fp32 values: just off bf16 midpoints, so a wrong
    tie rule or an intermediate fp32 rounding would show."""
    rng = np.random.default_rng(12)
    base = FINITE_BF16[(FINITE_BF16 & 0x7FFF) < 0x7F7F]
    base = base[rng.integers(0, base.size, 3000)]
    vals = []
    for b in base:
        lo = R.bf16_value(int(b))
        hi = R.bf16_value(int(b) + 1)          # next code up in magnitude
        mid = (lo + hi) / 2
        for d in (0, 2 ** -40, -(2 ** -40), 2 ** -60):
            v = float(mid * (1 + R.F(d)))
            vals.append(v)
    vals = np.array(vals)
    got = orc.bf16_from_double(vals)
    for v, g in zip(vals, got):
        assert g == R.bf16_round(R.F(v), negative_zero=bool(np.signbit(v))), v


def test_bf16_overflow_and_signed_zero(orc):
    assert orc.lib().oracle_bf16_from_double(3.4e38) == 0x7F80           # past the last midpoint
    assert orc.lib().oracle_bf16_from_double(3.3895313892515355e38) == 0x7F7F
    assert orc.lib().oracle_bf16_from_double(-0.0) == 0x8000
    assert orc.lib().oracle_bf16_from_double(1 + 2 ** -8) == 0x3F80      # tie to even
    assert orc.lib().oracle_bf16_from_double(1 + 3 * 2 ** -8) == 0x3F82
    assert orc.lib().oracle_bf16_from_double(2.0 ** -134) == 0x0000      # half the least subnormal: tie to 0
    assert orc.lib().oracle_bf16_from_double(3 * 2.0 ** -134) == 0x0002


# ------------------------------------------------------------------- e4m3fn --
def test_e4m3fn_decode_matches_torch(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3fn_table()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], want[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def _brute_e4m3(v):
    """Nearest finite e4m3fn magnitude by exhaustive search, ties to even code.
    Exact in double for |v| in [2^-12, 2^9]: both operands have all their bits
    inside a 28-bit window there."""
    mags = np.array([float(m) for m in R.E4M3_MAG])
    a = np.abs(v)
    d = np.abs(a[:, None] - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    ties = d == best
    idx = np.where(ties.sum(axis=1) > 1, np.argmax(ties & (np.arange(127) % 2 == 0)[None, :], axis=1),
                   np.argmin(d, axis=1))
    return (idx | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -7, 1.0 / 448, 3.0, 0.75])
def test_e4m3fn_encode_every_bf16_by_brute_force(orc, scale):
    v = _bf16_f64(FINITE_BF16) * scale
    inside = (np.abs(v) >= 2.0 ** -12) & (np.abs(v) <= 2.0 ** 9)
    got = orc.e4m3fn_encode(v)
    assert np.array_equal(got[inside], _brute_e4m3(v[inside]))
    small = np.abs(v) < 2.0 ** -12
    assert np.all((got[small] & 0x7F) == 0)
    big = np.abs(v) > 2.0 ** 9
    assert np.all((got[big] & 0x7F) == 0x7E)                         # saturation
    assert np.array_equal(got >> 7, np.signbit(v).astype(np.uint8))  # sign kept, also for -0 / underflow


def test_e4m3fn_encode_matches_torch_inside_range(orc):
    rng = np.random.default_rng(13)
    f = np.concatenate([rng.standard_normal(200_000) * 50, rng.standard_normal(50_000) * 2 ** -8,
                        np.array([2.625, 2.875, 448.0, 460.0, 2 ** -10, 3 * 2 ** -10, -2 ** -11])])
    f = f.astype(np.float32)
    f = f[np.abs(f) <= 448]
    want = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3fn_encode(f.astype(np.float64)), want)


def test_e4m3fn_hand_values(orc):
    cases = {2.625: 0x42, 2.875: 0x44, 2 ** -10: 0x00, 3 * 2 ** -10: 0x02, -(2 ** -11): 0x80,
             448.0: 0x7E, 460.0: 0x7E, 470.0: 0x7E, 384.0: 0x7C, 224.0: 0x76, 128.0: 0x70, 64.0: 0x68,
             56.0: 0x66, 1.75: 0x3E, 8.0: 0x50, -128.0: 0xF0, 1e30: 0x7E}
    for v, c in cases.items():
        assert orc.lib().oracle_e4m3fn_encode(v) == c, v


def test_e4m3fn_encode_arbitrary_doubles_exact(orc):
    """Quotients yb/s are arbitrary doubles: check against exact rationals."""
    rng = np.random.default_rng(14)
    v = rng.standard_normal(3000) * rng.choice([1e-3, 1, 30, 300], 3000)
    got = orc.e4m3fn_encode(v)
    for x, g in zip(v, got):
        want = R.nearest_code(abs(R.F(x)), R.E4M3_MAG) | (0x80 if x < 0 else 0)
        assert g == want, x


# --------------------------------------------------------------------- e2m1 --
def test_e2m1_decode_table(orc):
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(orc.e2m1_table()) == mags + [-m for m in mags]


def test_e2m1_ties_and_saturation(orc):
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 7.0: 7, 100.0: 7,
             0.2: 0, 0.3: 1, 5.01: 7, -0.1: 8, -5.5: 0xF, 4.99: 6}
    for v, c in cases.items():
        assert orc.lib().oracle_e2m1_encode(v) == c, v


def test_e2m1_encode_by_brute_force(orc):
    rng = np.random.default_rng(15)
    v = np.concatenate([rng.uniform(-8, 8, 20000), np.arange(-32, 33) / 4.0])
    got = orc.e2m1_encode(v)
    for x, g in zip(v, got):
        want = R.nearest_code(abs(R.F(x)), R.E2M1_MAG) | (0x8 if np.signbit(x) else 0)
        assert g == want, x


# ---------------------------------------------------------------------- e8m0 --
def test_mx_scale_exponent_definition(orc):
    pos = FINITE_BF16[(FINITE_BF16 < 0x7F80) & (FINITE_BF16 > 0)]
    for b in pos[::3]:
        amax = R.bf16_value(int(b))
        e = orc.mx_scale_exponent(float(amax))
        if -127 < e < 127:
            assert R.F(2) ** (e + 2) <= amax < R.F(2) ** (e + 3)
        elif e == -127:
            assert amax < R.F(2) ** (-127 + 3)
        else:
            assert amax >= R.F(2) ** (127 + 2)


# -------------------------------------------------------------- fp32 scale --
def test_fp8_scale_is_ieee_fp32_division(orc):
    """s = amax / 448 rounded once to fp32, for every positive finite bf16
    amax: compared with numpy's IEEE float32 division and, on a sample,
    with exact rational rounding."""
    amax = FINITE_BF16[(FINITE_BF16 > 0) & (FINITE_BF16 < 0x7F80)]
    rows = np.zeros((amax.size, 128), np.uint16)
    rows[:, 5] = amax
    _, s = orc.group_quant(rows, 128, 0)
    want = amax.astype(np.uint32) << 16
    want = want.view(np.float32) / np.float32(448.0)
    assert np.array_equal(s[:, 0].view(np.uint32), want.view(np.uint32))
    for b, sv in zip(amax[::97], s[::97, 0]):
        assert int(sv.view(np.uint32)) == R.f32_round(R.bf16_value(int(b)) / 448)
