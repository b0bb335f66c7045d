"""The kernel's per-element number helpers and the raw gfx950 converts,
checked on the GPU against the CPU oracle over exhaustive and adversarial
inputs (test-only probe library, tests/hip/convert_probe.hip)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from tests.gpu_util import bf16_f64, call_probe, dev, host, say

pytestmark = pytest.mark.gpu

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FIN16 = ALL16[((ALL16 >> 7) & 0xFF) != 0xFF]
MAG16 = FIN16[FIN16 < 0x8000]                 # +0 and every positive finite bf16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import fp4_quant_amd as fq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert fq.rmsq_device_supported(0), "GPU tests need a gfx950 device"


def _f32(bits16):
    return (bits16.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------ raw converts --
def test_hw_bf16_convert_is_round_to_nearest_even():
    say("raw v_cvt_pk_bf16_f32")
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 4_000_000, dtype=np.uint64).astype(np.uint32)
    mids = (FIN16.astype(np.uint32) << 16) | 0x8000
    bits = np.concatenate([bits, mids, mids + 1, mids - 1, FIN16.astype(np.uint32) << 16])
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    out = torch.empty(f.size, dtype=torch.int16, device="cuda")
    call_probe("probe_cvt_bf16", dev(f), out, n=f.size)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(host(out), want)


def test_hw_fp8_convert_matches_oracle(orc):
    say("raw v_cvt_pk_fp8_f32")
    rng = np.random.default_rng(2)
    v = np.concatenate([_f32(FIN16), rng.uniform(-463.9, 463.9, 2_000_000).astype(np.float32),
                        (rng.standard_normal(1_000_000) * 2.0 ** -8).astype(np.float32)])
    # every e4m3fn rounding midpoint and its fp32 neighbours
    t = orc.e4m3fn_table()
    mags = np.unique(np.abs(t[~np.isnan(t)]))
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    mb = mids.view(np.uint32)
    v = np.concatenate([v, mids, (mb + 1).view(np.float32), (mb - 1).view(np.float32), -mids, np.float32([0.0, -0.0])])
    v = v[np.abs(v) < 464]
    if v.size % 2:
        v = v[:-1]
    out = torch.empty(v.size * 2, dtype=torch.uint8, device="cuda")
    call_probe("probe_cvt_fp8", dev(v), out, n=v.size // 2)
    o = host(out).reshape(-1, 4)
    want = orc.e4m3fn_encode(v.astype(np.float64)).reshape(-1, 2)
    # low word holds (b, a), high word (a, b): the first operand lands in the lower byte
    assert np.array_equal(o[:, 0], want[:, 1]) and np.array_equal(o[:, 1], want[:, 0])
    assert np.array_equal(o[:, 2], want[:, 0]) and np.array_equal(o[:, 3], want[:, 1])


def test_hw_fp4_convert_matches_oracle(orc):
    say("raw v_cvt_scalef32_pk_fp4_f32")
    rng = np.random.default_rng(3)
    small = _f32(FIN16)
    small = small[np.abs(small) < 8]
    v = np.concatenate([small, rng.uniform(-7.999, 7.999, 1_000_000).astype(np.float32),
                        np.float32(np.arange(-32, 32) / 4.0)])
    v = v[: v.size // 8 * 8]
    out = torch.empty(v.size // 2, dtype=torch.uint8, device="cuda")
    call_probe("probe_cvt_fp4", dev(v), out, n=v.size // 8)
    o = host(out)
    got = np.stack([o & 0xF, o >> 4], -1).reshape(-1)
    want = orc.e2m1_encode(v.astype(np.float64))
    tab = orc.e2m1_table()
    assert np.array_equal(tab[got], tab[want])                  # as values (+-0 equal)
    nz = tab[want] != 0
    assert np.array_equal(got[nz], want[nz])                      # and as codes when nonzero


def test_hw_fp4_scaled_bf16_convert_every_scale_byte(orc):
    """v_cvt_scalef32_pk_fp4_bf16 with scale bits byte << 23 gives the e2m1
    code of v / 2^(byte - 127) (nearest even, saturating at 6), for every e8m0
    byte 0..254 and every finite bf16 v below 2^(byte - 127 + 4), i.e. up to
    twice the largest magnitude a group with that scale byte holds. Both
    nibbles of the pair are checked."""
    say("raw v_cvt_scalef32_pk_fp4_bf16, every scale byte")
    tab = orc.e2m1_table()
    vals = bf16_f64(FIN16)
    pairs, scales, want, owner = [], [], [], []
    for byte in range(255):
        e = byte - 127
        sel = np.abs(vals) < 2.0 ** (e + 4)
        b = FIN16[sel].astype(np.uint32)
        pairs.append(b | (b << 16))
        scales.append(np.full(b.size, np.uint32(byte << 23)).view(np.float32))
        want.append(orc.e2m1_encode(np.ldexp(vals[sel], -e)))
        owner.append(np.full(b.size, byte))
    p, sc, w, ow = (np.concatenate(a) for a in (pairs, scales, want, owner))
    out = torch.empty(p.size, dtype=torch.uint8, device="cuda")
    call_probe("probe_cvt_fp4_bf16_scaled", dev(p.view(np.int32)), dev(sc), out, n=p.size)
    o = host(out)
    bad = (tab[o & 0xF] != tab[w]) | (tab[o >> 4] != tab[w])
    assert not bad.any(), f"{bad.sum()} of {p.size} differ, first at scale byte {ow[bad][0]}"


def test_f64_to_bf16_single_rounding(orc):
    say("bf16_from_f64")
    rng = np.random.default_rng(4)
    base = bf16_f64(FIN16[(FIN16 & 0x7FFF) < 0x7F7F])
    nxt = bf16_f64(FIN16[(FIN16 & 0x7FFF) < 0x7F7F] + 1)
    mid = (base + nxt) / 2
    d = np.concatenate([mid, mid * (1 + 2.0 ** -40), mid * (1 - 2.0 ** -40), mid * (1 + 2.0 ** -52),
                        mid * (1 - 2.0 ** -52), rng.standard_normal(1_000_000) * 10.0 ** rng.integers(-40, 38, 1_000_000),
                        np.array([3.4e38, -3.4e38, 1e-45, -1e-46, 0.0, -0.0, 2.0 ** -134, 3 * 2.0 ** -134])])
    d = d[np.isfinite(d)]
    out = torch.empty(d.size, dtype=torch.int16, device="cuda")
    call_probe("probe_f64_to_bf16", dev(d), out, n=d.size)
    assert np.array_equal(host(out).view(np.uint16), orc.bf16_from_double(d))


# ------------------------------------------------------- kernel helpers --
def test_norm_bf16x8_matches_fp64_rounding(orc):
    say("norm_bf16x8")
    rng = np.random.default_rng(5)
    n = 400_000 * 8
    h = _f32(rng.choice(FIN16[(FIN16 & 0x7FFF) < 0x4700], n)).astype(np.float64)      # |h| < 32768
    g = _f32(rng.choice(FIN16[((FIN16 & 0x7FFF) > 0x3E00) & ((FIN16 & 0x7FFF) < 0x4000)], n)).astype(np.float64)
    hg = (h * g).astype(np.float32)                 # exact: 8 x 8 significant bits
    assert np.array_equal(hg.astype(np.float64), h * g)
    inv = 10.0 ** rng.uniform(-3, 2, n // 8)
    # one chunk in four aims its first product at a bf16 midpoint
    k = np.arange(0, n // 8, 4)
    target = hg[8 * k].astype(np.float64)
    tb = (target.astype(np.float32).view(np.uint32) & 0xFFFF0000) | 0x8000
    tmid = tb.view(np.float32).astype(np.float64)
    nz = target != 0
    inv[k[nz]] = tmid[nz] / target[nz]
    inv[k[nz]] *= 1 + rng.choice([-1, 0, 1], nz.sum()) * 2.0 ** -52
    ex = (rng.random(n // 8) < 0.05).astype(np.uint8)
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    am = torch.empty(n // 8, dtype=torch.int16, device="cuda")
    call_probe("probe_norm_bf16", dev(h.astype(np.float32)), dev(g.astype(np.float32)), dev(inv), dev(ex), out, am,
               n=n // 8)
    want = orc.bf16_from_double(hg.astype(np.float64) * np.repeat(inv, 8))
    assert np.array_equal(host(out).view(np.uint16), want)
    # the group maximum it returns: the largest bf16 magnitude of the 8 results
    assert np.array_equal(host(am).view(np.uint16), (want & 0x7FFF).reshape(-1, 8).max(axis=1))


def test_norm_bf16x8_products_outside_the_fp32_normal_range(orc):
    """h * gamma that is denormal, underflows to zero or overflows in fp32
    (extreme but finite bf16 inputs) still gives bf16(h * gamma * inv) taken
    in fp64, as the oracle computes it."""
    say("norm_bf16x8 extreme products")
    rng = np.random.default_rng(15)
    n = 100_000 * 8
    sig = lambda k: 1 + rng.integers(0, 128, k) / 128.0          # 8 significant bits
    sgn = lambda k: rng.choice([-1.0, 1.0], k)
    cases = []
    # denormal products (2^-149 <= |hg| < 2^-126) with inv up to 2^16
    e1 = rng.integers(-75, -63, n)
    cases.append((sgn(n) * sig(n) * 2.0 ** e1, sig(n) * 2.0 ** (rng.integers(-148, -126, n) - e1),
                  2.0 ** rng.uniform(0, 16, n // 8)))
    # products below 2^-150 (flush to zero in fp32) with inv up to 2^16
    e2 = rng.integers(-90, -75, n)
    cases.append((sgn(n) * sig(n) * 2.0 ** e2, sig(n) * 2.0 ** (rng.integers(-170, -151, n) - e2),
                  2.0 ** rng.uniform(0, 16, n // 8)))
    # products beyond the fp32 range with inv small enough for a finite y
    e3 = rng.integers(64, 120, n)
    cases.append((sgn(n) * sig(n) * 2.0 ** e3, sig(n) * 2.0 ** (rng.integers(128, 140, n) - e3),
                  2.0 ** rng.uniform(-30, -13, n // 8)))
    for h, g, inv in cases:
        h32, g32 = h.astype(np.float32), g.astype(np.float32)
        assert np.array_equal(h32.astype(np.float64), h) and np.array_equal(g32.astype(np.float64), g)
        assert np.array_equal(orc.bf16_to_double(orc.bf16_from_double(h)), h)      # bf16 values
        ex = np.zeros(n // 8, np.uint8)
        out = torch.empty(n, dtype=torch.int16, device="cuda")
        am = torch.empty(n // 8, dtype=torch.int16, device="cuda")
        call_probe("probe_norm_bf16", dev(h32), dev(g32), dev(inv), dev(ex), out, am, n=n // 8)
        want = orc.bf16_from_double(h * g * np.repeat(inv, 8))
        got = host(out).view(np.uint16)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"{bad.size} differ, first h={h[bad[0]]} g={g[bad[0]]} inv={inv[bad[0] // 8]}"
        assert np.array_equal(host(am).view(np.uint16), (want & 0x7FFF).reshape(-1, 8).max(axis=1))


def test_inverse_norm_fp32_and_row_test():
    """inv_norm32 (hardware v_rsq_f64, two Newton steps, a margin check with a
    fallback to the full fp64 formula) gives fl32 of inv = fl64(1 / fl64(sqrt(d)))
    and flags every row with inv > 2^16 or inv < 2^-100: random d over the
    range the kernels form, d aimed so that inv lies within a few hundred fp64
    ulps of an fp32 rounding midpoint, d around the row thresholds, and the
    ends (d = 0 and d = inf give inv = 0)."""
    say("inv_norm32")
    rng = np.random.default_rng(21)
    n = 1_000_000
    d_rand = np.ldexp(1.0 + rng.random(n), rng.integers(-280, 271, n))
    e = rng.integers(-120, 120, n)
    mid = np.ldexp(1.0 + (rng.integers(0, 2 ** 23, n) + 0.5) * 2.0 ** -23, e)
    d_aim = (1.0 / (mid * mid)) * (1.0 + rng.integers(-400, 401, n) * 2.0 ** -53)
    j = np.arange(-3000, 3001)
    d_thr = np.concatenate([1.0 / (t * (1.0 + j * 2.0 ** -53)) ** 2 for t in (2.0 ** 16, 2.0 ** -100)])
    d = np.concatenate([d_rand, d_aim, d_thr, [0.0, np.inf, 2.0 ** -149, 1.0, 0.25, 4.0]])
    inv32 = torch.empty(d.size, dtype=torch.float32, device="cuda")
    ex = torch.empty(d.size, dtype=torch.uint8, device="cuda")
    call_probe("probe_inv_norm", dev(d), inv32, ex, n=d.size)
    with np.errstate(divide="ignore"):
        inv = np.where(d > 0, 1.0 / np.sqrt(d), 0.0)
    got = host(inv32)
    with np.errstate(over="ignore"):   # inv above the fp32 range (d < 2^-256) rounds to inf, as in the kernel
        inv_f32 = inv.astype(np.float32)
    bad = np.flatnonzero(got.view(np.uint32) != inv_f32.view(np.uint32))
    assert bad.size == 0, f"{bad.size} differ, first d={d[bad[0]]!r} inv={inv[bad[0]]!r} got={got[bad[0]]!r}"
    flag = host(ex).astype(bool)
    must = (inv > 2.0 ** 16) | ((inv != 0) & (inv < 2.0 ** -100))
    must_not = (inv <= 2.0 ** 16 * (1 - 2.0 ** -47)) & ((inv == 0) | (inv >= 2.0 ** -100 * (1 + 2.0 ** -47)))
    assert np.all(flag[must]) and not np.any(flag[must_not])
    assert must.sum() > 1000 and must_not.sum() > 1000


def test_fp8_scale_every_amax():
    say("fp8_scale")
    out = torch.empty(MAG16.size, dtype=torch.float32, device="cuda")
    call_probe("probe_fp8_scale", dev(MAG16.view(np.int16).copy()), out, n=MAG16.size)
    want = _f32(MAG16) / np.float32(448.0)
    want[0] = 1.0
    assert np.array_equal(host(out).view(np.uint32), want.view(np.uint32))


def _amax_cases(rng):
    special = np.uint16([0x3F80, 0x4060, 0x40E0, 0x0001, 0x0080, 0x0100, 0x1000, 0x2000, 0x7F7F, 0x4360,
                         0x43E0, 0x3C00, 0x0C00])
    return np.concatenate([special, rng.choice(MAG16[MAG16 > 0], 40)])


def test_fp8_codes8_every_value_below_amax(orc):
    """For each group amax, every bf16 value v with |v| <= amax: code =
    e4m3fn(v / s) exactly, s the group scale."""
    say("fp8_codes8")
    rng = np.random.default_rng(6)
    for amax in _amax_cases(rng):
        vals = FIN16[(FIN16 & 0x7FFF) <= amax]
        vals = vals[: vals.size // 8 * 8]
        s = np.float32(_f32(np.uint16([amax]))[0] / np.float32(448.0))
        out = torch.empty(vals.size, dtype=torch.uint8, device="cuda")
        av = np.full(vals.size // 8, amax, np.uint16)
        call_probe("probe_fp8_codes", dev(_f32(vals)), dev(av.view(np.int16)), out, n=vals.size // 8)
        want = orc.e4m3fn_encode(bf16_f64(vals) / np.float64(s))
        got = host(out)
        assert np.array_equal(got, want), f"amax 0x{amax:04x}: {np.count_nonzero(got != want)} codes differ"


def test_fp8_exact_path(orc):
    say("fp8_exact")
    rng = np.random.default_rng(7)
    v = _f32(rng.choice(FIN16, 1_000_000))
    s = np.minimum(np.abs(v.astype(np.float64)) / rng.uniform(1e-3, 448, v.size), 3e38).astype(np.float32)
    s[s == 0] = np.float32(1e-45)
    s[: 1000] = np.float32(2.0 ** -140)                        # subnormal scales
    keep = np.abs(v.astype(np.float64) / s.astype(np.float64)) < 448
    v, s = v[keep], s[keep]
    out = torch.empty(v.size, dtype=torch.uint8, device="cuda")
    call_probe("probe_fp8_exact", dev(v), dev(s), out, n=v.size)
    assert np.array_equal(host(out), orc.e4m3fn_encode(v.astype(np.float64) / s.astype(np.float64)))


def test_mx_scale_byte_every_amax(orc):
    say("mx_scale_byte")
    out = torch.empty(MAG16.size, dtype=torch.uint8, device="cuda")
    call_probe("probe_mx_byte", dev(MAG16.view(np.int16).copy()), out, n=MAG16.size)
    want = np.array([127] + [orc.mx_scale_exponent(a) + 127 for a in bf16_f64(MAG16[1:])], np.uint8)
    assert np.array_equal(host(out), want)


def test_fp4_codes8_every_value_below_amax(orc):
    say("fp4_codes8")
    rng = np.random.default_rng(8)
    tab = orc.e2m1_table()
    for amax in _amax_cases(rng):
        vals = FIN16[(FIN16 & 0x7FFF) <= amax]
        vals = vals[: vals.size // 8 * 8]
        e = 0 if amax == 0 else orc.mx_scale_exponent(bf16_f64(np.uint16([amax]))[0])
        byte = np.full(vals.size // 8, e + 127, np.uint8)
        out = torch.empty(vals.size // 8, dtype=torch.int32, device="cuda")
        call_probe("probe_fp4_codes", dev(vals), dev(byte), out, n=vals.size // 8)
        w = host(out).view(np.uint32)
        got = np.stack([(w >> (4 * i)) & 0xF for i in range(8)], -1).reshape(-1)
        want = orc.e2m1_encode(np.ldexp(bf16_f64(vals), -e))
        assert np.array_equal(tab[got], tab[want]), f"amax 0x{amax:04x}"


# ------------------------------------------------- exhaustive pair sweeps --
# Inside a group every value satisfies |v| <= amax, and the group's codes
# depend only on (v, amax): the sweeps below cover every such pair of bf16
# values (1.07e9 pairs per format), in batches. RMSQ_EXHAUSTIVE_STRIDE > 1
# takes every k-th amax instead of all of them.
STRIDE = int(os.environ.get("RMSQ_EXHAUSTIVE_STRIDE", "1"))
_BY_MAG = FIN16[np.argsort(FIN16 & 0x7FFF, kind="stable")]
_MAGS = np.sort(FIN16 & 0x7FFF)


def _pair_batches(max_pairs=48_000_000):
    amaxes = MAG16[1:][::STRIDE]
    cnt = np.searchsorted(_MAGS, amaxes, side="right")          # values with |v| <= amax
    cnt8 = (cnt + 7) // 8 * 8
    i = 0
    while i < amaxes.size:
        j = i
        tot = 0
        while j < amaxes.size and (tot + cnt8[j] <= max_pairs or j == i):
            tot += cnt8[j]
            j += 1
        v = np.zeros(tot, np.uint16)
        owner = np.empty(tot // 8, np.int64)
        o = 0
        for k in range(i, j):
            v[o:o + cnt[k]] = _BY_MAG[:cnt[k]]
            owner[o // 8:(o + cnt8[k]) // 8] = k
            o += cnt8[k]
        yield amaxes, owner, v
        i = j


def _threaded(fn, arr, out, nthreads=16):
    parts = np.array_split(np.arange(arr.size), nthreads)
    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(lambda ix: out.__setitem__(ix, fn(arr[ix])) if ix.size else None, parts))


def test_rcp_within_one_ulp_for_every_scale():
    """Every scale the kernel forms (fl32(amax/448), amax >= 2^-100) has a
    v_rcp_f32 within 1 ulp of its exact reciprocal."""
    from fractions import Fraction
    say("v_rcp_f32 over all scales")
    amax = MAG16[MAG16 >= 0x0D80]
    s = _f32(amax) / np.float32(448.0)
    out = torch.empty(s.size, dtype=torch.float32, device="cuda")
    call_probe("probe_rcp", dev(s), out, n=s.size)
    r = host(out)
    up = np.nextafter(r, np.float32(np.inf))
    for sv, rv, uv in zip(s.tolist(), r.tolist(), up.tolist()):
        exact = 1 / Fraction(sv)
        assert abs(Fraction(rv) - exact) <= Fraction(uv) - Fraction(rv), sv


def test_fp8_codes8_every_value_amax_pair(orc):
    """The encode every kernel uses (bracketed hardware converts, undecided
    elements settled by the group's scale rounding direction, fp64 for
    scales below 2^-100) for every (bf16 value, bf16 amax) pair with
    |value| <= amax, under the scale the kernels form for that amax."""
    say(f"fp8_codes8 exhaustive pairs (stride {STRIDE})")
    total = 0
    for amaxes, owner, v in _pair_batches():
        s = (_f32(amaxes.astype(np.uint16)) / np.float32(448.0))[owner]
        vf = _f32(v)
        out = torch.empty(v.size, dtype=torch.uint8, device="cuda")
        av = amaxes.astype(np.uint16)[owner]
        call_probe("probe_fp8_codes", dev(vf), dev(av.view(np.int16)), out, n=v.size // 8)
        q = vf.astype(np.float64) / np.repeat(s.astype(np.float64), 8)
        want = np.empty(v.size, np.uint8)
        _threaded(orc.e4m3fn_encode, q, want)
        got = host(out)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"{bad.size} codes differ, first v={vf[bad[0]]} s={s[bad[0] // 8]}"
        total += v.size
    say(f"fp8 pairs checked: {total}")


def test_fp4_codes8_every_value_amax_pair(orc):
    say(f"fp4_codes8 exhaustive pairs (stride {STRIDE})")
    tab = orc.e2m1_table()
    total = 0
    for amaxes, owner, v in _pair_batches():
        ex = np.array([orc.mx_scale_exponent(a) for a in bf16_f64(amaxes)], np.int64)
        byte = (ex + 127).astype(np.uint8)[owner]
        out = torch.empty(v.size // 8, dtype=torch.int32, device="cuda")
        call_probe("probe_fp4_codes", dev(v), dev(byte), out, n=v.size // 8)
        w = host(out).view(np.uint32)
        got = np.stack([(w >> (4 * i)) & 0xF for i in range(8)], -1).reshape(-1)
        q = np.ldexp(bf16_f64(v), -np.repeat(ex[owner], 8))
        want = np.empty(v.size, np.uint8)
        _threaded(orc.e2m1_encode, q, want)
        bad = np.flatnonzero(tab[got] != tab[want])
        assert bad.size == 0, f"{bad.size} codes differ"
        total += v.size
    say(f"fp4 pairs checked: {total}")


# ------------------------------------------------------------ block-scaled MFMA --
_E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])


def _mfma_model(a, b, sa, sb, magnitude=False):
    """v_mfma_scale_f32_16x16x128_f8f6f4 with e2m1 A and B, as the GEMM uses
    it: lane l holds A row l % 16 and B column l % 16, K elements 32 * (l // 16)
    ... + 31 (element 8d + j in nibble j of dword d), with the e8m0 scale of
    that 32-block in byte 0 of its scale register; the result lane l holds
    column l % 16, rows 4 * (l // 16) ... + 3."""
    W = a.shape[0]
    out = np.zeros((W, 64, 4))
    for w in range(W):
        A, B = np.zeros((16, 128)), np.zeros((128, 16))
        for l in range(64):
            i, kb = l % 16, l // 16
            for d in range(4):
                for j in range(8):
                    A[i, 32 * kb + 8 * d + j] = _E2M1[(a[w, l, d] >> (4 * j)) & 15] * 2.0 ** (int(sa[w, l] & 255) - 127)
                    B[32 * kb + 8 * d + j, i] = _E2M1[(b[w, l, d] >> (4 * j)) & 15] * 2.0 ** (int(sb[w, l] & 255) - 127)
        D = np.abs(A) @ np.abs(B) if magnitude else A @ B
        for l in range(64):
            out[w, l] = D[4 * (l // 16):4 * (l // 16) + 4, l % 16]
    return out


def _e4m3(b):
    b = np.asarray(b, np.int64)
    sg = np.where(b & 0x80, -1.0, 1.0)
    E, m = (b >> 3) & 15, b & 7
    return sg * np.where(E == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (E - 7))


def _mfma8_model(ab, bb, sa, sb):
    """The same instruction with e4m3fn A and B: lane l holds A row l % 16 and
    B column l % 16, 32 K elements (byte j of the lane's 32 bytes is K element
    32 * (l // 16) + j; any order common to A and B gives the same sums);
    result as for e2m1. The scale bytes are taken as 2^(byte - 127) per lane,
    which the test only uses at 127."""
    W = ab.shape[0]
    out = np.zeros((W, 64, 4))
    for w in range(W):
        A, B = np.zeros((16, 128)), np.zeros((128, 16))
        for l in range(64):
            k = 32 * (l // 16) + np.arange(32)
            A[l % 16, k] = _e4m3(ab[w, l]) * 2.0 ** (int(sa[w, l] & 255) - 127)
            B[k, l % 16] = _e4m3(bb[w, l]) * 2.0 ** (int(sb[w, l] & 255) - 127)
        D = A @ B
        for l in range(64):
            out[w, l] = D[4 * (l // 16):4 * (l // 16) + 4, l % 16]
    return out


def test_hw_mfma_scale_fp8_layout():
    """The e4m3fn form of the block-scaled MFMA as the A16W8 GEMM uses it:
    unit scales (byte 0 of each scale register 127, the other bytes random),
    operand pairing and result layout. Codes of magnitude 0.5 .. 3.75 keep
    every sum of 128 products exact in fp32 and inside the 8-product
    alignment window."""
    say("raw v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3fn x e4m3fn)")
    rng = np.random.default_rng(31)
    W = 4

    def codes():
        return (rng.integers(6, 9, (W, 64, 32)) << 3 | rng.integers(0, 8, (W, 64, 32)) |
                rng.integers(0, 2, (W, 64, 32)) << 7).astype(np.uint8)
    ab, bb = codes(), codes()
    sa = np.uint32(127) | (rng.integers(0, 256, (W, 64)).astype(np.uint32) << 8)
    sb = np.uint32(127) | (rng.integers(0, 256, (W, 64)).astype(np.uint32) << 24)
    d = torch.zeros(W * 64 * 4, dtype=torch.float32, device="cuda")
    call_probe("probe_mfma_scale_fp8", dev(ab.view(np.int32).reshape(W, 64, 8)), dev(bb.view(np.int32).reshape(W, 64, 8)),
               dev(sa.view(np.int32)), dev(sb.view(np.int32)), d, n=W)
    assert np.array_equal(host(d).reshape(W, 64, 4).astype(np.float64), _mfma8_model(ab, bb, sa, sb))


def _mfma8_row0(pairs):
    """D[0][0] of one e4m3fn MFMA whose only nonzero operands are A row 0 and
    B column 0: pairs maps K element k (lane 16 * (k // 32), byte k % 32) to
    the two codes."""
    ab = np.zeros((1, 64, 32), np.uint8)
    bb = np.zeros((1, 64, 32), np.uint8)
    for k, (ca, cb) in pairs.items():
        ab[0, 16 * (k // 32), k % 32] = ca
        bb[0, 16 * (k // 32), k % 32] = cb
    unit = np.full((1, 64), 127, np.uint32)
    d = torch.zeros(256, dtype=torch.float32, device="cuda")
    call_probe("probe_mfma_scale_fp8", dev(ab.view(np.int32).reshape(1, 64, 8)), dev(bb.view(np.int32).reshape(1, 64, 8)),
               dev(unit.view(np.int32)), dev(unit.view(np.int32)), d, n=1)
    return float(host(d)[0])


def test_hw_mfma_fp8_block_alignment():
    """The accumulation model the A16W8 GEMM's error bound rests on: within
    each block of 8 consecutive K elements (8 bytes of a lane) the e4m3fn
    products are aligned to the largest and truncated toward zero 13 bits
    below its leading bit; across blocks nothing is lost at that distance.
    Big product 2^8 (16 x 16) at k = 0; a second product 2^(8-t) in the same
    block (k = 1) or the next (k = 8); and 1.875^2 * 2^(8-t), whose low bits
    show the truncation, for both signs."""
    say("e4m3fn MFMA block alignment")
    big = {0: (0x58, 0x58)}                               # 16 * 16 = 256

    def pow2(e):                                          # e4m3fn codes whose product is 2^e, e in -18..16
        ea = max(-9, min(8, e // 2))
        eb = e - ea

        def c(x):
            return x + 7 << 3 if x >= -6 else 1 << (x + 9)
        return c(ea), c(eb)
    for t in range(1, 24):
        p = pow2(8 - t)
        same = _mfma8_row0({**big, 1: p}) - 256.0
        nxt = _mfma8_row0({**big, 8: p}) - 256.0
        assert same == (2.0 ** (8 - t) if t <= 13 else 0.0), (t, same)
        assert nxt == 2.0 ** (8 - t), (t, nxt)
    for t in range(8, 17):
        ea = (8 - t) // 2
        x = 0x3F + (ea << 3) if ea >= -6 else None        # 1.875 * 2^ea
        y = 0x3F + ((8 - t - ea) << 3)                    # 1.875 * 2^(8 - t - ea)
        if x is None:
            continue
        small = 1.875 ** 2 * 2.0 ** (8 - t)
        kept = np.floor(small / 2.0 ** -5) * 2.0 ** -5     # multiples of 2^(8 - 13)
        assert _mfma8_row0({**big, 1: (x, y)}) - 256.0 == kept, t
        assert _mfma8_row0({**big, 1: (x | 0x80, y)}) - 256.0 == -kept, t


@pytest.mark.parametrize("lo,hi", [(126, 129), (112, 143)])
def test_hw_mfma_scale_fp4_layout(lo, hi):
    """The operand, scale and result layout of the block-scaled FP4 MFMA that
    the prequant GEMM is written against, on random codes and scale bytes in
    lo..hi-1 (the other bytes of the scale registers random). With bytes 126..128
    every product is a multiple of 2^-4 and every sum of 128 below 2^15, so
    the result is exact; with the wide range the fp32 sum may round, within
    128 * 2^-24 of the sum of |products|."""
    say(f"raw v_mfma_scale_f32_16x16x128_f8f6f4 (e2m1 x e2m1), scale bytes {lo}..{hi - 1}")
    rng = np.random.default_rng(21 + lo)
    W = 6
    a = rng.integers(0, 2 ** 32, (W, 64, 4), dtype=np.uint64).astype(np.uint32)
    b = rng.integers(0, 2 ** 32, (W, 64, 4), dtype=np.uint64).astype(np.uint32)
    sa = rng.integers(lo, hi, (W, 64)).astype(np.uint32) | (rng.integers(0, 256, (W, 64)).astype(np.uint32) << 8)
    sb = rng.integers(lo, hi, (W, 64)).astype(np.uint32) | (rng.integers(0, 256, (W, 64)).astype(np.uint32) << 16)
    d = torch.zeros(W * 64 * 4, dtype=torch.float32, device="cuda")
    call_probe("probe_mfma_scale_fp4", dev(a.view(np.int32)), dev(b.view(np.int32)), dev(sa.view(np.int32)),
               dev(sb.view(np.int32)), d, n=W)
    got = host(d).reshape(W, 64, 4).astype(np.float64)
    want = _mfma_model(a, b, sa, sb)
    if (lo, hi) == (126, 129):
        assert np.array_equal(got, want)
    else:
        absum = _mfma_model(a, b, sa, sb, magnitude=True)
        assert np.all(np.abs(got - want) <= 128 * 2.0 ** -24 * absum)
