"""Pins for the oracle's pipeline (residual add, RMSNorm, group quantization).

Expected values: a hand-worked row, closed forms, an exact re-derivation with
rationals and a 60-digit square root (tests/ref_exact.py), and invariants the
mathematics fixes. None of them is produced by the oracle.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from fp4_quant_amd import inputs
from tests import ref_exact as R

BF = inputs.to_bf16_bits


def _f(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------ hand-worked --
def _row_a():
    """N = 256, gamma = 1, eps = 0. sum(h^2) = 3.5^2 + 0.5^2 + 126 + 2*0.25 + 117
    = 256 = N, so mean(h^2) = 1, inv = 1 and y = h exactly."""
    h = np.zeros(256, np.float32)
    h[0], h[1] = 3.5, 0.5
    h[2:128] = 1.0
    h[128:130] = 0.5
    h[130:247] = 1.0
    return BF(h[None, :]), BF(np.ones(256, np.float32))


def test_row_a_fp8_by_hand(orc):
    x, g = _row_a()
    o = orc.rmsnorm_quant_group(x, g, 0.0, group=128, fmt=0, keep_bf16=True)
    assert np.array_equal(o["bf16"], x)
    # group 0: amax 3.5 -> s = 3.5/448 = 2^-7 exactly; 3.5/s = 448 -> 0x7E,
    # 0.5/s = 64 = 2^6 -> 0x68, 1/s = 128 = 2^7 -> 0x70
    # group 1: amax 1 -> s = fl32(1/448) = 0x3B124925; 1/s -> 448 -> 0x7E,
    # 0.5/s -> 224 = 1.75 * 2^7 -> 0x76, 0 -> 0x00
    assert list(o["scale"][0].view(np.uint32)) == [0x3C000000, 0x3B124925]
    want = [0x7E, 0x68] + [0x70] * 126 + [0x76] * 2 + [0x7E] * 117 + [0x00] * 9
    assert list(o["q"][0]) == want


def test_row_a_mxfp4_by_hand(orc):
    x, g = _row_a()
    for layout in (0, 1):
        o = orc.rmsnorm_quant_group(x, g, 0.0, group=32, fmt=1, scale_layout=layout)
        # group 0: amax 3.5 -> floor(log2) = 1 -> e = -1 (byte 126), X = 0.5:
        # 3.5/X = 7 saturates to 6 (code 7), 0.5/X = 1 (code 2), 1/X = 2 (code 4)
        # groups 1..7: amax 1 -> e = -2 (byte 125), X = 0.25: 1/X = 4 (code 6),
        # 0.5/X = 2 (code 4)
        want_s = [126] + [125] * 7
        got_s = o["scale"][0] if layout == 0 else o["scale"][[g * 32 for g in range(8)]]
        assert list(got_s) == want_s
        want_q = [0x27] + [0x44] * 15 + [0x66] * 48 + [0x44] + [0x66] * 58 + [0x06] + [0x00] * 4
        assert list(o["q"][0]) == want_q


def test_fp8_tie_heavy_group(orc):
    """Quant stage on a group with amax 3.5 (s = 2^-7, exact quotients): the
    quotients 2.625 and 2.875 are e4m3fn ties, 2^-10 and 3*2^-10 are ties
    between subnormals."""
    yb = np.zeros((1, 128), np.float32)
    yb[0, :6] = [3.5, 2.625 / 128, 2.875 / 128, 2.0 ** -17, 3 * 2.0 ** -17, -(2.0 ** -18)]
    q, s = orc.group_quant(BF(yb), 128, 0)
    assert s[0, 0] == 2.0 ** -7
    assert list(q[0, :6]) == [0x7E, 0x42, 0x44, 0x00, 0x02, 0x80]


# -------------------------------------------------------------- exact ref --
def _check_against_exact(orc, x, r, g, eps, group, fmt):
    o = orc.rmsnorm_quant_group(x, g, eps, residual=r, group=group, fmt=fmt, keep_bf16=True)
    for m in range(x.shape[0]):
        h, yb, sc, codes = R.reference_row(x[m], None if r is None else r[m], g, eps, group, fmt)
        if r is not None:
            assert list(o["residual_out"][m]) == h
        assert list(o["bf16"][m]) == yb
        if fmt == 0:
            assert list(o["scale"][m].view(np.uint32)) == sc
            assert list(o["q"][m]) == codes
        else:
            assert list(o["scale"][m]) == sc
            packed = [codes[2 * k] | (codes[2 * k + 1] << 4) for k in range(len(codes) // 2)]
            assert list(o["q"][m]) == packed


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("residual", [False, True])
def test_fp8_matches_exact_rational_reference(orc, seed, residual):
    p = inputs.make_problem(3, 256, seed_x=100 + seed, residual=residual, outliers=True)
    _check_against_exact(orc, p["x"], p.get("residual"), p["gamma"], 1e-6, 128, 0)


@pytest.mark.parametrize("seed", [0, 1])
def test_mxfp4_matches_exact_rational_reference(orc, seed):
    p = inputs.make_problem(2, 256, seed_x=200 + seed, residual=True, outliers=True)
    _check_against_exact(orc, p["x"], p["residual"], p["gamma"], 1e-6, 32, 1)


def test_tiny_workload_matches_exact_reference(orc):
    p = inputs.make_config("tiny")
    _check_against_exact(orc, p["x"], None, p["gamma"], p["eps"], 128, 0)


def test_eps_is_inside_the_root_and_large_eps_matters(orc):
    """With eps comparable to mean(h^2) the three plausible placements of eps
    give different rows; the exact reference puts it inside the root."""
    p = inputs.make_problem(2, 128, seed_x=300, residual=False, outliers=False)
    _check_against_exact(orc, p["x"], None, p["gamma"], 0.75, 128, 0)


# ------------------------------------------------------------ closed forms --
@pytest.mark.parametrize("k", [-3, 0, 2, 5])
def test_closed_form_rows(orc, k):
    """gamma = 1, eps = 0 and sum(h^2) = N * 4^k: inv = 2^-k exactly, so the
    bf16 output is h * 2^-k bit for bit."""
    rng = np.random.default_rng(7 + k)
    N = 512
    h = rng.choice(np.float32([1, -1, 0.5, -0.5]), N)
    # rebalance: pairs of (+-2, 0) keep sum(h^2) a known value, then top up
    ss = float((h.astype(np.float64) ** 2).sum())
    need = N - ss                                   # make sum(h^2) = N
    n_add = int(round(need / 0.75))                 # 0.5 -> 1 adds 0.75 each
    idx = np.flatnonzero(np.abs(h) == 0.5)[:n_add]
    h[idx] = np.sign(h[idx])
    assert (h.astype(np.float64) ** 2).sum() == N
    x = BF((h * np.float32(2.0 ** k))[None, :])
    g = BF(np.ones(N, np.float32))
    o = orc.rmsnorm_quant_group(x, g, 0.0, keep_bf16=True)
    assert np.array_equal(o["bf16"], BF(h[None, :]))


def test_zero_row_and_zero_group(orc):
    x = np.zeros((2, 256), np.float32)
    x[1, :128] = np.random.default_rng(1).standard_normal(128)
    for eps in (0.0, 1e-6):
        o = orc.rmsnorm_quant_group(BF(x), BF(np.ones(256, np.float32)), eps, keep_bf16=True)
        assert np.all(_f(o["bf16"][0]) == 0)
        assert list(o["scale"][0]) == [1.0, 1.0]          # safe scale for an all-zero group
        assert o["scale"][1, 1] == 1.0 and o["scale"][1, 0] != 1.0
        assert np.all(orc.e4m3fn_table()[o["q"][0]] == 0)
        assert np.all(orc.e4m3fn_table()[o["q"][1, 128:]] == 0)
        o4 = orc.rmsnorm_quant_group(BF(x), BF(np.ones(256, np.float32)), eps, group=32, fmt=1)
        assert list(o4["scale"][0]) == [127] * 8 and np.all(o4["q"][0] == 0)


# -------------------------------------------------------------- invariants --
shapes = st.tuples(st.integers(1, 6), st.sampled_from([128, 256, 512]))


@settings(max_examples=25, deadline=None)
@given(shapes, st.integers(0, 2 ** 31 - 1), st.booleans())
def test_fp8_group_amax_maps_to_448_and_bounds(orc, shape, seed, residual):
    M, N = shape
    p = inputs.make_problem(M, N, seed_x=seed, residual=residual, outliers=True)
    o = orc.rmsnorm_quant_group(p["x"], p["gamma"], 1e-6, residual=p.get("residual"), keep_bf16=True)
    yb = _f(o["bf16"]).reshape(M, N // 128, 128)
    q = orc.e4m3fn_table()[o["q"]].reshape(M, N // 128, 128)
    s = o["scale"].astype(np.float64)
    amax = np.abs(yb).max(axis=2)
    at_max = np.abs(yb) == amax[..., None]
    assert np.all(np.abs(q[at_max & (amax[..., None] > 0)]) == 448)
    assert np.all(np.abs(q * s[..., None]) <= amax[..., None] * (1 + 2.0 ** -23))
    # every code is the nearest code to yb / s: within half a code spacing
    assert np.all(np.sign(q) * np.sign(yb) >= 0)


@settings(max_examples=25, deadline=None)
@given(shapes, st.integers(0, 2 ** 31 - 1))
def test_mxfp4_amax_code_and_error_bound(orc, shape, seed):
    M, N = shape
    p = inputs.make_problem(M, N, seed_x=seed, residual=True, outliers=True)
    o = orc.rmsnorm_quant_group(p["x"], p["gamma"], 1e-6, residual=p["residual"], group=32, fmt=1,
                                keep_bf16=True)
    yb = _f(o["bf16"]).reshape(M, N // 32, 32)
    codes = np.stack([o["q"] & 0xF, o["q"] >> 4], axis=-1).reshape(M, N // 32, 32)
    q = orc.e2m1_table()[codes]
    X = 2.0 ** (o["scale"].astype(np.float64) - 127)
    amax = np.abs(yb).max(axis=2)
    at_max = (np.abs(yb) == amax[..., None]) & (amax[..., None] > 0)
    assert set(np.abs(q[at_max]).tolist()) <= {4.0, 6.0}
    assert np.all(np.abs(q) <= 6)
    v = yb / X[..., None]
    grid_step = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0))
    inside = np.abs(v) <= 6
    assert np.all(np.abs(q - v)[inside] <= grid_step[inside] / 2)
    assert np.all((2.0 ** 2 <= amax / X) | (amax == 0)) and np.all(amax / X < 8)


@settings(max_examples=20, deadline=None)
@given(st.integers(1, 4), st.integers(0, 2 ** 31 - 1), st.integers(-20, 20), st.sampled_from([0, 1]))
def test_quant_stage_scale_equivariance(orc, M, seed, k, fmt):
    """Q(2^k * v) has the same codes and the scale times 2^k (normal range)."""
    group = 128 if fmt == 0 else 32
    yb = inputs.make_problem(M, 256, seed_x=seed, residual=False, outliers=True)["x"]
    q0, s0 = orc.group_quant(yb, group, fmt)
    q1, s1 = orc.group_quant(BF(_f(yb) * 2.0 ** k), group, fmt)
    assert np.array_equal(q0, q1)
    if fmt == 0:
        assert np.array_equal(s1.astype(np.float64), s0.astype(np.float64) * 2.0 ** k)
    else:
        assert np.array_equal(s1.astype(np.int64), s0.astype(np.int64) + k)


@settings(max_examples=15, deadline=None)
@given(st.integers(1, 4), st.integers(0, 2 ** 31 - 1), st.integers(-30, 30))
def test_pipeline_invariant_under_power_of_two_input_scaling(orc, M, seed, k):
    """With eps = 0, RMSNorm removes a power-of-two scale of x exactly."""
    p = inputs.make_problem(M, 512, seed_x=seed, residual=False, outliers=True)
    o0 = orc.rmsnorm_quant_group(p["x"], p["gamma"], 0.0, keep_bf16=True)
    o1 = orc.rmsnorm_quant_group(BF(_f(p["x"]) * 2.0 ** k), p["gamma"], 0.0, keep_bf16=True)
    for key in ("bf16", "q", "scale"):
        assert np.array_equal(o0[key], o1[key])


# ------------------------------------------------------------- structure --
def test_fused_equals_the_unfused_chain(orc):
    p = inputs.make_problem(8, 1024, seed_x=5, residual=True, outliers=True)
    o = orc.rmsnorm_quant_group(p["x"], p["gamma"], 1e-6, residual=p["residual"], keep_bf16=True)
    h, yb = orc.add_rmsnorm(p["x"], p["gamma"], 1e-6, residual=p["residual"])
    q, s = orc.group_quant(yb)
    assert np.array_equal(h, o["residual_out"]) and np.array_equal(yb, o["bf16"])
    assert np.array_equal(q, o["q"]) and np.array_equal(s, o["scale"])


def test_tiled32_is_a_permutation_of_row_major(orc):
    M, N = 70, 256
    p = inputs.make_problem(M, N, seed_x=9, residual=True, outliers=True)
    row = orc.rmsnorm_quant_group(p["x"], p["gamma"], 1e-6, residual=p["residual"], group=32, fmt=1)
    til = orc.rmsnorm_quant_group(p["x"], p["gamma"], 1e-6, residual=p["residual"], group=32, fmt=1,
                                  scale_layout=1, scale_fill=0xEE)
    G = N // 32
    assert til["scale"].size == 96 * G
    for m in range(M):
        for g in range(G):
            assert til["scale"][(m // 32) * 32 * G + g * 32 + m % 32] == row["scale"][m, g]
    pad_rows = [(m // 32) * 32 * G + g * 32 + m % 32 for m in range(M, 96) for g in range(G)]
    assert np.all(til["scale"][pad_rows] == 0xEE)
    assert np.array_equal(til["q"], row["q"])


def test_column_major_scales_are_the_transpose(orc):
    p = inputs.make_problem(37, 640, seed_x=12, residual=True, outliers=True)
    for fmt, group in ((0, 128), (1, 32)):
        row = orc.rmsnorm_quant_group(p["x"], p["gamma"], 1e-6, residual=p["residual"], group=group, fmt=fmt)
        col = orc.rmsnorm_quant_group(p["x"], p["gamma"], 1e-6, residual=p["residual"], group=group, fmt=fmt,
                                      scale_layout=2)
        assert col["scale"].shape == (640 // group, 37)
        assert np.array_equal(col["scale"], row["scale"].T) and np.array_equal(col["q"], row["q"])


def test_row_stride_larger_than_n(orc):
    p = inputs.make_problem(5, 256, seed_x=4, residual=True, outliers=True)
    xs = np.zeros((5, 384), np.uint16)
    rs = np.zeros((5, 320), np.uint16)
    xs[:, :256] = p["x"]
    rs[:, :256] = p["residual"]
    a = orc.rmsnorm_quant_group(p["x"], p["gamma"], 1e-6, residual=p["residual"], keep_bf16=True)
    b = orc.rmsnorm_quant_group(xs[:, :256], p["gamma"], 1e-6, residual=rs[:, :256], keep_bf16=True)
    for key in a:
        assert np.array_equal(a[key], b[key])
