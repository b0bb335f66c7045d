"""Parity of the A16WFP4 prequant GEMM (through the C ABI) with the oracle.

The oracle sums the exact products of the dequantized operands in double;
the matrix cores sum them in fp32. Every product qa * qw * 2^(ea + ew - 254)
is exact in fp32 here (a few significant bits, exponents well inside the
fp32 range), so the only error is the rounding of the fp32 additions: with
n terms added in any order, |error| <= (n - 1) u sum|products| / (1 - (n-1) u),
u = 2^-24. The tests take n = K and allow twice that (K * 2^-23 sum|p|), which
also covers a hardware sum that rounds toward zero inside one instruction.
Inputs whose partial sums are all exact in fp32 must match bit for bit.
"""
import numpy as np
import pytest
import torch

import fp4_quant_amd as fq
from fp4_quant_amd import inputs
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert fq.rmsq_device_supported(0), "GPU tests need a gfx950 device"


def _dequant(codes, scales):
    lo, hi = codes & 0xF, codes >> 4
    q = np.stack([E2M1[lo], E2M1[hi]], -1).reshape(codes.shape[0], -1)
    return q * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)


def _abs_sum(orc, a, w, ws):
    """sum_k |dq(a)[m, k] * dq(w)[n, k]| from the oracle's group quantization."""
    qa, sa = orc.group_quant(a, 32, 1, 0)
    return np.abs(_dequant(qa, sa)) @ np.abs(_dequant(w, ws)).T


def shuffle_np(w, ws):
    """The preshuffled layout written out with numpy: for tile t, step s and
    lane l, row 16t + l%16 and 32-group 4s + l/16."""
    N, K = w.shape[0], w.shape[1] * 2
    S = K // 128
    c = w.reshape(N // 16, 16, S, 4, 16)            # [t, row in tile, s, kb, byte]
    c = c.transpose(0, 2, 3, 1, 4)                  # [t, s, kb, row, byte]: lane = kb * 16 + row
    e = ws.reshape(N // 16, 16, S, 4).transpose(0, 2, 3, 1)
    return np.ascontiguousarray(c).reshape(-1), np.ascontiguousarray(e).reshape(-1)


def run_gemm(a, w, ws, *, lda=None, ldc=None, layout=fq.W_ROW_MAJOR):
    M, K = a.shape
    N = w.shape[0]
    lda = lda or K
    ldc = ldc or N
    full = np.full((max(M, 1), lda), 0x7FC1, np.uint16)    # NaN padding must never be read
    full[:M, :K] = a
    da = dev(full)
    dw, dws = dev(w), dev(ws)
    if layout == fq.W_PRESHUFFLED:
        sw, sws = torch.empty_like(dw), torch.empty_like(dws)
        fq.mxfp4_weight_preshuffle(dw, dws, N, K, sw, sws)
        dw, dws = sw, sws
    guard = 1024
    out = torch.full((guard + max(M, 1) * ldc + guard,), float("nan"), dtype=torch.float32, device="cuda")
    say(f"gemm M={M} N={N} K={K} lda={lda} ldc={ldc} layout={layout}")
    fq.gemm_a16wfp4_prequant(da, lda, dw, dws, layout, M, N, K, out[guard:], ldc)
    torch.cuda.synchronize()
    o = host(out)
    assert np.all(np.isnan(o[:guard])) and np.all(np.isnan(o[guard + max(M, 1) * ldc:])), "guard band written"
    body = o[guard:guard + max(M, 1) * ldc].reshape(max(M, 1), ldc)
    if ldc > N:
        assert np.all(np.isnan(body[:M, N:])), "row padding written"
    return body[:M, :N]


def check(orc, a, w, ws, got):
    want = orc.gemm_a16wfp4_prequant(a, w, ws)
    K = a.shape[1]
    bound = K * 2.0 ** -23 * _abs_sum(orc, a, w, ws)
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(np.isfinite(got))
    bad = err > bound
    assert not bad.any(), (f"{bad.sum()} outputs beyond the bound; worst at {np.unravel_index(np.argmax(err - bound), err.shape)}: "
                           f"got {got.flat[np.argmax(err - bound)]} want {want.flat[np.argmax(err - bound)]}")
    return err


LAYOUTS = [fq.W_ROW_MAJOR, fq.W_PRESHUFFLED]

# Shapes: the decode workload, the small-M path (M <= 4, up to K = 8192 with
# 16 waves) and the per-wave path (K = 8320 needs a 17th wave; M > 4), one to
# four row tiles, row blocks past 64, ragged M in every tile count, and two
# column tiles per small-M workgroup (N/16 >= 256 and even; 4112 is odd).
SHAPES = [(4, 2112, 7168), (1, 16, 128), (3, 16, 128), (2, 48, 1152), (4, 48, 256), (4, 32, 8192),
          (4, 32, 8320), (5, 32, 256), (16, 64, 384), (17, 32, 1024), (33, 48, 512), (64, 32, 7168),
          (70, 16, 256), (130, 32, 640), (4, 256, 16384), (4, 4096, 256), (2, 4128, 384), (4, 4112, 256)]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_matches_oracle(orc, M, N, K, layout):
    g = inputs.make_gemm(M, N, K, seed=40 + M + K)
    got = run_gemm(g["a"], g["w"], g["ws"], layout=layout)
    check(orc, g["a"], g["w"], g["ws"], got)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (2112, 7168)])
def test_preshuffle_is_the_documented_permutation(N, K):
    w, ws = inputs.fp4_weights(N, K, seed=70 + N)
    dw, dws = dev(w), dev(ws)
    sw, sws = torch.empty_like(dw), torch.empty_like(dws)
    say(f"preshuffle N={N} K={K}")
    fq.mxfp4_weight_preshuffle(dw, dws, N, K, sw, sws)
    torch.cuda.synchronize()
    ew, es = shuffle_np(w, ws)
    assert np.array_equal(host(sw).reshape(-1), ew)
    assert np.array_equal(host(sws).reshape(-1), es)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemm_layouts_agree_bit_for_bit(M):
    """Both weight layouts feed the same operands in the same order."""
    g = inputs.make_gemm(M, 2112, 7168, seed=80 + M)
    r0 = run_gemm(g["a"], g["w"], g["ws"], layout=fq.W_ROW_MAJOR)
    r1 = run_gemm(g["a"], g["w"], g["ws"], layout=fq.W_PRESHUFFLED)
    assert np.array_equal(r0.view(np.uint32), r1.view(np.uint32))


@pytest.mark.parametrize("M", [5, 3])
def test_gemm_exact_when_partial_sums_are_exact(orc, M):
    """Activations 2^e * e2m1 with a 4 or 6 in every group (lossless under
    MXFP4), e in -2..2, weight scales 2^0: every product is a multiple of
    2^-4 below 2^8 in magnitude and every partial sum below 2^20, so any fp32
    summation order is exact and the GPU must equal the oracle bit for bit."""
    rng = np.random.default_rng(50 + M)
    N, K = 48, 7168
    codes = rng.integers(0, 16, (M, K))
    codes[:, ::32] = rng.choice([6, 7, 14, 15], (M, K // 32))
    A = E2M1[codes] * np.repeat(np.ldexp(1.0, rng.integers(-2, 3, (M, K // 32))), 32, axis=1)
    a = inputs.to_bf16_bits(A.astype(np.float32))
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = np.full((N, K // 32), 127, np.uint8)
    want = orc.gemm_a16wfp4_prequant(a, w, ws)
    for layout in LAYOUTS:
        got = run_gemm(a, w, ws, layout=layout)
        assert np.array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("M", [6, 3])
def test_gemm_strided_rows_and_padded_output(orc, M):
    g = inputs.make_gemm(M, 32, 256, seed=60 + M)
    for layout in LAYOUTS:
        got = run_gemm(g["a"], g["w"], g["ws"], lda=264, ldc=40, layout=layout)
        check(orc, g["a"], g["w"], g["ws"], got)


def test_gemm_zero_rows_and_special_groups(orc):
    """All-zero rows, a group of -0.0, a group of subnormal bf16 (scale byte
    0) met by weights scaled by 2^73 so its products stay fp32 normals, and a
    group near 2^99, against the oracle."""
    g = inputs.make_gemm(8, 32, 256, seed=61)
    a, ws = g["a"].copy(), g["ws"].copy()
    a[1] = 0
    a[2, 32:64] = 0x8000                                   # -0.0
    a[3, :32] = np.arange(1, 33, dtype=np.uint16)          # subnormal bf16, 2^-133 .. 2^-128
    ws[:, 0] = 200                                         # first K group of every column: 2^73
    a[4, 64:96] = 0x7100                                   # 2^99
    a[5, 96:128] = 0xF0C0                                  # -1.5 * 2^98
    got = run_gemm(a, g["w"], ws)
    assert np.all(got[1] == 0)
    check(orc, a, g["w"], ws, got)
    # the same groups on the small-M path (M <= 4)
    got = run_gemm(a[1:5], g["w"], ws, layout=fq.W_PRESHUFFLED)
    assert np.all(got[0] == 0)
    check(orc, a[1:5], g["w"], ws, got)


def test_gemm_m_zero_launches_nothing():
    w = torch.zeros((16, 64), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((16, 4), dtype=torch.uint8, device="cuda")
    a = torch.zeros((1, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((16,), 3.0, device="cuda")
    fq.gemm_a16wfp4_prequant(a, 128, w, ws, fq.W_ROW_MAJOR, 0, 16, 128, out, 16)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_gemm_repeatable():
    """The same call twice gives the same bits (fixed summation order)."""
    g = inputs.make_gemm(4, 2112, 7168, seed=62)
    a, w, ws = g["a"], g["w"], g["ws"]
    for layout in LAYOUTS:
        r1 = run_gemm(a, w, ws, layout=layout)
        r2 = run_gemm(a, w, ws, layout=layout)
        assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))


# ------------------------------------------------------------------ A16W8 --
def e4m3_values(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _abs_sum8(orc, a, w, ws):
    """sum_k |dq(a)[m, k] * dq(w)[n, k]| from the oracle's FP8 group quantization."""
    M, K = a.shape
    N = w.shape[0]
    qa, sa = orc.group_quant(a, 128, 0, 0)
    da = np.abs(e4m3_values(qa)) * np.repeat(sa.reshape(M, -1).astype(np.float64), 128, axis=1)
    dw = np.abs(e4m3_values(w)) * np.repeat(np.repeat(ws.astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    return da @ dw.T


def shuffle8_np(w):
    """The A16W8 preshuffled layout written out with numpy: for tile t, step s,
    half h and lane l, bytes 128s + 32(l/16) + 16h .. +15 of row 16t + l%16."""
    N, K = w.shape
    S = K // 128
    c = w.reshape(N // 16, 16, S, 4, 2, 16)          # [t, row in tile, s, q, h, byte]
    c = c.transpose(0, 2, 4, 3, 1, 5)                # [t, s, h, q, row, byte]: lane = q * 16 + row
    return np.ascontiguousarray(c).reshape(-1)


def run_gemm8(a, w, ws, *, lda=None, ldc=None, layout=fq.W_ROW_MAJOR):
    M, K = a.shape
    N = w.shape[0]
    lda = lda or K
    ldc = ldc or N
    full = np.full((max(M, 1), lda), 0x7FC1, np.uint16)
    full[:M, :K] = a
    da = dev(full)
    dw, dws = dev(w), dev(ws)
    if layout == fq.W_PRESHUFFLED:
        sw = torch.empty_like(dw)
        fq.fp8_weight_preshuffle(dw, N, K, sw)
        dw = sw
    guard = 1024
    out = torch.full((guard + max(M, 1) * ldc + guard,), float("nan"), dtype=torch.float32, device="cuda")
    say(f"gemm8 M={M} N={N} K={K} lda={lda} ldc={ldc} layout={layout}")
    fq.gemm_a16w8_prequant(da, lda, dw, dws, layout, M, N, K, out[guard:], ldc)
    torch.cuda.synchronize()
    o = host(out)
    assert np.all(np.isnan(o[:guard])) and np.all(np.isnan(o[guard + max(M, 1) * ldc:])), "guard band written"
    body = o[guard:guard + max(M, 1) * ldc].reshape(max(M, 1), ldc)
    if ldc > N:
        assert np.all(np.isnan(body[:M, N:])), "row padding written"
    return body[:M, :N]


def _block8_bound(orc, a, w, ws):
    """sum over the 8-element K blocks of 7 * 2^-13 * max |product| in the
    block: the e4m3fn matrix-core sum aligns the 8 products of a block to the
    largest and truncates the others to 13 bits below its leading bit (pinned
    by test_hw_mfma_fp8_block_alignment), so each block loses less than
    2^-13 of its largest product per other product."""
    M, K = a.shape
    N = w.shape[0]
    qa, sa = orc.group_quant(a, 128, 0, 0)
    da = np.abs(e4m3_values(qa)) * np.repeat(sa.reshape(M, -1).astype(np.float64), 128, axis=1)
    dw = np.abs(e4m3_values(w)) * np.repeat(np.repeat(ws.astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    total = np.zeros((M, N))
    for b in range(0, K, 8):
        total += np.max(da[:, None, b:b + 8] * dw[None, :, b:b + 8], axis=-1)
    return 7 * 2.0 ** -13 * total


def check8(orc, a, w, ws, got):
    """Within the matrix cores' block truncation (_block8_bound) plus
    K * 2^-23 * sum|products| for the fp32 sums over blocks, the scaling by
    sa * sw and the accumulation over K steps (twice the bound of K fp32
    additions)."""
    want = orc.gemm_a16w8_prequant(a, w, ws)
    bound = a.shape[1] * 2.0 ** -23 * _abs_sum8(orc, a, w, ws) + _block8_bound(orc, a, w, ws)
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(np.isfinite(got))
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} outputs beyond the bound; worst excess {float((err - bound).max())}"


# decode workload, the small-M path (M <= 4) and not, one or two row tiles, several row
# blocks, weight block rows that end inside a tile row (N = 2112: 16.5 blocks)
SHAPES8 = [(4, 2112, 7168), (1, 16, 128), (3, 32, 256), (4, 48, 8192), (4, 32, 8320), (5, 144, 384),
           (16, 64, 1024), (17, 32, 512), (33, 48, 256), (70, 16, 640), (4, 256, 16384)]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", SHAPES8)
def test_gemm8_matches_oracle(orc, M, N, K, layout):
    g = inputs.make_gemm8(M, N, K, seed=140 + M + K)
    got = run_gemm8(g["a"], g["w"], g["ws"], layout=layout)
    check8(orc, g["a"], g["w"], g["ws"], got)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (2112, 7168)])
def test_fp8_preshuffle_is_the_documented_permutation(N, K):
    w, _ = inputs.fp8_block_weights(N, K, seed=170 + N)
    dw = dev(w)
    sw = torch.empty_like(dw)
    say(f"fp8 preshuffle N={N} K={K}")
    fq.fp8_weight_preshuffle(dw, N, K, sw)
    torch.cuda.synchronize()
    assert np.array_equal(host(sw).reshape(-1), shuffle8_np(w))


@pytest.mark.parametrize("M", [3, 6])
def test_gemm8_exact_when_partial_sums_are_exact(orc, M):
    """Activations 2^e * e4m3fn with +-448 in every group (lossless under FP8,
    scale 2^e), e in -1..1, codes of magnitude 2^5 .. 448 and weight codes of
    magnitude 0.5 .. 3.75 with unit block scales: every product is a multiple
    of 2^-3 and (checked below) every partial sum stays below 2^21, so any
    fp32 summation order is exact; and within any 8-element block the
    smallest product is at most 11 bits below the largest, inside the matrix
    cores' 13-bit alignment window. The GPU must equal the oracle bit for
    bit."""
    rng = np.random.default_rng(60 + M)
    N, K = 48, 2048
    codes = (rng.integers(13, 16, (M, K)) << 3 | rng.integers(0, 8, (M, K)) | rng.integers(0, 2, (M, K)) << 7)
    codes = codes.astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    codes[:, ::128] = rng.choice([0x7E, 0xFE], (M, K // 128))
    e = rng.integers(-1, 2, (M, K // 128))
    A = e4m3_values(codes) * np.repeat(np.ldexp(1.0, e), 128, axis=1)
    a = inputs.to_bf16_bits(A.astype(np.float32))
    w = (rng.integers(6, 9, (N, K)) << 3 | rng.integers(0, 8, (N, K)) | rng.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    ws = np.ones((1, K // 128), np.float32)
    # premise: products are multiples of 2^(5 - 1 - 1 - 6) = 2^-3, |partial sums| < 2^21
    assert (np.abs(A) @ np.abs(e4m3_values(w)).T).max() < 2.0 ** 21
    want = orc.gemm_a16w8_prequant(a, w, ws)
    for layout in LAYOUTS:
        got = run_gemm8(a, w, ws, layout=layout)
        assert np.array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("M", [6, 3])
def test_gemm8_strided_rows_and_padded_output(orc, M):
    g = inputs.make_gemm8(M, 32, 256, seed=160 + M)
    for layout in LAYOUTS:
        got = run_gemm8(g["a"], g["w"], g["ws"], lda=264, ldc=40, layout=layout)
        check8(orc, g["a"], g["w"], g["ws"], got)


def test_gemm8_zero_rows_and_special_groups(orc):
    """All-zero rows and groups (scale 1, codes 0), a group of -0.0, a group
    with an e4m3fn-subnormal quotient range, and groups near 2^60."""
    g = inputs.make_gemm8(8, 32, 512, seed=161)
    a = g["a"].copy()
    a[1] = 0
    a[2, 128:256] = 0x8000
    a[3, :128] = 0x3F80                                   # 1.0 ...
    a[3, 0] = 0x4780                                      # ... with one 65536: 1.0 / s is an e4m3fn subnormal
    a[4, 256:384] = 0x5D80                                # 2^60
    a[5, 384:512] = 0xDD40                                # -1.5 * 2^59
    for rows in (slice(0, 8), slice(1, 5)):
        got = run_gemm8(a[rows], g["w"], g["ws"], layout=fq.W_PRESHUFFLED)
        check8(orc, a[rows], g["w"], g["ws"], got)
    got = run_gemm8(a, g["w"], g["ws"])
    assert np.all(got[1] == 0)


def test_gemm8_repeatable():
    g = inputs.make_gemm8(4, 2112, 7168, seed=162)
    for layout in LAYOUTS:
        r1 = run_gemm8(g["a"], g["w"], g["ws"], layout=layout)
        r2 = run_gemm8(g["a"], g["w"], g["ws"], layout=layout)
        assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemm8_layouts_agree_bit_for_bit(M):
    g = inputs.make_gemm8(M, 2112, 7168, seed=180 + M)
    r0 = run_gemm8(g["a"], g["w"], g["ws"], layout=fq.W_ROW_MAJOR)
    r1 = run_gemm8(g["a"], g["w"], g["ws"], layout=fq.W_PRESHUFFLED)
    assert np.array_equal(r0.view(np.uint32), r1.view(np.uint32))


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8"])
def test_python_wrappers(orc, fmt):
    """prequant_gemm / preshuffle_weights allocate, check and call the C ABI:
    the same bits as the raw entry points, on a strided activation view."""
    M, N, K = 4, 64, 512
    g = (inputs.make_gemm if fmt == "mxfp4" else inputs.make_gemm8)(M, N, K, seed=190)
    a_full = dev(np.concatenate([g["a"], np.zeros((M, 64), np.uint16)], axis=1))
    a = a_full[:, :K]
    w, ws = dev(g["w"]), dev(g["ws"])
    r_plain = fq.prequant_gemm(a, w, ws, fmt=fmt)
    sw, sws = fq.preshuffle_weights(w, ws, fmt=fmt)
    r_shuf = fq.prequant_gemm(a, sw, sws, fmt=fmt, preshuffled=True)
    torch.cuda.synchronize()
    raw = (run_gemm if fmt == "mxfp4" else run_gemm8)(g["a"], g["w"], g["ws"])
    assert np.array_equal(host(r_plain).view(np.uint32), raw.view(np.uint32))
    assert np.array_equal(host(r_shuf).view(np.uint32), raw.view(np.uint32))
    with pytest.raises(ValueError):
        fq.prequant_gemm(a.float(), w, ws, fmt=fmt)


def test_gemm_random_shape_sweep(orc):
    """Seeded random shapes for both GEMMs and both weight layouts: M in
    1..80, N a multiple of 16 up to 640, K a multiple of 128 up to 2560,
    padded activation and output strides."""
    rng = np.random.default_rng(2024)
    for case in range(24):
        fmt = "mxfp4" if case % 2 == 0 else "fp8"
        M = int(rng.choice([1, 2, 3, 4, int(rng.integers(5, 81))]))
        N = 16 * int(rng.integers(1, 41))
        K = 128 * int(rng.integers(1, 21))
        layout = LAYOUTS[(case // 2) % 2]
        lda = K + 8 * int(rng.integers(0, 3))
        ldc = N + int(rng.integers(0, 5))
        if fmt == "mxfp4":
            g = inputs.make_gemm(M, N, K, seed=300 + case)
            got = run_gemm(g["a"], g["w"], g["ws"], lda=lda, ldc=ldc, layout=layout)
            check(orc, g["a"], g["w"], g["ws"], got)
        else:
            g = inputs.make_gemm8(M, N, K, seed=300 + case)
            got = run_gemm8(g["a"], g["w"], g["ws"], lda=lda, ldc=ldc, layout=layout)
            check8(orc, g["a"], g["w"], g["ws"], got)
