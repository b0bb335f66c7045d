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

# Shapes: the decode workload, activations staged in LDS (M <= 4, up to
# K = 8192 with 16 waves) and not (K = 8320 needs a 17th wave; M > 4), one to
# four row tiles, row blocks past 64, ragged M in every tile count, and two
# column tiles per staged workgroup (N/16 >= 256 and even; 4112 is odd).
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
    # the same groups in a staged (M <= 4) call
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
