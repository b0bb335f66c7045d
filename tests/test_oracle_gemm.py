"""Pins for the oracle's GEMMs (CPU only): the prequant GEMMs and the GEMMs of
already quantized activations.

The expected values come from the definitions, not from the oracle: the e2m1
grid and the e8m0 scale are written out here, numpy's matmul does the
contraction, and the activation quantization is either avoided (inputs that
MXFP4 represents exactly, so quantizing is the identity) or taken from the
oracle's group quantization, which test_oracle_codecs and
test_oracle_pipeline pin on their own.
"""
import numpy as np
import pytest

from fp4_quant_amd import inputs

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])


def bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def dequant_rows(codes, scales):
    """[R, K/2] e2m1 codes (element 2k low nibble) and [R, K/32] e8m0 bytes -> [R, K] float64."""
    lo, hi = codes & 0xF, codes >> 4
    q = np.stack([E2M1[lo], E2M1[hi]], -1).reshape(codes.shape[0], -1)
    return q * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)


def random_weights(N, K, seed):
    rng = np.random.default_rng(seed)
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = rng.integers(118, 134, (N, K // 32)).astype(np.uint8)
    return w, ws


def test_hand_example(orc):
    # 32 ones then 32 twos: group scales 2^-2 and 2^-1, codes 4.0 -> exact; weights all 1.0
    a = np.array([[0x3F80] * 32 + [0x4000] * 32], np.uint16)
    w = np.full((2, 32), 0x22, np.uint8)
    ws = np.full((2, 2), 127, np.uint8)
    assert orc.gemm_a16wfp4_prequant(a, w, ws).tolist() == [[96.0, 96.0]]
    ws[1, 1] = 128                                   # second weight row's second group scaled by 2
    assert orc.gemm_a16wfp4_prequant(a, w, ws).tolist() == [[96.0, 32.0 + 128.0]]


def test_lossless_activations_match_numpy_matmul(orc):
    """Activations built from e2m1 codes times a power of two per 32-group,
    with a largest code of 4 or 6 in every group, are exactly MXFP4 values
    (the scale rule picks the same power of two), so the GEMM is
    A @ dequant(W)^T, computed here by numpy."""
    rng = np.random.default_rng(5)
    M, N, K = 7, 9, 256
    codes = rng.integers(0, 16, (M, K))
    codes[:, ::32] = rng.choice([6, 7, 14, 15], (M, K // 32))   # the group max: 4 or 6 in magnitude
    e = rng.integers(-20, 20, (M, K // 32))
    A = E2M1[codes] * np.repeat(np.ldexp(1.0, e), 32, axis=1)
    a = inputs.to_bf16_bits(A.astype(np.float32))
    assert np.array_equal(bf16_to_f32(a).astype(np.float64), A)
    w, ws = random_weights(N, K, 6)
    want = A @ dequant_rows(w, ws).T
    got = orc.gemm_a16wfp4_prequant(a, w, ws)
    assert np.allclose(got, want, rtol=1e-12, atol=0)


def test_equals_its_own_quantization_times_the_weights(orc):
    """On general bf16 rows the GEMM equals (the activations' MXFP4 group
    quantization, dequantized) @ dequant(W)^T."""
    p = inputs.make_problem(5, 512, seed_x=30, residual=False, outliers=True)
    w, ws = random_weights(11, 512, 7)
    qa, sa = orc.group_quant(p["x"], 32, 1, 0)
    want = dequant_rows(qa, sa) @ dequant_rows(w, ws).T
    got = orc.gemm_a16wfp4_prequant(p["x"], w, ws)
    assert np.allclose(got, want, rtol=1e-12, atol=0)


@pytest.mark.parametrize("k", [-7, 3])
def test_power_of_two_scaling(orc, k):
    """Scaling the activations by 2^k scales every output by 2^k exactly (the
    group scales absorb it); raising every weight scale byte by k does too."""
    p = inputs.make_problem(3, 256, seed_x=31, residual=False, outliers=True)
    w, ws = random_weights(4, 256, 8)
    base = orc.gemm_a16wfp4_prequant(p["x"], w, ws)
    xs = inputs.to_bf16_bits(bf16_to_f32(p["x"]) * np.float32(2.0 ** k))
    assert np.array_equal(orc.gemm_a16wfp4_prequant(xs, w, ws), base * 2.0 ** k)
    assert np.array_equal(orc.gemm_a16wfp4_prequant(p["x"], w, (ws.astype(int) + k).astype(np.uint8)),
                          base * 2.0 ** k)


def test_strided_rows_and_zero_rows(orc):
    p = inputs.make_problem(4, 256, seed_x=32, residual=False, outliers=False)
    w, ws = random_weights(5, 256, 9)
    wide = np.zeros((4, 384), np.uint16)
    wide[:, :256] = p["x"]
    wide[1, :256] = 0                                # an all-zero row: scale byte 127, codes 0
    x = p["x"].copy()
    x[1] = 0
    got = orc.gemm_a16wfp4_prequant(wide[:, :256], w, ws)
    assert np.array_equal(got, orc.gemm_a16wfp4_prequant(x, w, ws))
    assert np.all(got[1] == 0)


def test_rejects_undefined_shapes(orc):
    a = np.zeros((2, 48), np.uint16)
    with pytest.raises((ValueError, AssertionError)):
        orc.gemm_a16wfp4_prequant(a, np.zeros((3, 24), np.uint8), np.zeros((3, 1), np.uint8))


# ------------------------------------------------------------------ A16W8 --
def e4m3_values(codes):
    """e4m3fn bytes -> float64 through torch's own float8_e4m3fn dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def dequant_fp8_weights(w, ws):
    """[N, K] e4m3fn codes with [ceil(N/128), K/128] fp32 block scales -> [N, K] float64."""
    N, K = w.shape
    s = np.repeat(np.repeat(ws.astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    return e4m3_values(w) * s


def random_fp8_weights(N, K, seed):
    rng = np.random.default_rng(seed)
    w = rng.integers(0, 256, (N, K), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x7E                    # no NaN codes
    ws = rng.uniform(2.0 ** -12, 2.0 ** -6, (-(-N // 128), K // 128)).astype(np.float32)
    return w, ws


def test_a16w8_hand_example(orc):
    # 128 x 448 then 128 x 224: group scales 1 and 0.5 exactly, codes 448 -> exact; weights 1.0 (0x38)
    a = np.array([[0x43E0] * 128 + [0x4360] * 128], np.uint16)
    w = np.full((2, 256), 0x38, np.uint8)
    ws = np.ones((1, 2), np.float32)
    assert orc.gemm_a16w8_prequant(a, w, ws).tolist() == [[128 * 448.0 + 128 * 224.0] * 2]
    ws[0, 1] = 4.0                                   # second K block of the weights scaled by 4
    assert orc.gemm_a16w8_prequant(a, w, ws).tolist() == [[128 * 448.0 + 4 * 128 * 224.0] * 2]


def test_a16w8_lossless_activations_match_numpy_matmul(orc):
    """Activations built from e4m3fn values times a power of two per 128-group,
    with +-448 in every group, are exactly FP8 values (the scale is that power
    of two), so the GEMM is A @ dequant(W)^T, computed here by numpy. N = 200
    spans two 128-row weight blocks, K = 384 three K blocks."""
    rng = np.random.default_rng(15)
    M, N, K = 6, 200, 384
    codes = rng.integers(0, 256, (M, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    codes[:, ::128] = rng.choice([0x7E, 0xFE], (M, K // 128))   # +-448 in every group
    e = rng.integers(-20, 20, (M, K // 128))
    A = e4m3_values(codes) * np.repeat(np.ldexp(1.0, e), 128, axis=1)
    a = inputs.to_bf16_bits(A.astype(np.float32))
    assert np.array_equal(bf16_to_f32(a).astype(np.float64), A)
    w, ws = random_fp8_weights(N, K, 16)
    want = A @ dequant_fp8_weights(w, ws).T
    got = orc.gemm_a16w8_prequant(a, w, ws)
    assert np.allclose(got, want, rtol=1e-12, atol=0)


def test_a16w8_equals_its_own_quantization_times_the_weights(orc):
    """On general bf16 rows the GEMM equals (the activations' FP8 group
    quantization, dequantized) @ dequant(W)^T."""
    p = inputs.make_problem(5, 512, seed_x=33, residual=False, outliers=True)
    w, ws = random_fp8_weights(136, 512, 17)
    qa, sa = orc.group_quant(p["x"], 128, 0, 0)
    da = e4m3_values(qa) * np.repeat(sa.reshape(5, -1).astype(np.float64), 128, axis=1)
    want = da @ dequant_fp8_weights(w, ws).T
    got = orc.gemm_a16w8_prequant(p["x"], w, ws)
    assert np.allclose(got, want, rtol=1e-12, atol=0)


@pytest.mark.parametrize("k", [-7, 3])
def test_a16w8_power_of_two_scaling(orc, k):
    """Scaling the activations by 2^k scales every output by 2^k exactly (the
    fp32 group scales absorb it); scaling every weight block scale too."""
    p = inputs.make_problem(3, 256, seed_x=34, residual=False, outliers=True)
    w, ws = random_fp8_weights(20, 256, 18)
    base = orc.gemm_a16w8_prequant(p["x"], w, ws)
    xs = inputs.to_bf16_bits(bf16_to_f32(p["x"]) * np.float32(2.0 ** k))
    assert np.array_equal(orc.gemm_a16w8_prequant(xs, w, ws), base * 2.0 ** k)
    assert np.array_equal(orc.gemm_a16w8_prequant(p["x"], w, ws * np.float32(2.0 ** k)), base * 2.0 ** k)


def test_a16w8_rejects_undefined_shapes(orc):
    a = np.zeros((2, 192), np.uint16)
    with pytest.raises((ValueError, AssertionError)):
        orc.gemm_a16w8_prequant(a, np.zeros((3, 192), np.uint8), np.zeros((1, 1), np.float32))


# ------------------------------------------- GEMMs of quantized activations --
def layout_scales(S, layout):
    """A [M, G] scale matrix as the group quantization lays it out, built with
    numpy reshapes: row-major as is; 32-row tiles (rows padded to a multiple
    of 32, group-major inside a tile, the tile's 32 rows adjacent);
    column-major [G, M]."""
    if layout == 0:
        return np.ascontiguousarray(S)
    if layout == 2:
        return np.ascontiguousarray(S.T)
    M, G = S.shape
    Mp = -(-M // 32) * 32
    P = np.zeros((Mp, G), S.dtype)
    P[:M] = S
    return np.ascontiguousarray(P.reshape(Mp // 32, 32, G).transpose(0, 2, 1)).reshape(-1)


def test_afp4wfp4_hand_example(orc):
    # one row: 32 ones (scale byte 127) then 32 twos (codes 1.0, scale byte 128); weights all 1.0
    a_q = np.full((1, 32), 0x22, np.uint8)
    a_s = np.array([[127, 128]], np.uint8)
    w = np.full((2, 32), 0x22, np.uint8)
    ws = np.full((2, 2), 127, np.uint8)
    assert orc.gemm_afp4wfp4(a_q, a_s, w, ws).tolist() == [[96.0, 96.0]]
    ws[1, 0] = 126                                   # second weight row's first group halved
    assert orc.gemm_afp4wfp4(a_q, a_s, w, ws).tolist() == [[96.0, 16.0 + 64.0]]


@pytest.mark.parametrize("layout", [0, 1, 2])
def test_afp4wfp4_matches_numpy_dequant_matmul(orc, layout):
    """Random activation codes and scale bytes, the scales in each layout: the
    GEMM is dequant(A) @ dequant(W)^T, computed here by numpy. 37 rows: a
    ragged last 32-row tile."""
    rng = np.random.default_rng(41)
    M, N, K = 37, 9, 256
    a_q = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    S = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    w, ws = random_weights(N, K, 42)
    want = dequant_rows(a_q, S) @ dequant_rows(w, ws).T
    got = orc.gemm_afp4wfp4(a_q, layout_scales(S, layout), w, ws, scale_layout=layout)
    assert np.allclose(got, want, rtol=1e-12, atol=0)


@pytest.mark.parametrize("layout", [0, 1, 2])
def test_afp4wfp4_of_the_group_quant_is_the_prequant_gemm(orc, layout):
    """Quantizing bf16 rows with the group quantization (in any scale layout)
    and multiplying the result gives exactly the prequant GEMM of the rows."""
    p = inputs.make_problem(35, 256, seed_x=43, residual=False, outliers=True)
    w, ws = random_weights(7, 256, 44)
    qa, sa = orc.group_quant(p["x"], 32, 1, layout)
    assert np.array_equal(orc.gemm_afp4wfp4(qa, sa, w, ws, scale_layout=layout),
                          orc.gemm_a16wfp4_prequant(p["x"], w, ws))


def test_a8w8_hand_example(orc):
    # one row of 256: codes 1.0 (0x38) with scales 2 and 0.25; weights 1.0, block scales 1 and 3
    a_q = np.full((1, 256), 0x38, np.uint8)
    a_s = np.array([[2.0, 0.25]], np.float32)
    w = np.full((2, 256), 0x38, np.uint8)
    ws = np.array([[1.0, 3.0]], np.float32)
    assert orc.gemm_a8w8_blockscale(a_q, a_s, w, ws).tolist() == [[128 * 2.0 + 128 * 0.75] * 2]


@pytest.mark.parametrize("layout", [0, 2])
def test_a8w8_matches_numpy_dequant_matmul(orc, layout):
    """Random e4m3fn activation codes and fp32 group scales (row- or
    column-major): the GEMM is dequant(A) @ dequant(W)^T by numpy. N = 200
    spans two 128-row weight blocks, K = 384 three K blocks."""
    rng = np.random.default_rng(45)
    M, N, K = 6, 200, 384
    a_q = rng.integers(0, 256, (M, K), dtype=np.uint8)
    a_q[(a_q & 0x7F) == 0x7F] = 0x7E
    S = rng.uniform(2.0 ** -10, 2.0 ** 3, (M, K // 128)).astype(np.float32)
    w, ws = random_fp8_weights(N, K, 46)
    A = e4m3_values(a_q) * np.repeat(S.astype(np.float64), 128, axis=1)
    want = A @ dequant_fp8_weights(w, ws).T
    got = orc.gemm_a8w8_blockscale(a_q, layout_scales(S, layout), w, ws, scale_layout=layout)
    assert np.allclose(got, want, rtol=1e-12, atol=0)


@pytest.mark.parametrize("layout", [0, 2])
def test_a8w8_of_the_group_quant_is_the_prequant_gemm(orc, layout):
    p = inputs.make_problem(5, 512, seed_x=47, residual=False, outliers=True)
    w, ws = random_fp8_weights(136, 512, 48)
    qa, sa = orc.group_quant(p["x"], 128, 0, layout)
    assert np.array_equal(orc.gemm_a8w8_blockscale(qa, sa, w, ws, scale_layout=layout),
                          orc.gemm_a16w8_prequant(p["x"], w, ws))


def test_quantized_activation_gemms_reject_undefined_arguments(orc):
    with pytest.raises((ValueError, AssertionError)):      # K not a multiple of 32
        orc.gemm_afp4wfp4(np.zeros((2, 24), np.uint8), np.zeros((2, 1), np.uint8),
                          np.zeros((3, 24), np.uint8), np.zeros((3, 1), np.uint8))
    with pytest.raises(ValueError):                        # FP8 scales have no 32-row tiled layout
        orc.gemm_a8w8_blockscale(np.zeros((2, 128), np.uint8), np.ones(64, np.float32), np.zeros((3, 128), np.uint8),
                                 np.ones((1, 1), np.float32), scale_layout=1)
    assert orc.gemm_afp4wfp4(np.zeros((0, 32), np.uint8), np.zeros((0, 2), np.uint8), np.zeros((3, 32), np.uint8),
                             np.zeros((3, 2), np.uint8)).shape == (0, 3)
