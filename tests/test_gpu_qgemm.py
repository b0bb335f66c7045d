"""Parity of the GEMMs of already quantized activations (gemm_afp4wfp4,
gemm_a8w8_blockscale; through the C ABI) with the oracle.

The activations are codes and scales in each layout the group quantization
writes, made by the oracle's group quantization of seeded bf16 rows (so the
inputs never come from the GPU). The error bars are the prequant GEMMs':
K * 2^-23 * sum|products| for the fp32 sums, plus, for FP8, the matrix
cores' 8-product block truncation. With the same launch shape, the GEMM of
the group quantization of rows must equal the prequant GEMM of the rows bit
for bit, and the fused kernel's outputs feed it directly in every scale
layout.
"""
import numpy as np
import pytest
import torch

import fp4_quant_amd as fq
from fp4_quant_amd import inputs
from tests.gpu_util import dev, host, say
from tests.test_gpu_gemm import _abs_sum, _abs_sum8, _block8_bound, run_gemm, run_gemm8

pytestmark = pytest.mark.gpu

MX_LAYOUTS = [fq.SCALE_ROW_MAJOR, fq.SCALE_TILED32, fq.SCALE_COL_MAJOR]
FP8_LAYOUTS = [fq.SCALE_ROW_MAJOR, fq.SCALE_COL_MAJOR]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert fq.rmsq_device_supported(0), "GPU tests need a gfx950 device"


def run_qgemm(fmt, a_q, a_s, a_layout, w, ws, *, M, N, K, w_layout=fq.W_ROW_MAJOR, ldc=None):
    """One call through the C ABI with NaN guard bands around the output."""
    ldc = ldc or N
    dq, ds, dw, dws = dev(a_q), dev(a_s), dev(w), dev(ws)
    if w_layout == fq.W_PRESHUFFLED:
        sw = torch.empty_like(dw)
        if fmt == "mxfp4":
            sws = torch.empty_like(dws)
            fq.mxfp4_weight_preshuffle(dw, dws, N, K, sw, sws)
            dws = sws
        else:
            fq.fp8_weight_preshuffle(dw, N, K, sw)
        dw = sw
    guard = 1024
    out = torch.full((guard + max(M, 1) * ldc + guard,), float("nan"), dtype=torch.float32, device="cuda")
    say(f"qgemm {fmt} M={M} N={N} K={K} a_layout={a_layout} w_layout={w_layout} ldc={ldc}")
    call = fq.gemm_afp4wfp4 if fmt == "mxfp4" else fq.gemm_a8w8_blockscale
    call(dq, ds, a_layout, dw, dws, w_layout, M, N, K, out[guard:], ldc)
    torch.cuda.synchronize()
    o = host(out)
    assert np.all(np.isnan(o[:guard])) and np.all(np.isnan(o[guard + max(M, 1) * ldc:])), "guard band written"
    body = o[guard:guard + max(M, 1) * ldc].reshape(max(M, 1), ldc)
    if ldc > N:
        assert np.all(np.isnan(body[:M, N:])), "row padding written"
    return body[:M, :N]


def _within(got, want, bound):
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(np.isfinite(got))
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} outputs beyond the bound; worst excess {float((err - bound).max())}"


# decode, one to four row tiles of 16 (MXFP4) / one or two (FP8), several row
# blocks, a ragged last 32-row scale tile (37, 70, 130 rows), long K
# (two column tiles per workgroup above 64 rows when N/16 is even: 130 x 32, 200 x 96)
SHAPES = [(4, 2112, 7168), (1, 16, 128), (5, 32, 256), (16, 64, 384), (17, 32, 1024), (33, 48, 512),
          (37, 32, 256), (64, 32, 7168), (70, 16, 256), (130, 32, 640), (200, 96, 512), (4, 4096, 256),
          (4, 32, 8320)]
SHAPES8 = [(4, 2112, 7168), (1, 16, 128), (3, 32, 256), (5, 144, 384), (16, 64, 1024), (17, 32, 512),
           (33, 48, 256), (70, 16, 640), (4, 32, 8320)]


@pytest.mark.parametrize("a_layout", MX_LAYOUTS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_afp4wfp4_matches_oracle(orc, M, N, K, a_layout):
    g = inputs.make_gemm(M, N, K, seed=240 + M + K)
    qa, sa = orc.group_quant(g["a"], 32, 1, a_layout)
    got = run_qgemm("mxfp4", qa, sa, a_layout, g["w"], g["ws"], M=M, N=N, K=K,
                    w_layout=fq.W_PRESHUFFLED if (M + K) % 2 else fq.W_ROW_MAJOR)
    want = orc.gemm_afp4wfp4(qa, sa, g["w"], g["ws"], scale_layout=a_layout)
    _within(got, want, K * 2.0 ** -23 * _abs_sum(orc, g["a"], g["w"], g["ws"]))


@pytest.mark.parametrize("a_layout", FP8_LAYOUTS)
@pytest.mark.parametrize("M,N,K", SHAPES8)
def test_a8w8_blockscale_matches_oracle(orc, M, N, K, a_layout):
    g = inputs.make_gemm8(M, N, K, seed=340 + M + K)
    qa, sa = orc.group_quant(g["a"], 128, 0, a_layout)
    got = run_qgemm("fp8", qa, sa, a_layout, g["w"], g["ws"], M=M, N=N, K=K,
                    w_layout=fq.W_PRESHUFFLED if (M + K) % 2 else fq.W_ROW_MAJOR)
    want = orc.gemm_a8w8_blockscale(qa, sa, g["w"], g["ws"], scale_layout=a_layout)
    bound = K * 2.0 ** -23 * _abs_sum8(orc, g["a"], g["w"], g["ws"]) + _block8_bound(orc, g["a"], g["w"], g["ws"])
    _within(got, want, bound)


@pytest.mark.parametrize("M", [1, 4, 9, 16])
def test_afp4wfp4_of_the_group_quant_is_the_prequant_gemm_bit_for_bit(orc, M):
    """Up to 16 rows both GEMMs run 14 waves of 4 steps on the same operands
    in the same order (K = 7168)."""
    g = inputs.make_gemm(M, 2112, 7168, seed=440 + M)
    pre = run_gemm(g["a"], g["w"], g["ws"], layout=fq.W_PRESHUFFLED)
    for lay in MX_LAYOUTS:
        qa, sa = orc.group_quant(g["a"], 32, 1, lay)
        got = run_qgemm("mxfp4", qa, sa, lay, g["w"], g["ws"], M=M, N=2112, K=7168, w_layout=fq.W_PRESHUFFLED)
        assert np.array_equal(got.view(np.uint32), pre.view(np.uint32)), lay


@pytest.mark.parametrize("M", [1, 4])
def test_a8w8_of_the_group_quant_is_the_prequant_gemm_bit_for_bit(orc, M):
    g = inputs.make_gemm8(M, 2112, 7168, seed=460 + M)
    pre = run_gemm8(g["a"], g["w"], g["ws"], layout=fq.W_PRESHUFFLED)
    for lay in FP8_LAYOUTS:
        qa, sa = orc.group_quant(g["a"], 128, 0, lay)
        got = run_qgemm("fp8", qa, sa, lay, g["w"], g["ws"], M=M, N=2112, K=7168, w_layout=fq.W_PRESHUFFLED)
        assert np.array_equal(got.view(np.uint32), pre.view(np.uint32)), lay


def test_padded_output_rows_and_zero_rows(orc):
    g = inputs.make_gemm(20, 48, 256, seed=480)
    g["a"][3] = 0                                     # an all-zero row: scale byte 127, codes 0
    qa, sa = orc.group_quant(g["a"], 32, 1, fq.SCALE_TILED32)
    got = run_qgemm("mxfp4", qa, sa, fq.SCALE_TILED32, g["w"], g["ws"], M=20, N=48, K=256, ldc=56)
    want = orc.gemm_afp4wfp4(qa, sa, g["w"], g["ws"], scale_layout=fq.SCALE_TILED32)
    _within(got, want, 256 * 2.0 ** -23 * _abs_sum(orc, g["a"], g["w"], g["ws"]))
    assert np.all(got[3] == 0)


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8"])
def test_fused_kernel_outputs_feed_the_gemm_in_every_scale_layout(orc, fmt):
    """The fused residual + RMSNorm + quant (GPU) in each scale layout, then
    the GEMM of its codes and scales (GPU): equal to the prequant GEMM of the
    fused kernel's bf16 side-output (same launch shape, M = 4), and within
    the error bar of the oracle's chain (fused quantization, then GEMM)."""
    M, N, K = 4, 2112, 7168
    p = inputs.make_problem(M, K, seed_x=500, residual=True)
    g = inputs.make_gemm(M, N, K, seed=501) if fmt == "mxfp4" else inputs.make_gemm8(M, N, K, seed=501)
    x, r, gam = dev(p["x"]), dev(p["residual"]), dev(p["gamma"])
    dw, dws = dev(g["w"]), dev(g["ws"])
    f = 0 if fmt == "fp8" else 1
    for lay in (MX_LAYOUTS if fmt == "mxfp4" else FP8_LAYOUTS):
        q, sc, yb = fq.alloc_outputs(M, K, f, lay, keep_bf16=True)
        ro = torch.empty_like(r)
        say(f"fused {fmt} layout={lay} then GEMM")
        fq.rmsnorm_quant_group_multi(fq.problem_array([fq.make_problem(
            x, gam, p["eps"], q, sc, residual_in=r, residual_out=ro, out_bf16=yb, fmt=f, scale_layout=lay)]))
        out_q = torch.empty((M, N), dtype=torch.float32, device="cuda")
        out_p = torch.empty((M, N), dtype=torch.float32, device="cuda")
        if fmt == "mxfp4":
            fq.gemm_afp4wfp4(q, sc, lay, dw, dws, fq.W_ROW_MAJOR, M, N, K, out_q, N)
            fq.gemm_a16wfp4_prequant(yb, K, dw, dws, fq.W_ROW_MAJOR, M, N, K, out_p, N)
        else:
            fq.gemm_a8w8_blockscale(q, sc, lay, dw, dws, fq.W_ROW_MAJOR, M, N, K, out_q, N)
            fq.gemm_a16w8_prequant(yb, K, dw, dws, fq.W_ROW_MAJOR, M, N, K, out_p, N)
        torch.cuda.synchronize()
        got, pre = host(out_q), host(out_p)
        assert np.array_equal(got.view(np.uint32), pre.view(np.uint32)), lay
        o = orc.rmsnorm_quant_group(p["x"], p["gamma"], p["eps"], residual=p["residual"],
                                    group=32 if fmt == "mxfp4" else 128, fmt=f, scale_layout=lay, keep_bf16=True)
        if fmt == "mxfp4":
            want = orc.gemm_afp4wfp4(o["q"], o["scale"], g["w"], g["ws"], scale_layout=lay)
            _within(got, want, K * 2.0 ** -23 * _abs_sum(orc, o["bf16"], g["w"], g["ws"]))
        else:
            want = orc.gemm_a8w8_blockscale(o["q"], o["scale"], g["w"], g["ws"], scale_layout=lay)
            _within(got, want, K * 2.0 ** -23 * _abs_sum8(orc, o["bf16"], g["w"], g["ws"]) +
                    _block8_bound(orc, o["bf16"], g["w"], g["ws"]))


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8"])
def test_python_wrapper(orc, fmt):
    M, N, K = 3, 64, 512
    g = inputs.make_gemm(M, N, K, seed=520) if fmt == "mxfp4" else inputs.make_gemm8(M, N, K, seed=520)
    lay = fq.SCALE_COL_MAJOR
    qa, sa = orc.group_quant(g["a"], 32 if fmt == "mxfp4" else 128, 1 if fmt == "mxfp4" else 0, lay)
    w, ws = fq.preshuffle_weights(dev(g["w"]), dev(g["ws"]), fmt)
    got = host(fq.quantized_gemm(dev(qa), dev(sa), w, ws, fmt=fmt, scale_layout=lay, preshuffled=True))
    if fmt == "mxfp4":
        _within(got, orc.gemm_afp4wfp4(qa, sa, g["w"], g["ws"], scale_layout=lay),
                K * 2.0 ** -23 * _abs_sum(orc, g["a"], g["w"], g["ws"]))
    else:
        _within(got, orc.gemm_a8w8_blockscale(qa, sa, g["w"], g["ws"], scale_layout=lay),
                K * 2.0 ** -23 * _abs_sum8(orc, g["a"], g["w"], g["ws"]) + _block8_bound(orc, g["a"], g["w"], g["ws"]))
    with pytest.raises(ValueError):
        fq.quantized_gemm(dev(qa), dev(sa), w, ws, fmt="int4")
