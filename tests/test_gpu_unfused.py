"""Parity of the unfused pair (add_rmsnorm, then dynamic_per_group_scaled_quant)
with the oracle's two stages, and of their composition with the fused call,
bit for bit, through the C ABI."""
import numpy as np
import pytest
import torch

import fp4_quant_amd as fq
from fp4_quant_amd import inputs
from tests.gpu_util import compare, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert fq.rmsq_device_supported(0), "GPU tests need a gfx950 device"


def _norm_gpu(p):
    M, N = p["x"].shape
    x, g = dev(p["x"]), dev(p["gamma"])
    r = dev(p["residual"]) if "residual" in p else None
    ro = torch.full_like(r, 7.0) if r is not None else None
    yb = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    fq.add_rmsnorm(x, r, g, p["eps"], M, N, ro, yb)
    torch.cuda.synchronize()
    return (host(ro) if ro is not None else None), host(yb)


def _quant_gpu(yb_bits, fmt, layout):
    M, N = yb_bits.shape
    q, sc, _ = fq.alloc_outputs(M, N, fmt, layout)
    sc.view(torch.uint8).fill_(0xA5)
    fq.dynamic_per_group_scaled_quant(dev(yb_bits), M, N, 128 if fmt == 0 else 32, fmt, layout, q, sc)
    torch.cuda.synchronize()
    return host(q), host(sc)


@pytest.mark.parametrize("name", ["decode", "prefill", "mxfp4"])
def test_add_rmsnorm_matches_oracle_stage(orc, name):
    say(f"add_rmsnorm {name}")
    c = inputs.make_config(name)
    h, yb = _norm_gpu(c)
    wh, wyb = orc.add_rmsnorm(c["x"], c["gamma"], c["eps"], residual=c.get("residual"))
    assert np.array_equal(yb, wyb)
    if h is not None:
        assert np.array_equal(h, wh)


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("N, M", [(512, 1), (512, 1024), (7168, 1), (7168, 64)])
def test_add_rmsnorm_window_side_values(orc, N, M, sign):
    """The norm alone on rows whose fp32 products land on the midpoint
    window's side value and round the other way (built as in the fused
    parity tests): the bf16 output still equals the oracle's."""
    from tests.test_gpu_parity import side_crossing_row
    say(f"add_rmsnorm window side values N={N} M={M} sign={sign}")
    x, g, eps, _, _ = side_crossing_row(N, sign, 500 + N + (sign > 0))
    p = {"x": np.repeat(x[None, :], M, axis=0), "gamma": g, "eps": eps}
    _, yb = _norm_gpu(p)
    _, wyb = orc.add_rmsnorm(p["x"], g, eps)
    assert np.array_equal(yb, wyb)


@pytest.mark.parametrize("fmt,layout", [(0, 0), (1, 0), (1, 1), (0, 2), (1, 2)])
def test_group_quant_matches_oracle_stage(orc, fmt, layout):
    say(f"dynamic_per_group_scaled_quant fmt {fmt} layout {layout}")
    c = inputs.make_config("prefill" if fmt == 0 else "mxfp4")
    _, yb = orc.add_rmsnorm(c["x"], c["gamma"], c["eps"], residual=c.get("residual"))
    q, sc = _quant_gpu(yb, fmt, layout)
    wq, wsc = orc.group_quant(yb, 128 if fmt == 0 else 32, fmt, layout, scale_fill=0xA5)
    sc = sc.reshape(wsc.shape)
    assert np.array_equal(sc.view(np.uint8), wsc.view(np.uint8))
    if layout == 2:
        sc, wsc = sc.T.copy(), wsc.T.copy()
    compare({"q": q, "scale": sc}, {"q": wq, "scale": wsc}, fmt, (orc.e4m3fn_table(), orc.e2m1_table()),
            strict=True, yb_ref=yb)


@pytest.mark.parametrize("N", [128, 256, 384, 1536, 7168, 16384, 32768])
def test_pair_equals_fused_on_the_gpu(N):
    """add_rmsnorm then the quant kernel gives the fused call's bytes."""
    say(f"pair == fused, N {N}")
    p = inputs.make_problem(37, N, seed_x=400 + N, residual=True, outliers=True)
    h, yb = _norm_gpu(p)
    for fmt in (0, 1):
        q, sc = _quant_gpu(yb, fmt, 0)
        x, g, r = dev(p["x"]), dev(p["gamma"]), dev(p["residual"])
        (fyb, fq_, fsc), fh = fq.fused_rmsnorm_quant(x, g, p["eps"], residual=r, fmt="fp8" if fmt == 0 else "mxfp4",
                                                   keep_bf16=True)
        torch.cuda.synchronize()
        assert np.array_equal(host(fh), h) and np.array_equal(host(fyb), yb)
        assert np.array_equal(host(fq_), q) and np.array_equal(host(fsc).reshape(-1), sc.reshape(-1))


def test_group_quant_ragged_and_edge_rows(orc):
    say("quant kernel edge rows")
    N = 512
    y = np.random.default_rng(3).standard_normal((9, N)).astype(np.float32)
    y[0] = 0.0
    y[1, :128] = 0.0
    y[2] *= np.float32(1e-36)
    y[3, ::2] = -0.0
    yb = inputs.to_bf16_bits(y)
    for fmt, layout in ((0, 0), (1, 0), (1, 1), (0, 2), (1, 2)):
        q, sc = _quant_gpu(yb, fmt, layout)
        wq, wsc = orc.group_quant(yb, 128 if fmt == 0 else 32, fmt, layout, scale_fill=0xA5)
        assert np.array_equal(sc.view(np.uint8).reshape(-1), wsc.view(np.uint8).reshape(-1))
        tab = orc.e4m3fn_table() if fmt == 0 else orc.e2m1_table()
        if fmt == 0:
            assert np.array_equal(tab[q], tab[wq])
        else:
            assert np.array_equal(tab[q & 0xF], tab[wq & 0xF]) and np.array_equal(tab[q >> 4], tab[wq >> 4])
