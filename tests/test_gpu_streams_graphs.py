"""The fused call on non-default streams, from several host threads at once,
and captured in a HIP graph: every result equals the eager, default-stream
result bit for bit. (The library allocates nothing and issues no memsets, so
a captured launch is a single kernel node.)"""
import threading

import numpy as np
import pytest
import torch

import fp4_quant_amd as fq
from fp4_quant_amd import inputs
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert fq.rmsq_device_supported(0), "GPU tests need a gfx950 device"


def _buffers(p, fmt=0):
    M, N = p["x"].shape
    x, g, r = dev(p["x"]), dev(p["gamma"]), dev(p["residual"])
    ro = torch.zeros_like(r)
    q, sc, yb = fq.alloc_outputs(M, N, fmt, 0, True)
    for t in (q, sc, yb):
        t.zero_()
    prob = fq.make_problem(x, g, p["eps"], q, sc, residual_in=r, residual_out=ro, out_bf16=yb, fmt=fmt)
    return prob, (x, g, r, ro, q, sc, yb)


def _snapshot(bufs):
    return [host(t).copy() for t in bufs[3:]]


def test_non_default_stream_matches_default():
    say("non-default stream")
    p = inputs.make_problem(256, 7168, seed_x=71, residual=True, outliers=True)
    prob, bufs = _buffers(p)
    fq.rmsnorm_quant_group_multi([prob])
    torch.cuda.synchronize()
    want = _snapshot(bufs)
    for t in bufs[3:]:
        t.zero_()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fq.rmsnorm_quant_group_multi([prob])          # picks up the current (side) stream
    s.synchronize()
    for a, b in zip(_snapshot(bufs), want):
        assert np.array_equal(a, b)


def test_concurrent_host_threads_on_their_own_streams():
    say("4 host threads, 4 streams")
    probs = [inputs.make_problem(128, 7168, seed_x=80 + i, residual=True, outliers=True) for i in range(4)]
    sets = [_buffers(p, fmt=i % 2) for i, p in enumerate(probs)]
    for prob, _ in sets:
        fq.rmsnorm_quant_group_multi([prob])
    torch.cuda.synchronize()
    want = [_snapshot(b) for _, b in sets]
    for _, b in sets:
        for t in b[3:]:
            t.zero_()
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(20):
                    fq.rmsnorm_quant_group_multi([sets[i][0]])
            s.synchronize()
        except Exception as e:   # reported below
            errors.append(e)

    th = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (_, b), w in zip(sets, want):
        for a, c in zip(_snapshot(b), w):
            assert np.array_equal(a, c)


def test_graph_capture_and_replay():
    say("HIP graph capture / replay")
    pa = inputs.make_problem(512, 7168, seed_x=90, residual=True, outliers=True)
    pb = inputs.make_problem(512, 7168, seed_x=91, residual=True, outliers=True)
    prob, bufs = _buffers(pa)
    x, g, r = bufs[0], bufs[1], bufs[2]
    xa, ra = x.clone(), r.clone()
    xb, rb = dev(pb["x"]), dev(pb["residual"])

    def eager(xs, rs):
        x.copy_(xs)
        r.copy_(rs)
        fq.rmsnorm_quant_group_multi([prob])
        torch.cuda.synchronize()
        return _snapshot(bufs)

    want_a, want_b = eager(xa, ra), eager(xb, rb)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fq.rmsnorm_quant_group_multi([prob])          # warm-up on the capture stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        fq.rmsnorm_quant_group_multi([prob])
    for k in range(6):
        xs, rs, want = (xa, ra, want_a) if k % 2 == 0 else (xb, rb, want_b)
        x.copy_(xs)
        r.copy_(rs)
        for t in bufs[3:]:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, c in zip(_snapshot(bufs), want):
            assert np.array_equal(a, c), f"replay {k}"
        _ = (x.float() * 2).sum().item()              # eager work between replays


def test_graph_capture_of_a_mixed_set_two_launches(orc):
    """A multi-problem set mixing problems with and without a residual is
    enqueued as two launches; captured in a graph, every replay matches the
    oracle."""
    from tests.test_gpu_parity import run_oracle
    say("HIP graph capture of a mixed multi-problem set")
    pa = inputs.make_problem(96, 7168, seed_x=93, residual=True, outliers=True)
    pb = inputs.make_problem(1100, 1536, seed_x=94, residual=False, outliers=False)
    prob_a, bufs_a = _buffers(pa)
    xb, gb = dev(pb["x"]), dev(pb["gamma"])
    qb, sb, yb = fq.alloc_outputs(1100, 1536, 0, 0, True)
    prob_b = fq.make_problem(xb, gb, pb["eps"], qb, sb, out_bf16=yb)
    arr = fq.problem_array([prob_a, prob_b])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fq.rmsnorm_quant_group_multi(arr)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        fq.rmsnorm_quant_group_multi(arr)
    wa = run_oracle(orc, dict(pa, fmt=0))
    wb = run_oracle(orc, dict(pb, fmt=0))
    for k in range(3):
        for t in list(bufs_a[3:]) + [qb, sb, yb]:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ro, q, sc, ybo = (host(t) for t in bufs_a[3:])
        assert np.array_equal(ro, wa["residual_out"]), k
        assert np.array_equal(ybo, wa["bf16"]) and np.array_equal(q, wa["q"]), k
        assert np.array_equal(sc.reshape(-1).view(np.uint32), wa["scale"].reshape(-1).view(np.uint32)), k
        assert np.array_equal(host(yb), wb["bf16"]) and np.array_equal(host(qb), wb["q"]), k
        assert np.array_equal(host(sb).reshape(-1).view(np.uint32), wb["scale"].reshape(-1).view(np.uint32)), k
        _ = (xb.float() * 2).sum().item()              # eager work between replays


@pytest.mark.parametrize("fmt", [1, 0])
def test_graph_capture_of_the_prequant_gemms(fmt):
    """Both prequant GEMMs (preshuffled weights, the small-M path at M = 4
    and per-wave activations at M = 20) captured in one HIP graph: each
    replay, with new activations copied in and eager work between replays,
    equals the eager result bit for bit."""
    say(f"HIP graph capture of the prequant GEMM (fmt {fmt})")
    N, K = 2112, 7168
    mk = inputs.make_gemm if fmt == 1 else inputs.make_gemm8
    call = fq.gemm_a16wfp4_prequant if fmt == 1 else fq.gemm_a16w8_prequant
    g = mk(20, N, K, seed=95)
    w, ws = dev(g["w"]), dev(g["ws"])
    sw = torch.empty_like(w)
    if fmt == 1:
        sws = torch.empty_like(ws)
        fq.mxfp4_weight_preshuffle(w, ws, N, K, sw, sws)
    else:
        sws = ws
        fq.fp8_weight_preshuffle(w, N, K, sw)
    a = dev(g["a"])
    a_alt = dev(mk(20, N, K, seed=96)["a"])
    a_in = a.clone()
    outs = [torch.zeros((M, N), dtype=torch.float32, device="cuda") for M in (4, 20)]

    def launch():
        for o in outs:
            M = o.shape[0]
            call(a_in, K, sw, sws, fq.W_PRESHUFFLED, M, N, K, o, N)

    def eager(src):
        a_in.copy_(src)
        launch()
        torch.cuda.synchronize()
        return [host(o).copy() for o in outs]

    want = [eager(a), eager(a_alt)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        launch()
    for k in range(6):
        a_in.copy_(a if k % 2 == 0 else a_alt)
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, exp in zip([host(o) for o in outs], want[k % 2]):
            assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), f"replay {k}"
        _ = (a_in.float() * 2).sum().item()


@pytest.mark.parametrize("fmt", [1, 0])
def test_graph_capture_of_norm_quant_then_gemm(fmt):
    """The fused residual + RMSNorm + group quant feeding the GEMM of its
    quantized activations (32 rows: 32-row tiled MXFP4 scales, column-major
    FP8 scales), captured in one HIP graph: every replay, with new inputs
    copied in and eager work between replays, equals the eager result bit for
    bit (output, residual, codes and scales)."""
    say(f"HIP graph capture of norm + quant then GEMM (fmt {fmt})")
    M, N, K = 32, 2112, 7168
    lay = fq.SCALE_TILED32 if fmt == 1 else fq.SCALE_COL_MAJOR
    g = inputs.make_gemm(M, N, K, seed=97) if fmt == 1 else inputs.make_gemm8(M, N, K, seed=97)
    w, ws = dev(g["w"]), dev(g["ws"])
    sw = torch.empty_like(w)
    if fmt == 1:
        sws = torch.empty_like(ws)
        fq.mxfp4_weight_preshuffle(w, ws, N, K, sw, sws)
    else:
        sws = ws
        fq.fp8_weight_preshuffle(w, N, K, sw)
    srcs = [inputs.make_problem(M, K, seed_x=s, residual=True) for s in (98, 99)]
    x, r = dev(srcs[0]["x"]), dev(srcs[0]["residual"])
    gam = dev(srcs[0]["gamma"])
    ro = torch.empty_like(r)
    q, sc, _ = fq.alloc_outputs(M, K, fmt, lay)
    out = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    probs = fq.problem_array([fq.make_problem(x, gam, 1e-6, q, sc, residual_in=r, residual_out=ro, fmt=fmt,
                                              scale_layout=lay)])
    gemm = fq.gemm_afp4wfp4 if fmt == 1 else fq.gemm_a8w8_blockscale

    def launch(stream=None):
        st = stream.cuda_stream if stream is not None else None
        fq.rmsnorm_quant_group_multi(probs, st)
        gemm(q, sc, lay, sw, sws, fq.W_PRESHUFFLED, M, N, K, out, N, st)

    def load(k):
        x.copy_(dev(srcs[k]["x"]))
        r.copy_(dev(srcs[k]["residual"]))

    def snap():
        return [host(t).copy() for t in (out, ro, q, sc)]

    want = []
    for k in range(2):
        load(k)
        launch()
        torch.cuda.synchronize()
        want.append(snap())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        launch(s)
    for k in range(6):
        load(k % 2)
        for t in (out, ro, q, sc):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, exp in zip(snap(), want[k % 2]):
            assert np.array_equal(got.view(np.uint8), exp.view(np.uint8)), f"replay {k}"
        _ = (x.float() * 2).sum().item()
