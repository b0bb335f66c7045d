"""The benchmark's host-side accounting (CPU only): algorithmic bytes per
workload, the GEMMs' bytes, the traffic record's source-hash gate, and the
one-GPU contract."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fused_algorithmic_bytes_per_row():
    # per row of 7168: x 2 B + residual 2 B read, residual 2 B + bf16 2 B + code 1 B written
    # per element, plus 56 fp32 scales (FP8) or 224 e8m0 bytes (MXFP4)
    assert bench.algorithmic_bytes(1, 7168, 0, True, True) == 7168 * 9 + 56 * 4 == 64736
    assert bench.algorithmic_bytes(1, 7168, 0, True, False) == 7168 * 7 + 56 * 4 == 50400
    assert bench.algorithmic_bytes(1, 7168, 0, False, False) == 7168 * 3 + 56 * 4 == 21728
    assert bench.algorithmic_bytes(1, 7168, 1, True, False) == 7168 * 6 + 7168 // 2 + 224 == 46816
    assert bench.algorithmic_bytes(8192, 7168, 0, True, True) == 8192 * 64736 == 530317312


def test_gemm_bytes_of_the_decode_workloads():
    M, N, K = 4, 2112, 7168
    w4 = N * K // 2 + N * K // 32            # e2m1 codes + e8m0 scales
    w8 = N * K + 17 * 56 * 4                 # e4m3fn codes + fp32 128x128 block scales (17 block rows)
    assert bench.gemm_bytes(M, N, K, 1) == w4 + M * K * 2 + M * N * 4 == 8133632
    assert bench.gemm_bytes(M, N, K, 0) == w8 + M * K * 2 + M * N * 4 == 15233760
    assert bench.gemm_bytes(M, N, K, 1, aq=True) == w4 + M * (K // 2 + K // 32) + M * N * 4 == 8091520
    assert bench.gemm_bytes(M, N, K, 0, aq=True) == w8 + M * (K + K // 128 * 4) + M * N * 4 == 15205984


def test_traffic_record_only_for_the_current_source(monkeypatch):
    rec = bench.recorded_traffic("prefill")
    assert rec is None or rec > 0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda files=None: "0" * 64)
    assert bench.recorded_traffic("prefill") is None
    assert bench.recorded_traffic("no_such_config") is None


def test_committed_traffic_records_are_well_formed():
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if not name.startswith("traffic_"):
            continue
        lines = [l for l in open(os.path.join(ROOT, "profiles", name)) if l.startswith("{")]
        assert len(lines) == 1, name
        rec = json.loads(lines[0])
        assert rec["hbm_bytes_per_launch"] == rec["hbm_read_bytes"] + rec["hbm_write_bytes"] or \
            abs(rec["hbm_bytes_per_launch"] - rec["hbm_read_bytes"] - rec["hbm_write_bytes"]) <= 1, name
        assert abs(rec["traffic_over_algorithmic"] - rec["hbm_bytes_per_launch"] /
                   rec["algorithmic_bytes_per_launch"]) < 1e-4, name
        assert len(rec["kernel_source_sha256"]) == 64, name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _fake_capture(w, rows):
    """What Workload.capture returns, made from the oracle's own outputs."""
    got = []
    for p in w.host:
        o = bench._oracle_call(p, w.fmt, w.layout, w.keep_bf16, rows=rows)
        d = {"rows": rows, "q": o["q"].copy(), "scale": o["scale"].copy()}
        for k in ("residual_out", "bf16"):
            if k in o:
                d[k] = o[k].copy()
        got.append(d)
    return got


def test_parity_summary_reports_exact_and_detects_a_flipped_byte():
    import types
    from fp4_quant_amd import inputs
    for fmt, lay, keep in ((0, 0, True), (1, 1, False), (0, 2, False)):
        w = types.SimpleNamespace(host=[inputs.make_problem(40, 512, seed_x=5, residual=True)], fmt=fmt,
                                  layout=lay, keep_bf16=keep)
        cap = _fake_capture(w, 40)
        rep = bench.parity_summary({"w": (w, cap)})
        assert rep["all_bit_exact"], rep
        cap[0]["q"][3, 7] ^= 1
        rep = bench.parity_summary({"w": (w, cap)})
        assert not rep["all_bit_exact"]
        assert rep["workloads"]["w"][0]["codes_identical_frac"] < 1.0
        cap = _fake_capture(w, 40)
        cap[0]["residual_out"][0, 0] ^= 1
        assert not bench.parity_summary({"w": (w, cap)})["all_bit_exact"]


def test_identity_fields():
    a, b = bench.source_sha256(), bench.source_sha256()
    assert a == b and len(a) == 64
    sha, where = bench.git_identity()
    assert where.startswith(("checkout", "build", "unavailable"))
    assert sha is None or len(sha) == 40
    h = bench.host_info()
    assert h["logical_cpus"] >= 1
    assert bench.median([3, 1, 2]) == 2 and bench.median([4, 1, 2, 3]) == 2.5


def test_serial_oracle_is_one_thread_and_equal():
    """The single-thread CPU leg times the oracle built without OpenMP
    (oracle.serial()): one thread whatever the host's OpenMP runtime imposes,
    and the same outputs as the OpenMP build."""
    import numpy as np
    import oracle
    from fp4_quant_amd import inputs
    assert oracle.serial().num_threads() == 1
    p = inputs.make_problem(37, 1024, seed_x=5, residual=True, outliers=True)
    for fmt, layout in ((0, 0), (1, 1)):
        a = bench._oracle_out(p, fmt, layout, True, 37)
        b = bench._oracle_out(p, fmt, layout, True, 37)
        bench._oracle_call(p, fmt, layout, True, a)
        bench._oracle_call(p, fmt, layout, True, b, orc=oracle.serial())
        assert a.keys() == b.keys() and all(np.array_equal(a[k], b[k]) for k in a)
