"""Host-side tests of the C ABI: the library loads, exports every symbol the
header declares, and validates arguments before touching the GPU. Pointers
here are fake addresses that are never dereferenced: validation needs only
their values. A call that passed validation by mistake would enqueue a kernel
on those addresses, so where a gfx950 GPU is present the whole module is
skipped: these tests are for the CPU build, where such a regression shows up
as a failed assertion (the missing device stops the call)."""
import ctypes as C
import os
import re
import subprocess

import pytest

import fp4_quant_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(fq.rmsq_device_supported(0), reason="fake device addresses: CPU build only")

A = 0x7F0000000000          # fake, 256-byte aligned device addresses
MB = 1 << 20


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"rmsnorm_quant_group", "rmsnorm_quant_group_multi", "rmsq_device_supported"} <= set(names)
    L = fq.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(fq.EXPORTS) <= set(names)


@pytest.mark.parametrize("struct", ["rmsq_problem", "rmsq_launch_hint", "rmsq_launch_info", "rmsq_launch_plan"])
def test_struct_layout_matches_header(tmp_path, struct):
    """The ctypes mirrors of the header's structs have the C compiler's layout."""
    cls = getattr(fq, struct)
    fields = [f for f, _ in cls._fields_]
    src = tmp_path / "layout.c"
    body = "".join(f'printf("%zu\\n", offsetof({struct}, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "rmsq.h"\n'
                   f'int main(void){{printf("%zu\\n", sizeof({struct}));{body}return 0;}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == C.sizeof(cls)
    assert got[1:] == [getattr(cls, f).offset for f in fields]


def test_status_strings():
    L = fq.lib()
    assert L.rmsq_status_string(0) == b"RMSQ_OK"
    assert L.rmsq_status_string(1) == b"RMSQ_ERR_INVALID_ARG"
    assert L.rmsq_status_string(2) == b"RMSQ_ERR_UNSUPPORTED"
    assert L.rmsq_status_string(3) == b"RMSQ_ERR_HIP"
    assert L.rmsq_status_string(99) == b"RMSQ_UNKNOWN_STATUS"


def test_scale_bytes():
    assert fq.rmsq_scale_bytes(8192, 7168, 128, 0) == 8192 * 56 * 4
    assert fq.rmsq_scale_bytes(16384, 7168, 32, 1, 0) == 16384 * 224
    assert fq.rmsq_scale_bytes(33, 7168, 32, 1, 1) == 64 * 224
    assert fq.rmsq_scale_bytes(0, 7168, 32, 1, 1) == 0
    assert fq.rmsq_scale_bytes(8, 7168, 32, 0, 0) == 0          # FP8 needs group 128
    assert fq.rmsq_scale_bytes(8, 7168, 128, 0, 1) == 0         # tiled is MXFP4 only
    assert fq.rmsq_scale_bytes(8, 7168, 128, 0, 2) == 8 * 56 * 4
    assert fq.rmsq_scale_bytes(9, 7168, 32, 1, 2) == 9 * 224
    assert fq.rmsq_scale_bytes(8, 100, 32, 1, 0) == 0


def _call(x=A, r=None, g=A + 100 * MB, eps=1e-6, M=4, N=256, group=128, fmt=0,
          q=A + 200 * MB, s=A + 300 * MB, ro=None, yb=None):
    L = fq.lib()
    return L.rmsnorm_quant_group(x, r, g, eps, M, N, group, fmt, q, s, ro, yb, None)


def _multi(**kw):
    base = dict(x=A, ldx=0, residual_in=None, residual_out=None, ldr=0, gamma=A + 100 * MB, eps=1e-6,
                M=4, N=256, group=128, fmt=0, scale_layout=0, out_q=A + 200 * MB, out_scale=A + 300 * MB,
                out_bf16=None, ldb=0)
    probs = kw.pop("probs", None)
    if probs is None:
        base.update(kw)
        probs = [base]
    arr = (fq.rmsq_problem * len(probs))(*[fq.rmsq_problem(**p) for p in probs])
    return fq.lib().rmsnorm_quant_group_multi(arr, len(probs), None)


@pytest.mark.parametrize("kw,status", [
    (dict(group=64), fq.RMSQ_ERR_UNSUPPORTED),
    (dict(fmt=1, group=128), fq.RMSQ_ERR_UNSUPPORTED),
    (dict(fmt=7), fq.RMSQ_ERR_UNSUPPORTED),
    (dict(N=65536), fq.RMSQ_ERR_UNSUPPORTED),
    (dict(N=200), fq.RMSQ_ERR_INVALID_ARG),
    (dict(N=0), fq.RMSQ_ERR_INVALID_ARG),
    (dict(M=-1), fq.RMSQ_ERR_INVALID_ARG),
    (dict(eps=float("nan")), fq.RMSQ_ERR_INVALID_ARG),
    (dict(eps=-1.0), fq.RMSQ_ERR_INVALID_ARG),
    (dict(r=A + 400 * MB), fq.RMSQ_ERR_INVALID_ARG),            # residual_in without residual_out
    (dict(ro=A + 400 * MB), fq.RMSQ_ERR_INVALID_ARG),
    (dict(x=None), fq.RMSQ_ERR_INVALID_ARG),
    (dict(q=None), fq.RMSQ_ERR_INVALID_ARG),
    (dict(s=None), fq.RMSQ_ERR_INVALID_ARG),
    (dict(g=None), fq.RMSQ_ERR_INVALID_ARG),
    (dict(x=A + 8), fq.RMSQ_ERR_INVALID_ARG),                   # bf16 pointers 16-byte aligned
    (dict(g=A + 100 * MB + 2), fq.RMSQ_ERR_INVALID_ARG),
    (dict(yb=A + 500 * MB + 4), fq.RMSQ_ERR_INVALID_ARG),
    (dict(q=A + 200 * MB + 4), fq.RMSQ_ERR_INVALID_ARG),        # FP8 codes 8-byte aligned
    (dict(s=A + 300 * MB + 2), fq.RMSQ_ERR_INVALID_ARG),
    (dict(q=A + 100), fq.RMSQ_ERR_INVALID_ARG),                  # codes overlap x
    (dict(yb=A + 200 * MB), fq.RMSQ_ERR_INVALID_ARG),           # bf16 overlaps codes
    (dict(s=A + 200 * MB + 512), fq.RMSQ_ERR_INVALID_ARG),      # scales inside the 1 KiB of codes
    (dict(r=A + 400 * MB, ro=A + 400 * MB + 16), fq.RMSQ_ERR_INVALID_ARG),  # partial in-place
    (dict(r=A + 400 * MB, ro=A), fq.RMSQ_ERR_INVALID_ARG),      # residual_out over x
])
def test_validation_errors(kw, status):
    assert _call(**kw) == status
    assert fq.lib().rmsq_last_error()


def test_m_zero_is_a_noop_without_device():
    assert _call(M=0) == fq.RMSQ_OK
    assert _call(M=0, x=None, q=None, s=None, g=None) == fq.RMSQ_OK
    assert _call(M=0, r=None, ro=A + 400 * MB) == fq.RMSQ_OK     # empty tensors have NULL data


TB = 1 << 40


def test_launch_beyond_the_work_item_limit_is_refused_before_any_hip_call():
    """One launch covers at most 2^32 work-items per grid dimension: 70M rows
    of 512 (one 64-lane wave per row) exceed it, 60M rows do not. Buffers are
    fake addresses 1 TiB apart; the refusal comes before the device check."""
    big = dict(x=A, g=A + TB, q=A + 2 * TB, s=A + 3 * TB, N=512)
    assert _call(M=70_000_000, **big) == fq.RMSQ_ERR_UNSUPPORTED
    assert b"2^32" in fq.lib().rmsq_last_error()
    # a set that mixes a residual problem with such a one: neither launch is made
    small = dict(x=A + 4 * TB, ldx=0, residual_in=A + 5 * TB, residual_out=A + 6 * TB, ldr=0, gamma=A + TB,
                 eps=1e-6, M=4, N=512, group=128, fmt=0, scale_layout=0, out_q=A + 7 * TB, out_scale=A + 8 * TB,
                 out_bf16=None, ldb=0)
    huge = dict(small, x=A, residual_in=None, residual_out=None, M=70_000_000, out_q=A + 2 * TB,
                out_scale=A + 3 * TB)
    assert _multi(probs=[small, huge]) == fq.RMSQ_ERR_UNSUPPORTED
    assert b"2^32" in fq.lib().rmsq_last_error()
    L = fq.lib()
    assert L.dynamic_per_group_scaled_quant(A, 40_000_000, 128, 128, 0, 0, A + 2 * TB, A + 3 * TB,
                                            None) == fq.RMSQ_ERR_UNSUPPORTED
    assert b"2^32" in L.rmsq_last_error()
    # the widest rows (32768: 16 waves, 1024 work-items each): 2^22 - 1 rows fit, 2^22 do not
    wide = dict(big, N=32768)
    assert _call(M=1 << 22, **wide) == fq.RMSQ_ERR_UNSUPPORTED
    assert b"2^32" in fq.lib().rmsq_last_error()
    if not fq.rmsq_device_supported(0):   # within the limit: only the missing device stops it
        assert _call(M=(1 << 22) - 1, **wide) == fq.RMSQ_ERR_UNSUPPORTED
        assert b"gfx950" in fq.lib().rmsq_last_error()
        assert _call(M=60_000_000, **big) == fq.RMSQ_ERR_UNSUPPORTED
        assert b"gfx950" in fq.lib().rmsq_last_error()
        assert L.dynamic_per_group_scaled_quant(A, 30_000_000, 128, 128, 0, 0, A + 2 * TB, A + 3 * TB,
                                                None) == fq.RMSQ_ERR_UNSUPPORTED
        assert b"gfx950" in L.rmsq_last_error()


def test_valid_call_without_a_gfx950_device_is_unsupported():
    if fq.rmsq_device_supported(0):
        pytest.skip("a gfx950 device is present")
    assert _call() == fq.RMSQ_ERR_UNSUPPORTED
    assert _call(r=A + 400 * MB, ro=A + 400 * MB) == fq.RMSQ_ERR_UNSUPPORTED   # in place is valid
    assert b"gfx950" in fq.lib().rmsq_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(ldx=100), fq.RMSQ_ERR_INVALID_ARG),                   # stride not a multiple of 8
    (dict(ldx=128), fq.RMSQ_ERR_INVALID_ARG),                   # stride < N
    (dict(out_bf16=A + 500 * MB, ldb=260), fq.RMSQ_ERR_INVALID_ARG),
    (dict(scale_layout=1), fq.RMSQ_ERR_UNSUPPORTED),            # tiled scales with FP8
    (dict(scale_layout=3), fq.RMSQ_ERR_INVALID_ARG),
    (dict(fmt=1, group=32, scale_layout=1, out_q=A + 200 * MB + 4, out_scale=A + 300 * MB + 1),
     fq.RMSQ_ERR_UNSUPPORTED),                                 # valid MXFP4 tiled: no device here
])
def test_multi_validation(kw, status):
    if status == fq.RMSQ_ERR_UNSUPPORTED and fq.rmsq_device_supported(0) and kw.get("fmt") == 1:
        pytest.skip("a gfx950 device is present")
    assert _multi(**kw) == status


def test_multi_count_and_shared_fmt():
    L = fq.lib()
    assert L.rmsnorm_quant_group_multi(None, 1, None) == fq.RMSQ_ERR_INVALID_ARG
    p = dict(x=A, ldx=0, residual_in=None, residual_out=None, ldr=0, gamma=A + 100 * MB, eps=1e-6,
             M=4, N=256, group=128, fmt=0, scale_layout=0, out_q=A + 200 * MB, out_scale=A + 300 * MB,
             out_bf16=None, ldb=0)
    p2 = dict(p, x=A + 600 * MB, out_q=A + 700 * MB, out_scale=A + 800 * MB, fmt=1, group=32)
    assert _multi(probs=[p] * 5) == fq.RMSQ_ERR_INVALID_ARG
    assert _multi(probs=[p, p2]) == fq.RMSQ_ERR_INVALID_ARG
    # two problems whose outputs collide
    p3 = dict(p, x=A + 600 * MB)
    assert _multi(probs=[p, p3]) == fq.RMSQ_ERR_INVALID_ARG


def test_row_grouping_is_a_bijection():
    """The device mapping of workgroups to rows (written out here in Python
    from its definition) permutes the rows for every grid size and group."""
    def row_of_block(b, rows, lg):
        if lg == 0 or b >= (rows >> (lg + 3)) << (lg + 3):
            return b
        x, k = b & 7, b >> 3
        return ((((k >> lg) << 3) + x) << lg) + (k & ((1 << lg) - 1))
    for g in (0, 1, 2, 4, 5, 6):
        for rows in list(range(1, 700)) + [8192, 8191, 16384, 16383 + 256]:
            assert sorted(row_of_block(b, rows, g) for b in range(rows)) == list(range(rows)), (g, rows)


def test_row_split_block_mapping_is_a_bijection():
    """With 2^slg workgroups per row, block b -> (row, split) as the kernel
    computes it covers every (row, split) of the padded rows exactly once,
    keeps a row's splits on one XCD (b % 8), and the chunk ranges of a row's
    splits partition the row on group boundaries."""
    for slg in (1, 2, 3):
        S = 1 << slg
        for rows in (1, 7, 8, 9, 33, 64, 100, 128):
            padded = (rows + 7) // 8 * 8
            seen = {}
            for b in range(padded * S):
                split = (b >> 3) & (S - 1)
                row = ((b >> (3 + slg)) << 3) | (b & 7)
                assert (row, split) not in seen
                seen[(row, split)] = b
            assert set(seen) == {(r, k) for r in range(padded) for k in range(S)}
            for r in range(rows):
                assert len({seen[(r, k)] % 8 for k in range(S)}) == 1
        for C, q in ((896, 16), (192, 16), (64, 16), (16, 16), (896, 4), (12, 4), (48, 1)):
            if C // q < S:
                continue
            bounds = []
            for k in range(S):
                lo = ((k * (C // q)) >> slg) * q
                hi = C if k + 1 == S else (((k + 1) * (C // q)) >> slg) * q
                assert lo % q == 0 and hi % q == 0 or hi == C
                bounds.append((lo, hi))
            assert bounds[0][0] == 0 and bounds[-1][1] == C
            assert all(bounds[k][1] == bounds[k + 1][0] and bounds[k][0] < bounds[k][1] for k in range(S - 1))


def test_launch_shape_always_fits():
    """For every N the library accepts, the chosen shape covers the row with a
    legal workgroup (long per-lane rows use at most 4 waves)."""
    for N in range(8, 32768 + 1, 8):
        for rows in (1, 64, 512, 8192):
            J, W = fq.rmsq_query_shape(N, rows)
            C_ = N // 8
            assert J in (1, 2, 3, 4, 7, 8, 14) and 1 <= W <= (4 if J >= 7 else 16), (N, rows, J, W)
            assert J * W * 64 >= C_, (N, rows, J, W)
    assert fq.rmsq_query_shape(7168, 8192) == (2, 7)
    assert fq.rmsq_query_shape(7168, 768) == (2, 7)
    assert fq.rmsq_query_shape(7168, 512) == (1, 14)    # at most two rows per CU: most waves
    assert fq.rmsq_query_shape(7168, 64) == (1, 14)
    assert fq.rmsq_query_shape(1536, 8192) == (3, 1)
    with pytest.raises(fq.RmsqError):
        fq.rmsq_query_shape(32776, 1)


def test_unfused_entry_points_validate():
    L = fq.lib()
    g, r, ro, yb, q, sc = A + 100 * MB, A + 400 * MB, A + 500 * MB, A + 600 * MB, A + 200 * MB, A + 300 * MB
    # add_rmsnorm(x, residual_in, gamma, eps, M, N, residual_out, out_bf16, stream)
    assert L.add_rmsnorm(A, None, g, 1e-6, 4, 100, None, yb, None) == fq.RMSQ_ERR_INVALID_ARG   # N % 8
    assert L.add_rmsnorm(A, None, g, 1e-6, 4, 256, None, None, None) == fq.RMSQ_ERR_INVALID_ARG  # out_bf16 needed
    assert L.add_rmsnorm(A, r, g, 1e-6, 4, 256, None, yb, None) == fq.RMSQ_ERR_INVALID_ARG      # pairing
    assert L.add_rmsnorm(A, None, g, float("inf"), 4, 256, None, yb, None) == fq.RMSQ_ERR_INVALID_ARG
    assert L.add_rmsnorm(A, None, g, 1e-6, 4, 256, None, A + 16, None) == fq.RMSQ_ERR_INVALID_ARG  # overlap
    assert L.add_rmsnorm(A, None, g, 1e-6, 0, 256, None, None, None) == fq.RMSQ_OK
    # dynamic_per_group_scaled_quant(x, M, N, group, fmt, layout, out_q, out_scale, stream)
    assert L.dynamic_per_group_scaled_quant(A, 4, 256, 64, 0, 0, q, sc, None) == fq.RMSQ_ERR_UNSUPPORTED
    assert L.dynamic_per_group_scaled_quant(A, 4, 256, 128, 0, 1, q, sc, None) == fq.RMSQ_ERR_UNSUPPORTED
    assert L.dynamic_per_group_scaled_quant(A, 4, 200, 128, 0, 0, q, sc, None) == fq.RMSQ_ERR_INVALID_ARG
    assert L.dynamic_per_group_scaled_quant(A, 4, 256, 128, 0, 0, None, sc, None) == fq.RMSQ_ERR_INVALID_ARG
    assert L.dynamic_per_group_scaled_quant(A, 4, 256, 128, 0, 0, A + 64, sc, None) == fq.RMSQ_ERR_INVALID_ARG
    assert L.dynamic_per_group_scaled_quant(A, 0, 256, 32, 1, 1, None, None, None) == fq.RMSQ_OK
    if not fq.rmsq_device_supported(0):
        assert L.add_rmsnorm(A, r, g, 1e-6, 4, 256, ro, yb, None) == fq.RMSQ_ERR_UNSUPPORTED
        assert L.dynamic_per_group_scaled_quant(A, 4, 256, 32, 1, 1, q, sc, None) == fq.RMSQ_ERR_UNSUPPORTED


def test_gemm_validates():
    L = fq.lib()
    E = fq.RMSQ_ERR_INVALID_ARG
    w, s, o = A + 100 * MB, A + 200 * MB, A + 300 * MB
    R = fq.W_ROW_MAJOR

    def g(a=A, lda=256, w=w, s=s, lay=R, M=4, N=32, K=256, o=o, ldc=32):
        # gemm_a16wfp4_prequant(a, lda, w, w_scale, w_layout, M, N, K, out, ldc, stream)
        return L.gemm_a16wfp4_prequant(a, lda, w, s, lay, M, N, K, o, ldc, None)

    assert g(N=24, ldc=24) == E          # N % 16
    assert g(K=200) == E                 # K % 128
    assert g(M=-1) == E
    assert g(lda=128) == E               # lda < K
    assert g(lda=260) == E               # lda % 8
    assert g(lda=(1 << 25) + 8) == E     # lda beyond RMSQ_GEMM_LDA_MAX
    assert g(ldc=16) == E                # ldc < N
    assert g(lay=2) == E                 # unknown weight layout
    assert g(a=A + 2) == E               # a alignment
    assert g(w=w + 8) == E               # w alignment
    assert g(o=o + 2) == E               # out alignment
    assert g(o=A + 64) == E              # out overlaps a
    assert g(o=w + 1024) == E            # out overlaps w
    assert g(o=s) == E                   # out overlaps the scales
    assert g(a=None) == E                # NULL
    assert g(lda=1 << 21, K=1 << 21) == E   # K beyond the limit
    assert g(M=0) == fq.RMSQ_OK          # no-op
    assert g(M=0, lay=fq.W_PRESHUFFLED) == fq.RMSQ_OK
    assert g() in (fq.RMSQ_OK, fq.RMSQ_ERR_UNSUPPORTED)
    if not fq.rmsq_device_supported(0):
        assert g() == fq.RMSQ_ERR_UNSUPPORTED


def test_preshuffle_validates():
    L = fq.lib()
    E = fq.RMSQ_ERR_INVALID_ARG
    w, s, wo, so = A, A + 100 * MB, A + 200 * MB, A + 300 * MB
    # mxfp4_weight_preshuffle(w, w_scale, N, K, w_out, w_scale_out, stream)
    assert L.mxfp4_weight_preshuffle(w, s, 24, 256, wo, so, None) == E       # N % 16
    assert L.mxfp4_weight_preshuffle(w, s, 32, 192, wo, so, None) == E       # K % 128
    assert L.mxfp4_weight_preshuffle(w, s, 32, 256, w + 1024, so, None) == E  # output overlaps input
    assert L.mxfp4_weight_preshuffle(w, s, 32, 256, wo, s + 8, None) == E    # scale output overlaps
    assert L.mxfp4_weight_preshuffle(w, s, 32, 256, wo + 4, so, None) == E   # alignment
    assert L.mxfp4_weight_preshuffle(None, s, 32, 256, wo, so, None) == E
    if not fq.rmsq_device_supported(0):
        assert L.mxfp4_weight_preshuffle(w, s, 32, 256, wo, so, None) == fq.RMSQ_ERR_UNSUPPORTED


def test_gemm8_validates():
    L = fq.lib()
    E = fq.RMSQ_ERR_INVALID_ARG
    w, s, o = A + 100 * MB, A + 200 * MB, A + 300 * MB

    def g(a=A, lda=256, w=w, s=s, lay=fq.W_ROW_MAJOR, M=4, N=32, K=256, o=o, ldc=32):
        # gemm_a16w8_prequant(a, lda, w, w_scale, w_layout, M, N, K, out, ldc, stream)
        return L.gemm_a16w8_prequant(a, lda, w, s, lay, M, N, K, o, ldc, None)

    assert g(N=24, ldc=24) == E          # N % 16
    assert g(K=192, lda=192) == E        # K % 128
    assert g(M=-1) == E
    assert g(M=65535 * 32 + 1) == E      # more row blocks than the grid holds
    assert g(lda=128) == E
    assert g(ldc=16) == E
    assert g(lay=2) == E
    assert g(s=s + 2) == E               # scale alignment
    assert g(w=w + 8) == E
    assert g(o=w + 4096) == E            # out overlaps w (N * K = 8192 bytes)
    assert g(o=s + 4) == E               # out overlaps the block scales (1 x 2 floats)
    assert g(a=None) == E
    assert g(M=0) == fq.RMSQ_OK
    if not fq.rmsq_device_supported(0):
        assert g() == fq.RMSQ_ERR_UNSUPPORTED
    # fp8_weight_preshuffle(w, N, K, w_out, stream)
    assert L.fp8_weight_preshuffle(w, 24, 256, o, None) == E
    assert L.fp8_weight_preshuffle(w, 32, 256, w + 4096, None) == E
    assert L.fp8_weight_preshuffle(w, 32, 256, o + 8, None) == E
    if not fq.rmsq_device_supported(0):
        assert L.fp8_weight_preshuffle(w, 32, 256, o, None) == fq.RMSQ_ERR_UNSUPPORTED


def test_library_exports_only_the_declared_interface():
    """Built with hidden visibility: the dynamic symbol table holds the C ABI
    of include/rmsq.h and nothing else of the library's own code."""
    import shutil
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", fq.LIB_PATH], capture_output=True, text=True, check=True)
    text_syms = {l.split()[-1] for l in out.stdout.splitlines() if len(l.split()) == 3 and l.split()[1] == "T"}
    assert text_syms == set(_declared_functions())


def test_binding_refuses_host_tensors():
    """A CPU tensor never reaches the C ABI: its address would be dereferenced
    on the GPU."""
    import torch
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fq.dynamic_per_group_scaled_quant(x, 4, 256, 128, 0, 0, x, x, stream=0)
    with pytest.raises(ValueError):
        fq.gemm_a16wfp4_prequant(x, 256, x, x, fq.W_ROW_MAJOR, 4, 16, 256, x, 16, stream=0)


@pytest.mark.parametrize("entry", ["gemm_afp4wfp4", "gemm_a8w8_blockscale"])
def test_quantized_activation_gemms_validate(entry):
    L = fq.lib()
    E = fq.RMSQ_ERR_INVALID_ARG
    fp8 = entry == "gemm_a8w8_blockscale"
    q, sa, w, s, o = A, A + 50 * MB, A + 100 * MB, A + 200 * MB, A + 300 * MB
    R = fq.W_ROW_MAJOR
    f = getattr(L, entry)

    def g(q=q, sa=sa, al=fq.SCALE_ROW_MAJOR, w=w, s=s, lay=R, M=4, N=32, K=256, o=o, ldc=32):
        # entry(a_q, a_scale, a_scale_layout, w, w_scale, w_layout, M, N, K, out, ldc, stream)
        return f(q, sa, al, w, s, lay, M, N, K, o, ldc, None)

    assert g(N=24, ldc=24) == E          # N % 16
    assert g(K=200) == E                 # K % 128
    assert g(M=-1) == E
    assert g(ldc=16) == E                # ldc < N
    assert g(lay=2) == E                 # unknown weight layout
    assert g(al=3) == E                  # unknown activation scale layout
    assert (g(al=fq.SCALE_TILED32) == E) == fp8   # tiled scales: MXFP4 only
    assert g(q=q + 8) == E               # a_q alignment
    if fp8:
        assert g(sa=sa + 2) == E         # fp32 scales alignment
    assert g(w=w + 8) == E               # w alignment
    assert g(o=o + 2) == E               # out alignment
    assert g(o=q + 64) == E              # out overlaps the codes
    assert g(o=sa) == E                  # out overlaps the activation scales
    assert g(o=w + 1024) == E            # out overlaps w
    assert g(q=None) == E                # NULL
    assert g(sa=None) == E
    assert g(M=0) == fq.RMSQ_OK          # no-op, pointers unused
    assert g(M=0, q=None, sa=None) == fq.RMSQ_OK
    assert g() in (fq.RMSQ_OK, fq.RMSQ_ERR_UNSUPPORTED)
    if not fq.rmsq_device_supported(0):
        assert g() == fq.RMSQ_ERR_UNSUPPORTED


def test_make_problem_checks_the_tensors_before_taking_addresses():
    """The binding's problem builder refuses tensors that the library would
    misread (wrong dtype or shape, a row stride below N such as an expanded
    residual, a residual output with another row stride) before it takes any
    address; CPU tensors reach these checks first, so this runs without a GPU."""
    import torch
    M, N = 4, 256
    x = torch.zeros((M, N), dtype=torch.bfloat16)
    g = torch.ones(N, dtype=torch.bfloat16)
    q = torch.zeros((M, N), dtype=torch.uint8)
    s = torch.zeros((M, N // 128), dtype=torch.float32)
    bad = [
        dict(x=x.float()),
        dict(x=x.t().contiguous().t()),                                   # column stride M
        dict(gamma=g[:128]),
        dict(residual_in=torch.zeros(N, dtype=torch.bfloat16).expand(M, N),
             residual_out=torch.zeros((M, N), dtype=torch.bfloat16)),      # row stride 0
        dict(residual_in=torch.zeros((M, N + 64), dtype=torch.bfloat16)[:, :N],
             residual_out=torch.zeros((M, N), dtype=torch.bfloat16)),      # row strides differ
        dict(out_bf16=torch.zeros((M, N), dtype=torch.float16)),
    ]
    for kw in bad:
        args = dict(x=x, gamma=g)
        args.update(kw)
        xx, gg = args.pop("x"), args.pop("gamma")
        with pytest.raises(ValueError):
            fq.make_problem(xx, gg, 1e-6, q, s, **args)
    with pytest.raises(ValueError, match="GPU tensors"):    # a well-formed problem on the host
        fq.make_problem(x, g, 1e-6, q, s)


def test_make_problem_checks_the_output_buffers():
    """Codes and scales reach the C ABI as bare pointers, so their sizes are
    checked in the binding: a short, mistyped or non-contiguous code or scale
    buffer is refused before any address is taken (CPU tensors reach these
    checks first, so this runs without a GPU)."""
    import torch
    M, N = 33, 256
    x = torch.zeros((M, N), dtype=torch.bfloat16)
    g = torch.ones(N, dtype=torch.bfloat16)
    u8, f32 = torch.uint8, torch.float32
    ok = {0: (torch.zeros((M, N), dtype=u8), torch.zeros((M, N // 128), dtype=f32)),
          1: (torch.zeros((M, N // 2), dtype=u8), torch.zeros(64 * (N // 32), dtype=u8))}   # tiled: 64 rows
    bad = [
        (0, 0, torch.zeros((M, N - 8), dtype=u8), ok[0][1]),                 # codes short
        (0, 0, torch.zeros((M, N), dtype=torch.int8), ok[0][1]),             # codes mistyped
        (0, 0, torch.zeros((N, M), dtype=u8).t(), ok[0][1]),                 # codes not dense
        (0, 0, None, ok[0][1]),
        (0, 0, ok[0][0], torch.zeros((M, 1), dtype=f32)),                    # scales short
        (0, 0, ok[0][0], torch.zeros((M, 2), dtype=u8)),                     # FP8 scales are fp32
        (0, 2, ok[0][0], torch.zeros((2, M), dtype=f32)[:, :M - 1]),         # column-major, short
        (1, 0, torch.zeros((M, N), dtype=u8), ok[1][1]),                     # MXFP4 codes are N/2 per row
        (1, 1, ok[1][0], torch.zeros(M * (N // 32), dtype=u8)),              # tiled needs 64 rows here
        (1, 0, ok[1][0], torch.zeros(M * (N // 32), dtype=f32)),             # MXFP4 scales are bytes
        (1, 0, ok[1][0], None),
    ]
    for fmt, lay, q, s in bad:
        with pytest.raises(ValueError, match="out_q|out_scale"):
            fq.make_problem(x, g, 1e-6, q, s, fmt=fmt, scale_layout=lay)
    for fmt, lay in ((0, 0), (0, 2), (1, 0), (1, 1), (1, 2)):   # the right sizes pass on to the device check
        with pytest.raises(ValueError, match="GPU tensors"):
            fq.make_problem(x, g, 1e-6, *ok[fmt], fmt=fmt, scale_layout=lay)


def test_library_binds_to_torchs_hip_runtime():
    """Loaded through the binding, even before anything imported torch, the
    library's HIP calls resolve to the runtime torch loaded (the one that owns
    the streams and memory it is given), not to a second copy."""
    code = "import fp4_quant_amd as fq; fq.lib()"
    env = dict(os.environ, LD_DEBUG="bindings")
    r = subprocess.run([__import__("sys").executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if "librmsq.so" in l and "`hipLaunchKernel'" in l]
    assert lines, "no binding of hipLaunchKernel seen"
    assert all("torch/lib/libamdhip64" in l for l in lines), lines
