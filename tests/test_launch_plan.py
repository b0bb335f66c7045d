"""Launch planning on the host: rmsq_plan_launch reports the launches the
fused call would make for its arguments and an optional per-call hint,
without any HIP call. Problems carry fake, never dereferenced device
addresses; nothing here can launch a kernel, so it runs on any machine."""
import ctypes as C
import threading

import pytest

import fp4_quant_amd as fq

A = 0x7F0000000000
TB = 1 << 40


def prob(k=0, M=8192, N=7168, residual=True, fmt=0, layout=0, in_place=False, bf16=False):
    """A problem whose buffers are fake addresses k * 16 TiB apart."""
    base = A + k * 16 * TB
    r = base + 2 * TB if residual else None
    return dict(x=base, ldx=0, residual_in=r, residual_out=(r if in_place else base + 3 * TB) if residual else None,
                ldr=0, gamma=base + TB, eps=1e-6, M=M, N=N, group=128 if fmt == 0 else 32, fmt=fmt,
                scale_layout=layout, out_q=base + 4 * TB, out_scale=base + 5 * TB,
                out_bf16=base + 6 * TB if bf16 else None, ldb=0)


def plan(probs, hint=None):
    arr = (fq.rmsq_problem * len(probs))(*[fq.rmsq_problem(**p) for p in probs])
    return fq.rmsq_plan_launch(arr, hint)


def test_default_plans_of_the_workloads():
    pre = plan([prob(bf16=True)])
    assert len(pre) == 1
    assert (pre[0]["chunks_per_lane"], pre[0]["waves_per_row"]) == (2, 7)
    assert pre[0]["workgroups"] == 8192 and pre[0]["threads_per_workgroup"] == 448
    assert pre[0]["row_splits"] == 1 and pre[0]["residual"] == 1
    dec = plan([prob(M=64)])[0]
    assert (dec["chunks_per_lane"], dec["waves_per_row"], dec["row_splits"]) == (1, 14, 4)
    assert dec["workgroups"] == 64 * 4
    mla = plan([prob(0, M=4096, N=1536, residual=False), prob(1, M=4096, N=512, residual=False)])
    assert len(mla) == 1 and mla[0]["problems"] == 2 and mla[0]["rows"] == 8192
    assert (mla[0]["chunks_per_lane"], mla[0]["waves_per_row"], mla[0]["waves_per_workgroup"]) == (3, 1, 8)
    assert mla[0]["lanes_per_row"] == [64, 64]       # one row per wave
    assert mla[0]["workgroups"] == 1024
    assert mla[0]["tail"] == 2                       # whole 64-lane steps: the wave skips the rest
    assert pre[0]["tail"] == 1 and dec["tail"] == 0  # exact rows; split rows are bounded per lane
    assert plan([prob(M=4096, N=1536, residual=False)])[0]["tail"] == 1
    assert plan([prob(0, M=4096, N=1536, residual=False), prob(1, M=4096, N=640, residual=False)])[0]["tail"] == 0
    mx = plan([prob(M=16384, fmt=1, layout=1)])[0]
    assert (mx["chunks_per_lane"], mx["waves_per_row"], mx["row_group"]) == (2, 7, 16)


def test_mixed_residual_set_takes_two_launches_residual_first():
    p = plan([prob(0, M=100, residual=False), prob(1, M=30, residual=True)])
    assert [l["residual"] for l in p] == [1, 0]
    assert [l["rows"] for l in p] == [30, 100]


def test_in_place_residual_is_never_split():
    assert plan([prob(M=64)])[0]["row_splits"] == 4
    assert plan([prob(M=64, in_place=True)])[0]["row_splits"] == 1
    assert plan([prob(M=64, in_place=True)], fq.launch_hint(row_splits=8))[0]["row_splits"] == 1


def test_hint_fields_take_effect():
    p = [prob(M=512, bf16=True)]
    assert plan(p, fq.launch_hint(2, 7))[0]["chunks_per_lane"] == 2
    l = plan(p, fq.launch_hint(4, 7))[0]
    assert (l["chunks_per_lane"], l["waves_per_row"], l["threads_per_workgroup"]) == (4, 7, 448)
    assert plan(p, fq.launch_hint(row_splits=2))[0]["row_splits"] == 2
    assert plan(p, fq.launch_hint(row_splits=7))[0]["row_splits"] == 4          # power of two below
    assert plan([prob(M=8192, layout=2)], fq.launch_hint(row_group=32))[0]["row_group"] == 32
    assert plan([prob(M=8192, layout=2)])[0]["row_group"] == 16
    one = [prob(M=2048, N=1536, residual=False)]
    assert plan(one)[0]["waves_per_workgroup"] == 8
    l = plan(one, fq.launch_hint(waves_per_workgroup=3))[0]
    assert l["waves_per_workgroup"] == 3 and l["workgroups"] == -(-2048 // 3) and l["threads_per_workgroup"] == 192
    mla = [prob(0, M=4096, N=1536, residual=False), prob(1, M=4096, N=512, residual=False)]
    l = plan(mla, fq.launch_hint(4, 1))[0]
    assert l["lanes_per_row"] == [64, 64] and l["workgroups"] == 1024 and l["tail"] == 2
    assert plan(mla, fq.launch_hint(lanes_per_row=64)) == plan(mla)
    # the default plan is what no hint and an all-zero hint give
    assert plan(p) == plan(p, fq.launch_hint())


@pytest.mark.parametrize("hint", [
    fq.launch_hint(2, 0), fq.launch_hint(0, 7), fq.launch_hint(5, 7), fq.launch_hint(7, 5),
    fq.launch_hint(1, 17), fq.launch_hint(1, 7),            # 1 x 7 waves cannot cover 7168
    fq.launch_hint(row_group=-1), fq.launch_hint(row_group=65), fq.launch_hint(waves_per_workgroup=17),
    fq.launch_hint(row_splits=9), fq.launch_hint(row_splits=-2), fq.launch_hint(lanes_per_row=8),
    fq.launch_hint(lanes_per_row=48), fq.launch_hint(lanes_per_row=128)])
def test_bad_hints_are_refused(hint):
    arr = (fq.rmsq_problem * 1)(fq.rmsq_problem(**prob()))
    out = fq.rmsq_launch_plan()
    assert fq.lib().rmsq_plan_launch(arr, 1, C.byref(hint), C.byref(out)) == fq.RMSQ_ERR_INVALID_ARG
    assert b"hint" in fq.lib().rmsq_last_error()
    assert out.launches == 0
    # the launching entry point refuses the same hint before any HIP call
    assert fq.lib().rmsnorm_quant_group_multi_ex(arr, 1, C.byref(hint), None) == fq.RMSQ_ERR_INVALID_ARG


def test_packed_lanes_per_row():
    """Packed rows of one chunk per lane take the fewest lanes (16, 32, 64)
    that hold the row; a wave then holds 64 / lanes rows, and a problem whose
    row count is not a multiple of that leaves its last wave part empty
    (ragged tail). Rows of more chunks per lane keep one row per wave."""
    for N, lanes in ((128, 16), (256, 32), (512, 64), (1024, 64)):
        l = plan([prob(M=4096, N=N, residual=False)])[0]
        assert l["waves_per_workgroup"] == 8 and l["lanes_per_row"] == [lanes], N
        waves = 4096 * lanes // 64
        assert l["workgroups"] == waves // 8 and l["tail"] == 1, N
    l = plan([prob(M=4096, N=2048, residual=False)])[0]          # two waves per row: not packed
    assert (l["waves_per_row"], l["waves_per_workgroup"], l["lanes_per_row"]) == (2, 1, [128])
    l = plan([prob(M=4099, N=128, residual=False)])[0]          # 1025 waves, the last one 3/4 empty
    assert l["workgroups"] == -(-1025 // 8) and l["tail"] == 0
    l = plan([prob(M=4096, N=128, residual=False)], fq.launch_hint(lanes_per_row=32))[0]
    assert l["lanes_per_row"] == [32] and l["workgroups"] == 2048 // 8 and l["tail"] == 0   # half of each row's lanes idle
    mixed = plan([prob(0, M=515, N=512, residual=False), prob(1, M=299, N=256, residual=False),
                  prob(2, M=45, N=128, residual=False)], fq.launch_hint(waves_per_workgroup=8))[0]
    assert mixed["lanes_per_row"] == [64, 32, 16] and mixed["tail"] == 0
    assert mixed["workgroups"] == -(-(515 + 150 + 12) // 8)
    # fewer than 64 lanes per row need rows of one chunk per lane, and must hold the row
    for N, lanes in ((1536, 32), (512, 32), (256, 16)):
        arr = (fq.rmsq_problem * 1)(fq.rmsq_problem(**prob(M=4096, N=N, residual=False)))
        out = fq.rmsq_launch_plan()
        h = fq.launch_hint(lanes_per_row=lanes)
        assert fq.lib().rmsq_plan_launch(arr, 1, C.byref(h), C.byref(out)) == fq.RMSQ_ERR_INVALID_ARG, N
    # unpacked launches report the lanes of their whole row
    assert plan([prob(M=8192)])[0]["lanes_per_row"] == [7 * 64]


def test_plan_validates_like_the_call():
    arr = (fq.rmsq_problem * 1)(fq.rmsq_problem(**dict(prob(), N=200)))
    out = fq.rmsq_launch_plan()
    assert fq.lib().rmsq_plan_launch(arr, 1, None, C.byref(out)) == fq.RMSQ_ERR_INVALID_ARG
    assert fq.lib().rmsq_plan_launch(arr, 1, None, None) == fq.RMSQ_ERR_INVALID_ARG
    assert plan([prob(M=0)]) == []


def test_two_threads_plan_independently():
    """Hints belong to their call: two host threads planning the same problem
    with different hints at the same time each always get their own plan, and
    a third thread without a hint always gets the default."""
    p = [prob(M=512, bf16=True)]
    arr = (fq.rmsq_problem * 1)(fq.rmsq_problem(**p[0]))
    default = plan(p)[0]
    cases = {"a": (fq.launch_hint(4, 7, row_splits=2), (4, 7, 2)),
             "b": (fq.launch_hint(2, 7, row_splits=1), (2, 7, 1)),
             "c": (None, (default["chunks_per_lane"], default["waves_per_row"], default["row_splits"]))}
    bad = []
    start = threading.Barrier(len(cases))

    def worker(name):
        hint, want = cases[name]
        out = fq.rmsq_launch_plan()
        start.wait()
        for _ in range(3000):
            rc = fq.lib().rmsq_plan_launch(arr, 1, C.byref(hint) if hint is not None else None, C.byref(out))
            l = out.launch[0]
            if rc != fq.RMSQ_OK or (l.chunks_per_lane, l.waves_per_row, l.row_splits) != want:
                bad.append((name, rc, l.chunks_per_lane, l.waves_per_row, l.row_splits))
                return

    ts = [threading.Thread(target=worker, args=(n,)) for n in cases]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not bad, bad


def test_query_shape_matches_the_plan():
    for N, rows in ((7168, 8192), (7168, 64), (7168, 512), (1536, 8192), (512, 4096), (32768, 3)):
        J, W = fq.rmsq_query_shape(N, rows)
        l = plan([prob(M=rows, N=N, residual=False)])[0]
        assert (l["chunks_per_lane"], l["waves_per_row"]) == (J, W), (N, rows)
