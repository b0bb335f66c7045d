"""End-to-end parity of the HIP path (through the C ABI) with the CPU oracle,
element by element on the same seeded inputs: the workloads at full size,
shape sweeps with ragged tails, forced launch shapes, and edge cases. Every
output buffer is surrounded by guard bands that must stay untouched."""
import numpy as np
import pytest
import torch

import fp4_quant_amd as fq
from fp4_quant_amd import inputs
from tests.gpu_util import compare, dev, host, say

pytestmark = pytest.mark.gpu

GUARD = 4096
SENT = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert fq.rmsq_device_supported(0), "GPU tests need a gfx950 device"


class Guarded:
    """A device output buffer with sentinel bytes before and after it."""

    def __init__(self, nbytes, dtype, shape):
        self.buf = torch.full((GUARD + nbytes + GUARD,), SENT, dtype=torch.uint8, device="cuda")
        self.n = nbytes
        self.t = self.buf[GUARD:GUARD + nbytes].view(dtype).view(shape)

    def check(self, name):
        b = host(self.buf)
        assert np.all(b[:GUARD] == SENT) and np.all(b[GUARD + self.n:] == SENT), f"{name}: guard band written"


def _strided_dev(a, ld):
    """Device bf16 [M, N] with row stride ld (padding filled with sentinel)."""
    M, N = a.shape
    full = np.full((M, ld), 0x7FC1, np.uint16)
    full[:, :N] = a
    return dev(full)[:, :N]


def run_gpu(problems, single_entry=False, hint=None):
    """problems: dicts with numpy x, gamma, eps and optional residual,
    fmt, scale_layout, keep_bf16, inplace, ldx, ldr, ldb. Returns a list of
    dicts of numpy outputs, after checking every guard band."""
    structs, keep, outs = [], [], []
    for p in problems:
        M, N = p["x"].shape
        fmt = p.get("fmt", 0)
        lay = p.get("scale_layout", 0)
        x = _strided_dev(p["x"], p.get("ldx", N))
        g = dev(p["gamma"])
        o = {"q": Guarded(M * (N if fmt == 0 else N // 2), torch.uint8, (M, -1) if M else (0,)),
             "scale": Guarded(fq.rmsq_scale_bytes(M, N, 128 if fmt == 0 else 32, fmt, lay),
                              torch.float32 if fmt == 0 else torch.uint8, (-1,))}
        r = ro = yb = None
        if "residual" in p:
            r = _strided_dev(p["residual"], p.get("ldr", N))
            if p.get("inplace"):
                ro = r
            else:
                ld = p.get("ldr", N)
                o["residual_out"] = Guarded(max(M * ld * 2, 2), torch.bfloat16, (M, ld) if M else (-1,))
                ro = o["residual_out"].t[:, :N] if M else o["residual_out"].t
        if p.get("keep_bf16"):
            ld = p.get("ldb", N)
            o["bf16"] = Guarded(max(M * ld * 2, 2), torch.bfloat16, (M, ld) if M else (-1,))
            yb = o["bf16"].t[:, :N] if M else o["bf16"].t
        keep += [x, g, r]
        outs.append((o, ro, yb, r, p))
        if single_entry:
            fq.rmsnorm_quant_group(x, r, g, p["eps"], M, N, 128 if fmt == 0 else 32, fmt, o["q"].t,
                                   o["scale"].t, ro, yb)
        else:
            structs.append(fq.make_problem(x, g, p["eps"], o["q"].t, o["scale"].t, residual_in=r,
                                           residual_out=ro, out_bf16=yb, fmt=fmt, scale_layout=lay))
    if not single_entry:
        fq.rmsnorm_quant_group_multi(structs, hint=hint)
    torch.cuda.synchronize()
    res = []
    for o, ro, yb, r, p in outs:
        d = {}
        for k, gb in o.items():
            gb.check(k)
        N = p["x"].shape[1]
        for k in ("residual_out", "bf16"):
            if k in o and o[k].t.dim() == 2 and o[k].t.shape[1] > N:
                pad = host(o[k].t)[:, N:]
                assert np.all(pad == 0xA5A5), f"{k}: row padding written"
        d["q"] = host(o["q"].t)
        d["scale"] = host(o["scale"].t)
        if ro is not None:
            d["residual_out"] = host(ro)
        if yb is not None:
            d["bf16"] = host(yb)
        lay = p.get("scale_layout", 0)
        if p["x"].shape[0] and lay == 0:
            d["scale"] = d["scale"].reshape(p["x"].shape[0], -1)
        elif p["x"].shape[0] and lay == 2:
            d["scale"] = d["scale"].reshape(-1, p["x"].shape[0])
        res.append(d)
    return res


def run_oracle(orc, p):
    M, N = p["x"].shape
    fmt = p.get("fmt", 0)
    return orc.rmsnorm_quant_group(p["x"], p["gamma"], p["eps"], residual=p.get("residual"),
                                   group=128 if fmt == 0 else 32, fmt=fmt,
                                   scale_layout=p.get("scale_layout", 0),
                                   keep_bf16=True, scale_fill=SENT if fmt == 1 else 0)


def check(orc, problems, single_entry=False, strict=True, hint=None):
    got = run_gpu(problems, single_entry, hint)
    reps = []
    for g, p in zip(got, problems):
        want = run_oracle(orc, p)
        if p.get("fmt", 0) == 1 and p.get("scale_layout", 0) == 1:
            M, G = p["x"].shape[0], p["x"].shape[1] // 32
            owned = np.array([(m // 32) * 32 * G + gi * 32 + m % 32 for m in range(M) for gi in range(G)], np.int64)
            g = dict(g, scale=g["scale"][owned])
            want = dict(want, scale=want["scale"][owned])
        if p.get("scale_layout", 0) == 2:
            assert g["scale"].shape == want["scale"].shape
            g = dict(g, scale=g["scale"].T.copy())
            want = dict(want, scale=want["scale"].T.copy())
        reps.append(compare(g, want, p.get("fmt", 0), (orc.e4m3fn_table(), orc.e2m1_table()), strict,
                            yb_ref=want["bf16"]))
    return reps


def _cfg(name, M=None):
    c = inputs.make_config(name, M)
    p = {"x": c["x"], "gamma": c["gamma"], "eps": c["eps"], "fmt": c["fmt"], "keep_bf16": c["keep_bf16"]}
    if "residual" in c:
        p["residual"] = c["residual"]
    return p


# ----------------------------------------------------------- workloads --
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill512", "prefill"])
def test_fp8_workloads_full_size(orc, name):
    say(f"workload {name}")
    p = _cfg(name)
    rep = check(orc, [p])[0]
    say(f"{name}: {rep}")


@pytest.mark.parametrize("layout", [0, 1])
def test_mxfp4_workload_full_size(orc, layout):
    say(f"workload mxfp4 layout {layout}")
    p = dict(_cfg("mxfp4"), scale_layout=layout)
    check(orc, [p])


@pytest.mark.parametrize("fmt", [0, 1])
def test_column_major_scales(orc, fmt):
    say(f"column-major scales fmt {fmt}")
    for M in (1, 37, 512):
        p = inputs.make_problem(M, 7168, seed_x=60 + M, residual=True, outliers=True)
        check(orc, [dict(p, fmt=fmt, scale_layout=2, keep_bf16=True)])
    c = _cfg("prefill" if fmt == 0 else "mxfp4")
    check(orc, [dict(c, scale_layout=2)])


def test_mla_two_problems_one_launch_from_one_projection_buffer(orc):
    """q (N=1536) and kv (N=512) latents as strided column slices of one
    [4096, 2112] projection output, normalized and quantized in one launch."""
    say("workload mla")
    c = inputs.make_config("mla")
    pq, pk = c["problems"]
    probs = [{"x": pq["x"], "gamma": pq["gamma"], "eps": 1e-6, "ldx": 2112},
             {"x": pk["x"], "gamma": pk["gamma"], "eps": 1e-6, "ldx": 2112}]
    check(orc, probs)
    # in 4-chunk steps (the kv rows then use one of four)
    say("workload mla hint J=4")
    check(orc, probs, hint=fq.launch_hint(4, 1))


def test_single_entry_point(orc):
    say("single entry point, decode")
    check(orc, [_cfg("decode")], single_entry=True)
    check(orc, [dict(_cfg("tiny"), keep_bf16=True)], single_entry=True)
    check(orc, [dict(_cfg("mxfp4", M=96))], single_entry=True)


# --------------------------------------------------------- shape sweeps --
@pytest.mark.parametrize("fmt", [0, 1])
def test_shape_sweep_ragged(orc, fmt):
    Ns = [128, 256, 384, 512, 640, 896, 1024, 1536, 2048, 2176, 4096, 7168, 8192, 16384, 32768]
    if fmt == 1:
        Ns = [32, 96, 160] + Ns
    for i, N in enumerate(Ns):
        M = [1, 3, 37][i % 3]
        say(f"sweep fmt {fmt} M {M} N {N}")
        p = inputs.make_problem(M, N, seed_x=1000 + N, residual=(i % 2 == 0), outliers=True)
        p.update(fmt=fmt, keep_bf16=True)
        check(orc, [p])


@pytest.mark.parametrize("N", [7168, 1536, 512])
def test_every_launch_shape_gives_the_same_result(orc, N):
    p = inputs.make_problem(40, N, seed_x=77, residual=True, outliers=True)
    p.update(fmt=0, keep_bf16=True)
    want = None
    C = N // 8
    for J in (1, 2, 3, 4, 7, 8, 14):
        for W in range(1, 17):
            if J * W * 64 < C or (J >= 7 and W > 4) or (J * (W - 1) * 64 >= C and W > 1):
                continue
            say(f"shape J={J} W={W} N={N}")
            h = fq.launch_hint(J, W)
            check(orc, [p], hint=h)
            got = run_gpu([p], hint=h)[0]
            if want is None:
                want = got
            for k in got:
                assert np.array_equal(got[k], want[k]), (J, W, k)


@pytest.mark.parametrize("R", [2, 3, 4, 8, 16])
def test_rows_packed_one_per_wave(orc, R):
    """Short rows packed R per workgroup (one per wave): ragged row counts,
    both formats, every scale layout, with and without residual, two problems
    of different widths, and forced XCD row grouping."""
    for k, (M, N, fmt, lay, res) in enumerate([(1030, 1536, 0, 0, False), (37, 512, 1, 1, True),
                                                 (257, 2048, 0, 2, True), (65, 256, 1, 2, False)]):
        say(f"packed rows R={R} M={M} N={N} fmt={fmt} layout={lay}")
        p = inputs.make_problem(M, N, seed_x=600 + k, residual=res, outliers=True)
        check(orc, [dict(p, fmt=fmt, scale_layout=lay, keep_bf16=(k % 2 == 0))],
              hint=fq.launch_hint(waves_per_workgroup=R))
    a = inputs.make_problem(515, 1536, seed_x=610, residual=False, outliers=True)
    b = inputs.make_problem(299, 512, seed_x=611, residual=False, outliers=True)
    for g in (0, 16, 64):
        check(orc, [dict(a, fmt=0, scale_layout=2), dict(b, fmt=0, scale_layout=0, keep_bf16=True)],
              hint=fq.launch_hint(waves_per_workgroup=R, row_group=g))


@pytest.mark.parametrize("R", [2, 8])
def test_rows_packed_by_lanes(orc, R):
    """Rows of at most 256 elements packed 16 or 32 lanes each (4 or 2 rows
    per wave, one chunk per lane): row counts that leave a problem's last
    wave part empty, rows narrower than their lanes, both formats, every
    scale layout (the tiled MXFP4 layout with the rows of one tile spread
    over several waves), residual or not, and problems of different widths
    and lanes in one launch."""
    for k, (M, N, fmt, lay, res, T) in enumerate([
            (37, 128, 0, 0, True, 16), (65, 256, 1, 1, False, 32), (130, 128, 0, 2, True, 32),
            (33, 192, 1, 0, False, 32), (70, 64, 1, 2, False, 16), (41, 256, 0, 0, True, 32)]):
        say(f"packed by lanes R={R} M={M} N={N} fmt={fmt} layout={lay} lanes={T}")
        p = inputs.make_problem(M, N, seed_x=620 + k, residual=res, outliers=True)
        check(orc, [dict(p, fmt=fmt, scale_layout=lay, keep_bf16=(k % 2 == 0))],
              hint=fq.launch_hint(waves_per_workgroup=R, lanes_per_row=T))
    a = inputs.make_problem(515, 512, seed_x=630, residual=False, outliers=True)
    b = inputs.make_problem(299, 256, seed_x=631, residual=False, outliers=True)
    c = inputs.make_problem(45, 128, seed_x=632, residual=False, outliers=True)
    say(f"packed by lanes R={R} three widths (64 / 32 / 16 lanes)")
    check(orc, [dict(a, fmt=0, scale_layout=2), dict(b, fmt=0, scale_layout=0, keep_bf16=True),
                dict(c, fmt=0, scale_layout=0)], hint=fq.launch_hint(waves_per_workgroup=R))


def test_every_lane_count_gives_the_same_result(orc):
    """The same 128-wide rows packed 64, 32 or 16 lanes each give identical
    outputs (one chunk per lane; the statistics' summation tree is the same)."""
    p = inputs.make_problem(44, 128, seed_x=640, residual=True, outliers=True)
    p.update(fmt=0, keep_bf16=True)
    want = None
    for T in (64, 32, 16):
        say(f"lanes T={T}")
        h = fq.launch_hint(waves_per_workgroup=4, lanes_per_row=T)
        check(orc, [p], hint=h)
        got = run_gpu([p], hint=h)[0]
        if want is None:
            want = got
        for k in got:
            assert np.array_equal(got[k], want[k]), (T, k)


@pytest.mark.parametrize("S", [2, 4, 8])
def test_rows_split_over_workgroups(orc, S):
    """Each row split over S workgroups (every one recomputes the row's
    statistics and handles its share of the groups): both formats, scale
    layouts, residual or not, ragged widths whose groups do not divide
    evenly, and two problems of different widths in one launch."""
    h = fq.launch_hint(row_splits=S)
    for k, (M, N, fmt, lay, res) in enumerate([(64, 7168, 0, 0, True), (5, 7168, 1, 1, True),
                                                 (33, 1536, 0, 2, False), (7, 384, 1, 2, False),
                                                 (3, 128, 0, 0, True), (9, 32768, 0, 0, True)]):
        say(f"row splits S={S} M={M} N={N} fmt={fmt} layout={lay}")
        p = inputs.make_problem(M, N, seed_x=700 + k, residual=res, outliers=True)
        check(orc, [dict(p, fmt=fmt, scale_layout=lay, keep_bf16=(k % 2 == 0))], hint=h)
    a = inputs.make_problem(40, 1536, seed_x=710, residual=False, outliers=True)
    b = inputs.make_problem(24, 512, seed_x=711, residual=False, outliers=True)
    check(orc, [dict(a, fmt=0, scale_layout=2), dict(b, fmt=0, scale_layout=0, keep_bf16=True)], hint=h)
    # an in-place residual is never split (the library keeps one workgroup per row)
    c = inputs.make_problem(16, 7168, seed_x=712, residual=True, outliers=True)
    check(orc, [dict(c, fmt=0, keep_bf16=True, inplace=True)], hint=h)


def test_automatic_row_splits_for_decode(orc):
    """The decode workload (64 rows) takes the automatic split; its result is
    the oracle's, and the same with splitting switched off."""
    say("decode with automatic row splits")
    p = dict(_cfg("decode"), keep_bf16=True)
    check(orc, [p])
    auto = run_gpu([p])[0]
    one = run_gpu([p], hint=fq.launch_hint(row_splits=1))[0]
    for k in auto:
        assert np.array_equal(auto[k], one[k]), k


# ------------------------------------------------------------ edge cases --
def test_zero_rows_zero_groups_and_signed_zeros(orc):
    say("edge: zeros")
    N = 512
    x = inputs.normal_rows(6, N, 5, False)
    x[0] = 0.0                              # zero row
    x[1, 128:256] = 0.0                     # zero group (FP8) / four zero groups (MXFP4)
    x[2, :] = -0.0                          # negative zero row
    x[3, ::2] = -0.0
    g = inputs.gamma_vec(N, 7)
    for fmt in (0, 1):
        for eps in (0.0, 1e-6):
            p = {"x": inputs.to_bf16_bits(x), "gamma": g, "eps": eps, "fmt": fmt, "keep_bf16": True}
            check(orc, [p])


def test_tiny_and_huge_rows_take_the_exact_path(orc):
    say("edge: extreme magnitudes")
    N = 1024
    x = inputs.normal_rows(8, N, 6, True)
    x[0] *= np.float32(1e-30)               # inv ~ 1e30 with eps = 0
    x[1] *= np.float32(1e30)                # inv ~ 1e-30
    x[2] *= np.float32(1e-38)               # bf16 subnormal inputs
    x[3, :128] *= np.float32(1e-35)         # a group whose scale is an fp32 subnormal
    x[4, 128:256] = np.float32(2.0 ** -130) # tiny constant group
    g = inputs.gamma_vec(N, 8)
    for fmt in (0, 1):
        for eps in (0.0, 1e-6):
            p = {"x": inputs.to_bf16_bits(x), "gamma": g, "eps": eps, "fmt": fmt, "keep_bf16": True}
            check(orc, [p])


def test_gamma_products_outside_the_fp32_range(orc):
    """Gamma columns so small that h * gamma is an fp32 denormal, or so large
    that it overflows fp32, in rows whose norm keeps y finite: those elements
    take the fp64 path and still match the oracle."""
    say("edge: h * gamma outside the fp32 normal range")
    N = 1024
    g = inputs.gamma_vec(N, 9).view(np.uint16).copy()
    gf = inputs.gamma_vec(N, 9).view(np.uint16)
    small = inputs.to_bf16_bits(np.float32(2.0 ** -130) * (1 + np.arange(128, dtype=np.float32) / 128))
    g[128:256] = small                                   # bf16 denormal gammas: h * g denormal in fp32
    g[256:320] = inputs.to_bf16_bits(np.float32(2.0 ** 100) * np.ones(64, np.float32))
    x = inputs.normal_rows(6, N, 16, False)
    x[3:] *= np.float32(2.0 ** 30)                       # h * 2^100 overflows fp32; inv ~ 2^-30 keeps y finite
    for fmt in (0, 1):
        p = {"x": inputs.to_bf16_bits(x), "gamma": g, "eps": 1e-6, "fmt": fmt, "keep_bf16": True}
        check(orc, [p])
    assert not np.array_equal(g, gf)


def tie_rows(M, N, seed):
    """Rows with gamma = 1, eps = 0 and sum(h^2) = 4N exactly, so inv = 1/2 and
    y = h/2 with no rounding. Every 32-block starts with +-3.5 (group amax
    1.75 after the norm: FP8 scale 2^-8, MXFP4 scale 2^-2) and holds values
    whose quotients are exact e4m3fn midpoints (2.125 ... 3.375, 1.0625,
    1.1875, 0.53125 before the norm) and exact e2m1 midpoints (0.25 ... 5 in
    units of the MXFP4 scale); the rest is filled so the squares add up."""
    rng = np.random.default_rng(seed)
    fp8_ties = [2.125, 2.375, 2.625, 2.875, 3.125, 3.375, 1.0625, 1.1875, 0.53125]
    e2m1_ties = [0.125, 0.375, 0.625, 0.875, 1.25, 1.75, 2.5]    # y / X = 0.25 ... 5 with X = 2^-2
    fixed = [3.5] + fp8_ties + e2m1_ties
    rows = []
    for m in range(M):
        h = np.zeros(N, np.float64)
        for b0 in range(0, N, 32):
            h[b0:b0 + len(fixed)] = np.array(fixed) * rng.choice([-1, 1], len(fixed))
        R = 4.0 * N - float((h ** 2).sum())
        free = list(np.flatnonzero(h == 0))
        for v in (2.0, 1.0, 0.5, 0.25, 0.125, 0.0625, 0.03125):
            while R >= v * v and free:
                h[free.pop()] = v * rng.choice([-1, 1])
                R -= v * v
        assert R == 0 and (h ** 2).sum() == 4.0 * N, R
        rows.append(h)
    return inputs.to_bf16_bits(np.array(rows, np.float32))


def test_tie_heavy_rows_exact_codes(orc):
    say("edge: ties")
    N = 1024
    x = tie_rows(16, N, 9)
    g = inputs.to_bf16_bits(np.ones(N, np.float32))
    check(orc, [{"x": x, "gamma": g, "eps": 0.0, "fmt": 0, "keep_bf16": True}])
    check(orc, [{"x": x, "gamma": g, "eps": 0.0, "fmt": 1, "keep_bf16": True}])


def bf16_tie_rows(M, N, seed):
    """Rows whose normalized values sit exactly on bf16 rounding midpoints
    with gamma = 1.5 and eps = 0: sum(h^2) = 4N exactly, so inv = 1/2, and
    about a quarter of each row are values h in [2, 4) whose product 1.5 h
    needs one bit more than bf16 holds (the ninth significant bit set, or the
    two dropped bits 10): y = 0.75 h is then a tie. The rest are +-2 and
    smaller powers of two that make the squares add up."""
    rng = np.random.default_rng(seed)
    mant = np.arange(128, 256)
    p = 3 * mant
    tie = ((p < 512) & (p % 2 == 1)) | ((p >= 512) & (p % 4 == 2))
    vals = mant[tie] / 64.0                      # 8 significant bits, in [2, 4)
    rows = []
    for m in range(M):
        h = np.zeros(N, np.float64)
        k = N // 4
        h[:k] = rng.choice(vals, k) * rng.choice([-1, 1], k)
        R = 4.0 * N - float((h ** 2).sum())
        free = list(range(k, N))
        rng.shuffle(free)
        for v in (2.0, 1.0, 0.5, 0.25, 0.125, 0.0625, 0.03125, 0.015625):
            while R >= v * v and free:
                h[free.pop()] = v * rng.choice([-1, 1])
                R -= v * v
        assert R == 0 and (h ** 2).sum() == 4.0 * N, R
        rows.append(rng.permutation(h))
    return inputs.to_bf16_bits(np.array(rows, np.float32))


def test_bf16_ties_and_near_ties_through_the_kernel(orc):
    """Exact bf16 ties of the normalized value (eps = 0: inv = 1/2 exactly)
    take the even bf16 and the codes derived from it; with eps = 2^-30 the
    same products lie about 2^-34 below their midpoints (inv a hair under
    1/2, fl32(inv) still 1/2), which the rare path decides in fp32 from
    inv_lo. Both against the oracle, FP8 and MXFP4, with the bf16 output,
    in one-row-per-wave and row-spanning launches."""
    say("edge: bf16 ties through the kernel")
    for N, M in ((1024, 64), (7168, 8)):
        x = bf16_tie_rows(M, N, 21 + N)
        g = inputs.to_bf16_bits(np.full(N, 1.5, np.float32))
        for eps in (0.0, 2.0 ** -30):
            for fmt in (0, 1):
                check(orc, [{"x": x, "gamma": g, "eps": eps, "fmt": fmt, "keep_bf16": True}])


def _inv_like_the_definition(ss, N, eps32):
    """fl64(1 / fl64(sqrt(fl64(ss / N) + eps))) for an exact fp64 ss."""
    d = np.float64(ss) / np.float64(N) + np.float64(np.float32(eps32))
    return np.float64(1.0) / np.sqrt(d)


def side_crossing_row(N, sign, seed):
    """One row (bf16 bits), gamma = 1 and an fp32 eps such that the row's
    values +-h0 normalize to y = h0 * inv just past a bf16 rounding midpoint
    M0, while the fp32 product with fl32(inv) lands on the side value of the
    row's window and rounds the other way: inv lies 0.30 to 0.48 of an fp32
    ulp from the fp32 grid, past M0 / h0 on the side the window covers (above
    it with fl32(inv) below, sign = +1; below it with fl32(inv) above,
    sign = -1). An eighth of the row holds +-h0, the rest powers of two that
    make the sum of squares exact; eps places inv. Returns x, gamma, eps,
    h0 and M0."""
    rng = np.random.default_rng(seed)
    mids = (2 * np.arange(128) + 257) / 256.0                 # bf16 midpoints in (1, 2)
    for _ in range(20000):
        h0 = rng.integers(128, 256) / 128.0
        M0 = float(rng.choice(mids))
        q = M0 / h0
        if not 0.6 <= q < 2.0:
            continue
        lo = np.float32(q)
        if np.float64(lo) > q:
            lo = np.nextafter(lo, np.float32(0))
        ulp = np.float64(np.nextafter(lo, np.float32(4))) - np.float64(lo)
        frac = (q - np.float64(lo)) / ulp
        if not (0.30 <= frac <= 0.48 if sign > 0 else 0.52 <= frac <= 0.70):
            continue
        k = N // 8
        h = np.zeros(N)
        h[:k] = h0 * rng.choice([-1.0, 1.0], k)
        target = 1.0 / (q * (1.0 + sign * 2.0 ** -30)) ** 2
        ss = np.floor((N * target - N * 2.0 ** -12) * 2.0 ** 16) / 2.0 ** 16
        R = ss - k * h0 * h0
        free = list(range(k, N))
        for v in (2.0, 1.0, 0.5, 0.25, 0.125, 0.0625, 0.03125, 0.015625, 0.0078125, 0.00390625):
            while R >= v * v and free:
                h[free.pop()] = v * rng.choice([-1.0, 1.0])
                R -= v * v
        if R != 0 or float((h * h).sum()) != ss:
            continue
        eps0 = np.float32(target - ss / N)
        for t in sorted(range(-3000, 3001), key=abs):
            eps = np.float32(eps0 + np.float32(t) * (np.nextafter(eps0, np.float32(1)) - eps0))
            if eps < 0:
                continue
            inv = _inv_like_the_definition(ss, N, eps)
            Y = np.float64(h0) * inv
            y32 = np.float32(h0) * np.float32(inv)
            L = int(np.array(y32, np.float32).view(np.uint32)) & 0xFFFF
            if sign > 0 and Y > M0 and y32 < M0 and L == 0x7FFF:
                break
            if sign < 0 and Y < M0 and y32 > M0 and L == 0x8001:
                break
        else:
            continue
        x = inputs.to_bf16_bits(rng.permutation(h).astype(np.float32))
        return x, inputs.to_bf16_bits(np.ones(N, np.float32)), float(eps), h0, M0
    raise AssertionError("no side-crossing row found")


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("N, M", [(128, 1024), (256, 1024), (512, 1), (512, 1024), (1024, 1), (1024, 1024),
                                  (7168, 1), (7168, 64)])
def test_window_side_values_through_the_kernel(orc, N, M, sign):
    """The midpoint window's side value (0x7FFF in rows with fl32(inv) <= inv,
    0x8001 in the others) must be redone: rows built so that the fp32 product
    of the values +-h0 lands there while the definition's value lies past
    the midpoint on the other side. Checked on the host first (the rows do
    cross), then the kernel against the oracle in every launch shape these
    sizes take (rows over one or several waves, rows packed one per wave,
    rows split over workgroups, rows packed 16 or 32 lanes each with a window
    per lane; the split and the direct rare paths)."""
    say(f"edge: window side values N={N} M={M} sign={sign}")
    x, g, eps, h0, M0 = side_crossing_row(N, sign, 100 + N + (sign > 0))
    xr = np.repeat(x[None, :], M, axis=0)
    want = run_oracle(orc, {"x": xr[:1], "gamma": g, "eps": eps, "fmt": 0})
    yb = want["bf16"].reshape(1, -1).view(np.uint16)[0]
    hv = (x.astype(np.uint32) << 16).view(np.float32)
    inv = _inv_like_the_definition(float((hv.astype(np.float64) ** 2).sum()), N, eps)
    y32 = (hv * np.float32(inv)).astype(np.float32)
    b32 = ((y32.view(np.uint32) + 0x7FFF + ((y32.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    sel = np.abs(hv) == np.float32(h0)
    L = y32.view(np.uint32)[sel] & 0xFFFF
    assert sel.sum() == N // 8 and np.all(L == (0x7FFF if sign > 0 else 0x8001))
    assert np.all(b32[sel] != yb[sel])          # the fp32 product alone would round the wrong way
    for fmt in (0, 1):
        check(orc, [{"x": xr, "gamma": g, "eps": eps, "fmt": fmt, "keep_bf16": True}])


def test_window_side_values_mla_launch(orc):
    """The side-value rows in the MLA launch shape: 1536-wide rows (fl32(inv)
    below inv) and 512-wide rows (fl32(inv) above inv) as two problems of one
    call, 1024 rows each (rows packed one per wave, steps past the shorter
    rows skipped), and the 1536-wide rows alone (three chunks per lane, exact
    tails)."""
    say("edge: window side values, MLA launch")
    xa, ga, ea, _, _ = side_crossing_row(1536, 1, 301)
    xb, gb, eb, _, _ = side_crossing_row(512, -1, 302)
    pa = {"x": np.repeat(xa[None, :], 1024, axis=0), "gamma": ga, "eps": ea, "fmt": 0, "keep_bf16": True}
    pb = {"x": np.repeat(xb[None, :], 1024, axis=0), "gamma": gb, "eps": eb, "fmt": 0, "keep_bf16": True}
    check(orc, [pa, pb])
    check(orc, [pa])
    check(orc, [dict(pa, fmt=1), dict(pb, fmt=1)])


def test_strides_inplace_and_tiles(orc):
    say("edge: strides, in place, tiles")
    p = inputs.make_problem(33, 7168, seed_x=31, residual=True, outliers=True)
    check(orc, [dict(p, fmt=0, keep_bf16=True, ldx=7168 + 64, ldr=7168 + 8, ldb=7176)])
    check(orc, [dict(p, fmt=0, keep_bf16=True, inplace=True)])
    check(orc, [dict(p, fmt=1, scale_layout=1, keep_bf16=True, inplace=True)])
    check(orc, [dict(p, fmt=1, scale_layout=1, keep_bf16=False)])
    q = inputs.make_problem(1, 7168, seed_x=32, residual=True, outliers=True)
    check(orc, [dict(q, fmt=0, keep_bf16=True)])
    check(orc, [dict(q, fmt=1, scale_layout=1)])


def test_four_problems_mixed(orc):
    say("edge: four problems")
    ps = []
    for i, (M, N, res) in enumerate([(5, 7168, True), (64, 1536, False), (1, 512, True), (70, 256, False)]):
        p = inputs.make_problem(M, N, seed_x=50 + i, residual=res, outliers=True)
        ps.append(dict(p, fmt=1, scale_layout=i % 2, keep_bf16=bool(i % 2)))
    check(orc, ps)
    for p in ps:
        p["fmt"] = 0
        p["scale_layout"] = 0
    check(orc, ps)


def test_m_zero_problem_is_skipped(orc):
    say("edge: M = 0")
    p0 = inputs.make_problem(0, 512, seed_x=3, residual=True)
    p1 = inputs.make_problem(3, 512, seed_x=4, residual=True)
    got = run_gpu([dict(p0, fmt=0), dict(p1, fmt=0, keep_bf16=True)])
    assert got[0]["q"].size == 0
    check(orc, [dict(p1, fmt=0, keep_bf16=True)])


def test_repeatable(orc):
    say("repeatability")
    p = dict(_cfg("decode"), keep_bf16=True)
    a = run_gpu([p])[0]
    b = run_gpu([p])[0]
    for k in a:
        assert np.array_equal(a[k], b[k])


def test_fused_convenience_wrapper_tuples():
    say("tuple wrapper")
    p = _cfg("decode")
    x, r, g = dev(p["x"]), dev(p["residual"]), dev(p["gamma"])
    (q, s), res = fq.fused_rmsnorm_quant(x, g, 1e-6, residual=r)
    (yb, q2, s2), res2 = fq.fused_rmsnorm_quant(x, g, 1e-6, residual=r, keep_bf16=True)
    torch.cuda.synchronize()
    assert q.shape == (64, 7168) and s.shape == (64, 56) and res.shape == (64, 7168)
    assert torch.equal(q, q2) and torch.equal(s, s2) and torch.equal(res, res2)
    (q4, s4), _ = fq.fused_rmsnorm_quant(x, g, 1e-6, fmt="mxfp4", scale_layout="tiled32")
    torch.cuda.synchronize()
    assert q4.shape == (64, 3584) and s4.numel() == 64 * 224
    with pytest.raises(fq.RmsqError):
        fq.fused_rmsnorm_quant(x[:, :100], g[:100], 1e-6)   # N = 100: no whole FP8 group


def test_fused_convenience_wrapper_padded_residual():
    """A residual that is a view with padded rows: the residual output is
    allocated with the same row stride (the library writes it with that
    stride) and equals the contiguous call's, and the padding stays as it was."""
    say("wrapper, padded residual rows")
    p = _cfg("decode")
    x, r, g = dev(p["x"]), dev(p["residual"]), dev(p["gamma"])
    big = torch.full((64, 7168 + 64), 7.0, dtype=torch.bfloat16, device="cuda")
    big[:, :7168] = r
    rv = big[:, :7168]
    (q, s), res = fq.fused_rmsnorm_quant(x, g, 1e-6, residual=r)
    (qv, sv), resv = fq.fused_rmsnorm_quant(x, g, 1e-6, residual=rv)
    torch.cuda.synchronize()
    assert resv.stride() == rv.stride()
    assert torch.equal(q, qv) and torch.equal(s, sv) and torch.equal(res, resv)
    (qi, si), resi = fq.fused_rmsnorm_quant(x, g, 1e-6, residual=rv, inplace_residual=True)
    torch.cuda.synchronize()
    assert resi.data_ptr() == rv.data_ptr() and torch.equal(resi, res) and torch.equal(qi, q)
    assert torch.all(big[:, 7168:] == 7.0)
