"""Register and scratch budget of the HIP kernels, read from the gfx950 code
object metadata that hipcc emits for the library source (device-only
assembly, compiled here on the CPU). Occupancy is what keeps enough bytes in
flight for the HBM-bound launches, so a change that raises the register
count of the hot variants, spills, or starts using scratch memory fails here
before it reaches a GPU.

Limits (512 VGPRs per SIMD lane slot, allocated in granules of 8):
  * J = 1, 2 (the shapes of the 7168-wide rows): at most 64 VGPRs, 8 waves per SIMD;
  * J = 3: at most 80 VGPRs, 6 waves per SIMD, and at most 64 (8 waves) for
    packed rows (the MLA latents: the whole launch resident at once); J = 4:
    at most 96, 5 waves, and 64 for packed rows quantized without a residual
    whose rows end inside the launch shape (the MLA latents with the 512-wide
    rows 16 lanes each);
  * J = 7, 8: at most 128 VGPRs, J = 14: at most 168 (4-wave workgroups);
  * no kernel spills or uses private (scratch) memory.
"""
import os
import re
import subprocess
import tempfile

import pytest

from fp4_quant_amd import build as B

NAME = re.compile(r"^_ZN4rmsq17rmsq_fused_kernelILi(\d)ELi(\d+)ELb(\d)ELi(\d)ELi(\d)EEEviiiiiiiiiNS_6LaunchE$")


@pytest.fixture(scope="module")
def kernels():
    text = ""
    with tempfile.TemporaryDirectory() as d:
        for src in B.SOURCES:
            out = os.path.join(d, src + ".s")
            flags = [f for f in B.HIP_FLAGS if f not in ("-shared", "-fPIC")]
            subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(B.ROOT, "include"),
                            "-I", B.CSRC, os.path.join(B.CSRC, src), "-o", out],
                           check=True, capture_output=True)
            text += open(out).read()
    ks = {}
    blocks = []
    for part in text.split("amdhsa.kernels:")[1:]:
        blocks += re.split(r"\n  - ", part)[1:]
    for block in blocks:
        def field(k):
            m = re.search(r"\." + k + r":\s+(\S+)", block)
            return m.group(1) if m else None
        ks[field("name")] = {k: int(field(k) or 0) for k in
                             ("vgpr_count", "agpr_count", "sgpr_count", "vgpr_spill_count", "sgpr_spill_count",
                              "private_segment_fixed_size", "group_segment_fixed_size")}
    # kernel descriptors (.amdhsa_kernel blocks) carry the preload length
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S):
        pl = re.search(r"\.amdhsa_user_sgpr_kernarg_preload_length (\d+)", m.group(2))
        if m.group(1) in ks:
            ks[m.group(1)]["kernarg_preload"] = int(pl.group(1)) if pl else 0
    return ks


def test_every_kernel_variant_is_present(kernels):
    fused = [n for n in kernels if NAME.match(n or "")]
    # 3 formats (FP8, MXFP4, norm only) x residual or not x (7 shapes + 4 packed-row shapes),
    # the 4 short shapes and 4 packed-row shapes also for rows that exactly fill the launch,
    # the 4 packed-row shapes for rows of whole 64-lane steps (uniform tail), and rows
    # packed by lanes (one chunk per lane), bounded or exact
    assert len(fused) == 3 * 2 * (7 + 4 + 4 + 4 + 4 + 2), sorted(fused)
    assert sum(1 for n in fused if NAME.match(n).group(4) == "2") == 3 * 2 * 2
    assert sum(1 for n in kernels if "rmsq_group_quant_kernel" in (n or "")) == 2


def test_launch_scalars_are_preloaded(kernels):
    """The fused kernels' nine leading int arguments are preloaded into
    SGPRs (gfx950 kernel-argument preloading)."""
    fused = [n for n in kernels if NAME.match(n or "")]
    assert fused and all(kernels[n]["kernarg_preload"] == 9 for n in fused)


def test_no_spills_and_no_scratch(kernels):
    for n, k in kernels.items():
        assert k["vgpr_spill_count"] == 0 and k["sgpr_spill_count"] == 0, (n, k)
        assert k["private_segment_fixed_size"] == 0, (n, k)


@pytest.mark.parametrize("J,limit", [(1, 64), (2, 64), (3, 80), (4, 96), (7, 128), (8, 128), (14, 168)])
def test_register_budget(kernels, J, limit):
    for n, k in kernels.items():
        m = NAME.match(n or "")
        if m and int(m.group(2)) == J:
            packed = m.group(4) != "0"
            capped = packed and (J == 3 or (J == 4 and m.group(1) != "2" and m.group(3) == "0" and m.group(5) != "1"))
            lim = 64 if capped else limit
            assert k["vgpr_count"] + k["agpr_count"] <= lim, (n, k)


def test_gemm_variants_fit_sixteen_waves(kernels):
    """The GEMM launches up to 16 waves per workgroup (4 per SIMD), fewer for
    variants with more accumulator tiles per wave, so each variant must fit
    the registers its wave count leaves (VGPRs + AGPRs) and the LDS of its
    partial sums."""
    gemm = {n: k for n, k in kernels.items() if "rmsq_gemm_fp4_kernel" in (n or "")}
    # (4 row-tile counts + the small-M variant with 1 or 2 column tiles; quantized
    # activations: 4 row-tile counts loading pairs of steps, their 4 x 2 tile
    # variant and the one-tile variant loading operands directly) x 2 weight layouts
    assert len(gemm) == 24, sorted(gemm)
    gemm8 = {n: k for n, k in kernels.items() if "rmsq_gemm_fp8_kernel" in (n or "")}
    # (1 or 2 row tiles + the small-M variant; quantized activations: 1 or 2 row tiles
    # loading 8 rows per load and the one-tile variant loading operands directly) x 2 weight layouts
    assert len(gemm8) == 12, sorted(gemm8)
    gemm.update(gemm8)
    for n, k in gemm.items():
        # waves per workgroup: 16, or fewer when MT * CT accumulator tiles per wave
        # would overflow 64 KiB of partial sums; registers per lane: 512 over the
        # waves each SIMD holds
        m = re.search(r"fp4_kernelILi(\d+)ELi\d+ELb\dELb\dELi(\d+)E", n)
        nt = int(m.group(1)) * int(m.group(2)) if m else 1
        waves = min(16, 64 // nt)
        assert k["vgpr_count"] + k["agpr_count"] <= 512 // -(-waves // 4), (n, k)
        assert k["group_segment_fixed_size"] <= 64 * 1024, (n, k)
