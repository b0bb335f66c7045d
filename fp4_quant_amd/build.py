"""Build librmsq.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librmsq.so")
# translation units of the library: the fused kernels' ABI and the GEMMs' ABI
SOURCES = ("rmsq_abi.hip", "rmsq_gemm_abi.hip")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    # only the C ABI of include/rmsq.h is exported
    "-fvisibility=hidden",
    # lane flags are combined with bitwise | on purpose: no short-circuit branches
    "-Wno-bitwise-instead-of-logical",
    # the fused kernel's 9 leading int arguments arrive preloaded in SGPRs
    # (the code object keeps a fallback that loads them when the firmware
    # does not preload)
    "-mllvm", "-amdgpu-kernarg-preload-count=9",
]


def build(verbose: bool = False, extra=()) -> str:
    cmd = [HIPCC, *HIP_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, f) for f in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(LIB + ".tmp", LIB)
    write_build_info()
    return LIB


def write_build_info() -> None:
    """Record the checkout's HEAD next to the library (build_info.json, not
    versioned), so a copy of the tree without its git metadata can still name
    the commit it was built from."""
    import json
    info = {"git_sha": None, "git_modified": None}
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=20)
        if r.returncode == 0:
            info["git_sha"] = r.stdout.strip()
            d = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"],
                               capture_output=True, text=True, timeout=20)
            info["git_modified"] = bool(d.stdout.strip())
    except (OSError, subprocess.SubprocessError):
        pass
    with open(os.path.join(HERE, "build_info.json"), "w") as f:
        json.dump(info, f)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
