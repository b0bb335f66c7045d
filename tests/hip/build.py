"""Build the test-only probe library (tests/hip/libconvert_probe.so) for gfx950:
number-format probes and HBM stream probes."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libconvert_probe.so")


def build(verbose: bool = False) -> str:
    sys.path.insert(0, ROOT)
    from fp4_quant_amd.build import HIPCC, HIP_FLAGS, CSRC
    cmd = [HIPCC, *HIP_FLAGS, "-I", CSRC, "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "convert_probe.hip"),
           os.path.join(HERE, "stream_probe.hip"), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(
            l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
