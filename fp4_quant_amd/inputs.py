"""Seeded synthetic inputs, shared by the HIP path's tests/benchmark and the
CPU oracle's tests. This module holds none of the method's arithmetic: it
draws numbers and converts them to bf16 with torch's own cast.

Recipe (the pages measure on served models and GSM8K / random-token serving;
these tensors stand in for the activations at the shapes those runs feed the
norm: chunked prefill of 8192 tokens, decode batches of 64, hidden 7168, MLA
latents of 1536 and 512):

* x ~ N(0, 1), drawn in float32 by numpy's PCG64 with seed ``seed_x``.
* outlier channels: 1% of the columns (``round(0.01 * N)``), chosen once with
  ``default_rng(3).choice(N, k, replace=False)``, scaled by 50 before rounding.
* residual ~ N(0, 1), seed ``seed_x + 1``.
* gamma ~ U(0.5, 1.5), seed ``seed_x + 2``.
* every value rounded to bf16 by ``torch.Tensor.to(torch.bfloat16)``.

The A16WFP4 GEMM (``make_gemm``) takes activations drawn as x above (seed
``seed``, with the outlier channels) and random MXFP4 weights: code bytes
uniform over 0..255 (two e2m1 codes each, seed ``seed + 1``) and e8m0 scale
bytes uniform over 116..123 (seed ``seed + 2``), the scales of 1x32 groups of
N(0, 0.02) weights. Its workload is the projection that follows the attention
input norm of a 7168-wide model (1536 + 576 outputs) at a decode batch of 4.
The A16W8 GEMM (``make_gemm8``) takes the same activations and random FP8
weights: e4m3fn code bytes uniform over the 254 non-NaN codes (seed
``seed + 1``) and fp32 128x128 block scales uniform over [1e-4, 1e-3] (seed
``seed + 2``), the range of amax/448 for blocks of N(0, 0.02) weights.

bf16 tensors are returned as numpy ``uint16`` bit patterns.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def outlier_channels(N: int) -> np.ndarray:
    k = int(round(0.01 * N))
    return np.sort(np.random.default_rng(3).choice(N, k, replace=False))


def normal_rows(M: int, N: int, seed: int, outliers: bool) -> np.ndarray:
    a = np.random.default_rng(seed).standard_normal((M, N), dtype=np.float32)
    if outliers:
        a[:, outlier_channels(N)] *= np.float32(50.0)
    return a


def gamma_vec(N: int, seed: int) -> np.ndarray:
    return to_bf16_bits(np.random.default_rng(seed).uniform(0.5, 1.5, N).astype(np.float32))


def make_problem(M: int, N: int, *, seed_x: int = 0, residual: bool = True,
                 outliers: bool = True) -> dict:
    p = {"x": to_bf16_bits(normal_rows(M, N, seed_x, outliers)),
         "gamma": gamma_vec(N, seed_x + 2), "eps": 1e-6}
    if residual:
        p["residual"] = to_bf16_bits(normal_rows(M, N, seed_x + 1, False))
    return p


# Workloads: name -> description. "fmt" 0 = FP8 e4m3fn group 128, 1 = MXFP4
# group 32. "layouts" lists the scale layouts the workload is run with.
CONFIGS = {
    "tiny": dict(M=4, N=256, fmt=0, group=128, residual=False, keep_bf16=False, outliers=False),
    "decode": dict(M=64, N=7168, fmt=0, group=128, residual=True, keep_bf16=False, outliers=True),
    "prefill": dict(M=8192, N=7168, fmt=0, group=128, residual=True, keep_bf16=True, outliers=True),
    "prefill512": dict(M=512, N=7168, fmt=0, group=128, residual=True, keep_bf16=True, outliers=True),
    "mxfp4": dict(M=16384, N=7168, fmt=1, group=32, residual=True, keep_bf16=False, outliers=True),
}
# Two independent latent norms in one launch (MLA q and kv), no residual.
MLA = [dict(M=4096, N=1536, seed_x=10), dict(M=4096, N=512, seed_x=20)]


GEMM = dict(M=4, N=2112, K=7168)


def fp4_weights(N: int, K: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """MXFP4 weights [N, K]: e2m1 code bytes [N, K/2] and e8m0 scale bytes [N, K/32]."""
    w = np.random.default_rng(seed).integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = np.random.default_rng(seed + 1).integers(116, 124, (N, K // 32)).astype(np.uint8)
    return w, ws


def fp8_block_weights(N: int, K: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """FP8 weights [N, K]: e4m3fn code bytes (no NaN codes) and fp32 block scales [ceil(N/128), K/128]."""
    w = np.random.default_rng(seed).integers(0, 254, (N, K), dtype=np.uint8)
    w = w + (w >= 0x7F)                           # skip 0x7F: the 254 codes 0..0x7E, 0x80..0xFE
    ws = np.random.default_rng(seed + 1).uniform(1e-4, 1e-3, (-(-N // 128), K // 128)).astype(np.float32)
    return w.astype(np.uint8), ws


def make_gemm8(M: int, N: int, K: int, seed: int = 40) -> dict:
    """bf16 activations a [M, K] and FP8 block-scaled weights (w, ws) for the A16W8 GEMM."""
    a = to_bf16_bits(normal_rows(M, K, seed, True))
    w, ws = fp8_block_weights(N, K, seed + 1)
    return {"a": a, "w": w, "ws": ws}


def make_gemm(M: int, N: int, K: int, seed: int = 40) -> dict:
    """bf16 activations a [M, K] and MXFP4 weights (w, ws) for the GEMM."""
    a = to_bf16_bits(normal_rows(M, K, seed, True))
    w, ws = fp4_weights(N, K, seed + 1)
    return {"a": a, "w": w, "ws": ws}


def make_config(name: str, M: int | None = None) -> dict:
    """Inputs for a named workload (optionally with fewer rows: the first M
    rows of the full workload, since rows are drawn in order)."""
    if name == "mla":
        return {"problems": [make_problem(M or p["M"], p["N"], seed_x=p["seed_x"],
                                          residual=False, outliers=False) for p in MLA]}
    c = CONFIGS[name]
    rows = M or c["M"]
    p = make_problem(rows, c["N"], seed_x=0, residual=c["residual"], outliers=c["outliers"])
    if name == "tiny":
        # one all-zero group, and one row that is 2^8 times another (exact in bf16)
        xf = normal_rows(rows, c["N"], 0, False)
        xf[1, 128:256] = 0.0
        xf[3] = xf[2] * np.float32(256.0)
        p["x"] = to_bf16_bits(xf)
    p.update({k: c[k] for k in ("fmt", "group", "keep_bf16")})
    return p


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
