"""Helpers for the GPU tests: device tensors from numpy bit patterns, the
test-only probe library, and the comparator that applies the parity bar."""
from __future__ import annotations

import ctypes as C
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_PATH = os.path.join(HERE, "hip", "libconvert_probe.so")
_probe = None


def say(msg: str) -> None:
    """Name the case before each GPU step, flushed, so a failing run shows it."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def probe():
    global _probe
    if _probe is None:
        import fp4_quant_amd
        fp4_quant_amd.lib()   # torch first, so the probes share its HIP runtime
        if not os.path.exists(PROBE_PATH):
            raise RuntimeError(f"{PROBE_PATH} is not built: run __graft_entry__.build()")
        L = C.CDLL(PROBE_PATH)
        for name in ("probe_norm_bf16", "probe_fp8_scale", "probe_fp8_codes", "probe_mx_byte",
                     "probe_fp4_codes", "probe_cvt_bf16", "probe_cvt_fp8", "probe_cvt_fp4",
                     "probe_f64_to_bf16", "probe_fp8_exact", "probe_rcp", "probe_cvt_fp4_bf16_scaled",
                     "probe_cvt_fp8_bf16_scaled", "probe_mfma_scale_fp4", "probe_mfma_scale_fp8"):
            f = getattr(L, name)
            f.restype = C.c_int
        _probe = L
    return _probe


def call_probe(name: str, *tensors, n: int) -> None:
    args = [t.data_ptr() if t is not None else None for t in tensors]
    rc = getattr(probe(), name)(*[C.c_void_p(a) for a in args], C.c_int64(n),
                                C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, f"{name} launch failed"
    torch.cuda.synchronize()


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy array -> device tensor with the same bytes (uint16 -> bfloat16)."""
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_f64(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------- comparator --
def compare(got: dict, want: dict, fmt: int, tables, strict: bool = True, yb_ref=None) -> dict:
    """Apply the parity bar to one problem's outputs.

    * residual_out and bf16: bit-exact.
    * FP8 scales: relative error <= 1e-6; e8m0 scale bytes: exact.
    * codes: >= 99.99% identical as decoded values, every other one exactly
      one code step away with the oracle's quotient yb/s within 2^-20
      (relative) of that step's rounding midpoint.
    With ``strict`` the codes must also be identical as decoded values
    everywhere (the HIP path is designed to be exact). Only the outputs
    present in ``got`` are compared; ``yb_ref`` (the oracle's bf16 rows)
    feeds the tie rule. Returns counts.
    """
    rep = {}
    for key in ("residual_out", "bf16"):
        if key in got:
            diff = int(np.count_nonzero(got[key] != want[key]))
            rep[key + "_mismatch"] = diff
            assert diff == 0, f"{key}: {diff} elements differ"
    gs, ws = got["scale"], want["scale"]
    if fmt == 0:
        rel = np.abs(gs.astype(np.float64) - ws.astype(np.float64)) / np.abs(ws.astype(np.float64))
        rep["scale_max_rel"] = float(rel.max()) if rel.size else 0.0
        rep["scale_mismatch"] = int(np.count_nonzero(gs.view(np.uint32) != ws.view(np.uint32)))
        assert rep["scale_max_rel"] <= 1e-6, rep
    else:
        rep["scale_mismatch"] = int(np.count_nonzero(gs != ws))
        assert rep["scale_mismatch"] == 0, rep

    gq, wq = got["q"], want["q"]
    if fmt == 0:
        gc, wc, table = gq, wq, tables[0]
    else:
        gc = np.stack([gq & 0xF, gq >> 4], -1).reshape(gq.shape[0], -1)
        wc = np.stack([wq & 0xF, wq >> 4], -1).reshape(wq.shape[0], -1)
        table = tables[1]
    gv, wv = table[gc], table[wc]
    bad = gv != wv
    nbad = int(np.count_nonzero(bad))
    rep["codes_total"] = int(gv.size)
    rep["codes_differ"] = nbad
    if nbad:
        assert nbad <= 1e-4 * gv.size, rep
        yb = bf16_f64(yb_ref)
        M = yb.shape[0]
        G = 128 if fmt == 0 else 32
        if fmt == 0:
            s = np.repeat(ws.astype(np.float64), G, axis=1)
        else:
            s = np.repeat(2.0 ** (ws.reshape(M, -1).astype(np.float64) - 127), G, axis=1)
        quot = (yb / s)[bad]
        mid = (gv[bad] + wv[bad]) / 2
        one_step = np.abs(np.searchsorted(np.sort(np.unique(table[~np.isnan(table)])), gv[bad]) -
                          np.searchsorted(np.sort(np.unique(table[~np.isnan(table)])), wv[bad])) == 1
        assert np.all(one_step), "a code differs by more than one step"
        assert np.all(np.abs(quot - mid) <= np.abs(mid) * 2.0 ** -20), "a differing code is not at a tie"
    if strict:
        assert nbad == 0, f"codes differ from the exact result at {nbad} elements"
    return rep
