"""fp4_quant_amd: fused residual-add + RMSNorm + per-group FP8 / MXFP4
quantization for AMD Instinct MI355X (gfx950).

Every step of the operation runs in the HIP kernels of ``librmsq.so``; this
module only marshals arguments over its C ABI (``include/rmsq.h``), with torch
providing device memory and streams. There is no CPU fallback: if the
library is not built, or the GPU is not a gfx950, calls raise.

The raw entry points keep the C names and argument order:

* ``rmsnorm_quant_group(x, residual_in, gamma, eps, M, N, group, fmt, out_q,
  out_scale, residual_out, out_bf16_or_null, stream=None)``
* ``rmsnorm_quant_group_multi(problems, stream=None)``

``fused_rmsnorm_quant`` allocates the outputs and returns them in the tuple
shape of the pull request "[AMD] Add fused all-reduce RMSNorm per-group quant
for Qwen3.5 FP8" (Modifications): ``((q, scale), residual)`` or, with the bf16
side-output, ``((bf16, q, scale), residual)``.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librmsq.so")

RMSQ_OK, RMSQ_ERR_INVALID_ARG, RMSQ_ERR_UNSUPPORTED, RMSQ_ERR_HIP = 0, 1, 2, 3
FMT_FP8_E4M3FN, FMT_MXFP4_E2M1 = 0, 1
SCALE_ROW_MAJOR, SCALE_TILED32, SCALE_COL_MAJOR = 0, 1, 2
W_ROW_MAJOR, W_PRESHUFFLED = 0, 1
MAX_PROBLEMS = 4
N_MAX = 32768
_FMT = {"fp8": FMT_FP8_E4M3FN, "mxfp4": FMT_MXFP4_E2M1}
_GROUP = {FMT_FP8_E4M3FN: 128, FMT_MXFP4_E2M1: 32}
_LAYOUT = {"row": SCALE_ROW_MAJOR, "tiled32": SCALE_TILED32, "col": SCALE_COL_MAJOR}


class RmsqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_STATUS = {0: "RMSQ_OK", 1: "RMSQ_ERR_INVALID_ARG", 2: "RMSQ_ERR_UNSUPPORTED", 3: "RMSQ_ERR_HIP"}


class rmsq_problem(C.Structure):
    _fields_ = [("x", C.c_void_p), ("ldx", C.c_int64),
                ("residual_in", C.c_void_p), ("residual_out", C.c_void_p), ("ldr", C.c_int64),
                ("gamma", C.c_void_p), ("eps", C.c_float),
                ("M", C.c_int64), ("N", C.c_int64), ("group", C.c_int32), ("fmt", C.c_int32),
                ("scale_layout", C.c_int32),
                ("out_q", C.c_void_p), ("out_scale", C.c_void_p), ("out_bf16", C.c_void_p),
                ("ldb", C.c_int64)]


class rmsq_launch_hint(C.Structure):
    _fields_ = [("chunks_per_lane", C.c_int32), ("waves_per_row", C.c_int32), ("row_group", C.c_int32),
                ("waves_per_workgroup", C.c_int32), ("row_splits", C.c_int32), ("lanes_per_row", C.c_int32)]


class rmsq_launch_info(C.Structure):
    _fields_ = [("problems", C.c_int32), ("rows", C.c_int32), ("chunks_per_lane", C.c_int32),
                ("waves_per_row", C.c_int32), ("waves_per_workgroup", C.c_int32), ("row_splits", C.c_int32),
                ("row_group", C.c_int32), ("threads_per_workgroup", C.c_int32), ("workgroups", C.c_int64),
                ("residual", C.c_int32), ("tail", C.c_int32), ("lanes_per_row", C.c_int32 * 4)]


class rmsq_launch_plan(C.Structure):
    _fields_ = [("launches", C.c_int32), ("reserved", C.c_int32), ("launch", rmsq_launch_info * 2)]


EXPORTS = ("rmsnorm_quant_group", "rmsnorm_quant_group_multi", "rmsnorm_quant_group_multi_ex", "rmsq_plan_launch",
           "add_rmsnorm", "dynamic_per_group_scaled_quant", "rmsq_device_supported",
           "rmsq_scale_bytes", "rmsq_status_string", "rmsq_last_error", "rmsq_query_shape",
           "gemm_a16wfp4_prequant", "mxfp4_weight_preshuffle", "gemm_a16w8_prequant", "fp8_weight_preshuffle",
           "gemm_afp4wfp4", "gemm_a8w8_blockscale")

_lib = None


def lib() -> C.CDLL:
    """Load librmsq.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "(the HIP library is required; there is no CPU fallback)")
        # The library must call the same HIP runtime as the torch whose
        # streams and memory it is given. torch ships its own runtime and
        # loads it into the process-wide symbol scope, so with torch loaded
        # first the library's HIP calls bind to it; loaded before torch, they
        # would bind to the system runtime, a second runtime on the same GPU.
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        p, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
        L.rmsnorm_quant_group.restype = i32
        L.rmsnorm_quant_group.argtypes = [p, p, p, C.c_float, i64, i64, i32, i32, p, p, p, p, p]
        L.rmsnorm_quant_group_multi.restype = i32
        L.rmsnorm_quant_group_multi.argtypes = [C.POINTER(rmsq_problem), i32, p]
        L.add_rmsnorm.restype = i32
        L.add_rmsnorm.argtypes = [p, p, p, C.c_float, i64, i64, p, p, p]
        L.dynamic_per_group_scaled_quant.restype = i32
        L.dynamic_per_group_scaled_quant.argtypes = [p, i64, i64, i32, i32, i32, p, p, p]
        L.rmsq_device_supported.restype = i32
        L.rmsq_device_supported.argtypes = [i32]
        L.rmsq_scale_bytes.restype = C.c_size_t
        L.rmsq_scale_bytes.argtypes = [i64, i64, i32, i32, i32]
        L.rmsq_status_string.restype = C.c_char_p
        L.rmsq_status_string.argtypes = [i32]
        L.rmsq_last_error.restype = C.c_char_p
        L.rmsq_last_error.argtypes = []
        L.rmsnorm_quant_group_multi_ex.restype = i32
        L.rmsnorm_quant_group_multi_ex.argtypes = [C.POINTER(rmsq_problem), i32, C.POINTER(rmsq_launch_hint), p]
        L.rmsq_plan_launch.restype = i32
        L.rmsq_plan_launch.argtypes = [C.POINTER(rmsq_problem), i32, C.POINTER(rmsq_launch_hint),
                                       C.POINTER(rmsq_launch_plan)]
        L.rmsq_query_shape.restype = i32
        L.rmsq_query_shape.argtypes = [i64, i64, C.POINTER(i32), C.POINTER(i32)]
        L.gemm_a16wfp4_prequant.restype = i32
        L.gemm_a16wfp4_prequant.argtypes = [p, i64, p, p, i32, i64, i64, i64, p, i64, p]
        L.mxfp4_weight_preshuffle.restype = i32
        L.mxfp4_weight_preshuffle.argtypes = [p, p, i64, i64, p, p, p]
        L.gemm_a16w8_prequant.restype = i32
        L.gemm_a16w8_prequant.argtypes = [p, i64, p, p, i32, i64, i64, i64, p, i64, p]
        L.fp8_weight_preshuffle.restype = i32
        L.fp8_weight_preshuffle.argtypes = [p, i64, i64, p, p]
        for name in ("gemm_afp4wfp4", "gemm_a8w8_blockscale"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [p, p, i32, p, p, i32, i64, i64, i64, p, i64, p]
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != RMSQ_OK:
        raise RmsqError(status, lib().rmsq_last_error().decode())


def _ptr(t):
    """Device address of a tensor (None for None). A host tensor is refused:
    the kernels would dereference its address on the GPU."""
    if t is None:
        return None
    if getattr(t, "is_cuda", True) is False:
        raise ValueError("fp4_quant_amd: buffers must be GPU tensors (got a tensor on %s)" % t.device)
    return t.data_ptr()


def _stream(stream, device=None):
    if stream is None:
        import torch
        return torch.cuda.current_stream(device).cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ------------------------------------------------------------- raw ABI --
def rmsnorm_quant_group(x, residual_in, gamma, eps, M, N, group, fmt, out_q, out_scale,
                        residual_out, out_bf16_or_null, stream=None) -> None:
    """The C entry point with torch tensors (or None) for the buffers."""
    _check(lib().rmsnorm_quant_group(
        _ptr(x), _ptr(residual_in), _ptr(gamma), float(eps), int(M), int(N), int(group), int(fmt),
        _ptr(out_q), _ptr(out_scale), _ptr(residual_out), _ptr(out_bf16_or_null),
        _stream(stream, x.device if x is not None else None)))


def _ld(t):
    """Row stride in elements for the library (0 = N: absent, or one row,
    whose stride is never applied)."""
    return 0 if t is None or t.shape[0] <= 1 else int(t.stride(0))


def _check_rows(t, M, N, name):
    """t: [M, N] bf16 rows with unit column stride and rows that do not
    overlap (row stride >= N; the library also needs it a multiple of 8)."""
    import torch
    if M == 0:   # nothing is read or written (empty tensors may come in any shape)
        return
    if (t.dtype != torch.bfloat16 or t.dim() != 2 or tuple(t.shape) != (M, N) or (N > 1 and t.stride(1) != 1)
            or (M > 1 and t.stride(0) < N)):
        raise ValueError(f"{name} must be a [{M}, {N}] bf16 tensor with unit column stride and row stride >= N "
                         f"(got {tuple(t.shape)} {t.dtype}, strides {tuple(t.stride())})")


def _check_quant_outputs(out_q, out_scale, M, N, fmt, scale_layout):
    """out_q: M*N (FP8) or M*N/2 (MXFP4) dense uint8 code bytes; out_scale:
    dense float32 (FP8) or uint8 (MXFP4) scales holding at least the bytes the
    layout needs. The C ABI takes bare pointers and cannot see a buffer's
    size, so a short one is refused here, before any address is taken."""
    import torch
    if M == 0:
        return
    if fmt not in _GROUP:
        return   # the library reports the unknown format
    group = _GROUP[fmt]
    if N % group:
        return   # the library reports the shape
    want_q = M * N if fmt == FMT_FP8_E4M3FN else M * N // 2
    if out_q is None or out_q.dtype != torch.uint8 or out_q.numel() != want_q or not out_q.is_contiguous():
        raise ValueError(f"out_q must be {want_q} contiguous uint8 code bytes"
                         + ("" if out_q is None else f" (got {out_q.numel()} {out_q.dtype})"))
    dt = torch.float32 if fmt == FMT_FP8_E4M3FN else torch.uint8
    need = rmsq_scale_bytes(M, N, group, fmt, scale_layout)
    if out_scale is None or out_scale.dtype != dt or not out_scale.is_contiguous() or (
            need and out_scale.numel() * out_scale.element_size() < need):
        raise ValueError(f"out_scale must be contiguous {dt} holding at least {need} bytes for scale layout "
                         f"{scale_layout}" + ("" if out_scale is None else
                                              f" (got {out_scale.numel()} {out_scale.dtype})"))


def make_problem(x, gamma, eps, out_q, out_scale, *, residual_in=None, residual_out=None,
                 out_bf16=None, fmt=FMT_FP8_E4M3FN, scale_layout=SCALE_ROW_MAJOR) -> rmsq_problem:
    """One problem for ``rmsnorm_quant_group_multi``. The tensors are checked
    here for dtype, shape, size and device (the library checks strides,
    alignment, overlaps and the formats); residual_in and residual_out share
    one row stride, which the library applies to both."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, N]")
    M, N = x.shape
    _check_rows(x, M, N, "x")
    if M and (gamma.dtype != torch.bfloat16 or gamma.numel() != N or not gamma.is_contiguous()):
        raise ValueError(f"gamma must be {N} contiguous bf16 values")
    if residual_in is not None:
        _check_rows(residual_in, M, N, "residual_in")
    if residual_out is not None:
        _check_rows(residual_out, M, N, "residual_out")
        if residual_in is not None and M > 1 and residual_out.stride(0) != residual_in.stride(0):
            raise ValueError("residual_out must have the row stride of residual_in")
    if out_bf16 is not None:
        _check_rows(out_bf16, M, N, "out_bf16")
    _check_quant_outputs(out_q, out_scale, M, N, fmt, scale_layout)
    if M:
        for name, t in (("gamma", gamma), ("residual_in", residual_in), ("residual_out", residual_out),
                        ("out_bf16", out_bf16), ("out_q", out_q), ("out_scale", out_scale)):
            if t is not None and t.device != x.device:
                raise ValueError(f"{name} is on {t.device}, x on {x.device}")
    return rmsq_problem(x=_ptr(x), ldx=_ld(x), residual_in=_ptr(residual_in),
                        residual_out=_ptr(residual_out), ldr=_ld(residual_in), gamma=_ptr(gamma),
                        eps=float(eps), M=M, N=N, group=_GROUP.get(fmt, 0), fmt=fmt,
                        scale_layout=scale_layout, out_q=_ptr(out_q), out_scale=_ptr(out_scale),
                        out_bf16=_ptr(out_bf16), ldb=_ld(out_bf16))


def problem_array(problems):
    """A ctypes array of ``rmsq_problem`` to pass to the multi-problem call
    repeatedly without rebuilding it."""
    return (rmsq_problem * len(problems))(*problems)


def launch_hint(J=0, W=0, row_group=0, waves_per_workgroup=0, row_splits=0, lanes_per_row=0) -> rmsq_launch_hint:
    """A per-call launch hint (0 = the library's choice for that field)."""
    return rmsq_launch_hint(int(J), int(W), int(row_group), int(waves_per_workgroup), int(row_splits),
                            int(lanes_per_row))


def rmsnorm_quant_group_multi(problems, stream=None, hint=None) -> None:
    """Up to four independent problems (``rmsq_problem`` structs from
    ``make_problem``, or an array from ``problem_array``) in one kernel
    launch. ``stream``: a torch stream, a raw hipStream_t handle, or None for
    torch's current stream. ``hint``: an optional ``launch_hint`` for this
    call only (``rmsnorm_quant_group_multi_ex``)."""
    arr = problems if isinstance(problems, C.Array) else problem_array(problems)
    if hint is None:
        _check(lib().rmsnorm_quant_group_multi(arr, len(arr), _stream(stream)))
    else:
        _check(lib().rmsnorm_quant_group_multi_ex(arr, len(arr), C.byref(hint), _stream(stream)))


def rmsq_plan_launch(problems, hint=None):
    """The launches the library would make for these problems (and hint),
    as a list of dicts, without launching anything (no GPU needed)."""
    arr = problems if isinstance(problems, C.Array) else problem_array(problems)
    plan = rmsq_launch_plan()
    _check(lib().rmsq_plan_launch(arr, len(arr), C.byref(hint) if hint is not None else None, C.byref(plan)))
    out = []
    for k in range(plan.launches):
        d = {f: getattr(plan.launch[k], f) for f, _ in rmsq_launch_info._fields_}
        d["lanes_per_row"] = list(d["lanes_per_row"])[:d["problems"]]
        out.append(d)
    return out


def add_rmsnorm(x, residual_in, gamma, eps, M, N, residual_out, out_bf16, stream=None) -> None:
    """The add + RMSNorm kernel alone (bf16 output), C argument order."""
    _check(lib().add_rmsnorm(_ptr(x), _ptr(residual_in), _ptr(gamma), float(eps), int(M), int(N),
                             _ptr(residual_out), _ptr(out_bf16),
                             _stream(stream, x.device if x is not None else None)))


def dynamic_per_group_scaled_quant(x, M, N, group, fmt, scale_layout, out_q, out_scale, stream=None) -> None:
    """The per-group quantization alone on bf16 rows, C argument order."""
    _check(lib().dynamic_per_group_scaled_quant(_ptr(x), int(M), int(N), int(group), int(fmt),
                                                int(scale_layout), _ptr(out_q), _ptr(out_scale),
                                                _stream(stream, x.device if x is not None else None)))


def gemm_a16wfp4_prequant(a, lda, w, w_scale, w_layout, M, N, K, out, ldc, stream=None) -> None:
    """The A16WFP4 prequant GEMM (bf16 activations quantized to MXFP4 inside
    the GEMM, MXFP4 weights, fp32 output), C argument order."""
    _check(lib().gemm_a16wfp4_prequant(_ptr(a), int(lda), _ptr(w), _ptr(w_scale), int(w_layout), int(M), int(N),
                                       int(K), _ptr(out), int(ldc),
                                       _stream(stream, a.device if a is not None else None)))


def mxfp4_weight_preshuffle(w, w_scale, N, K, w_out, w_scale_out, stream=None) -> None:
    """Row-major MXFP4 weights to the preshuffled layout, C argument order."""
    _check(lib().mxfp4_weight_preshuffle(_ptr(w), _ptr(w_scale), int(N), int(K), _ptr(w_out), _ptr(w_scale_out),
                                         _stream(stream, w.device if w is not None else None)))


def gemm_a16w8_prequant(a, lda, w, w_scale, w_layout, M, N, K, out, ldc, stream=None) -> None:
    """The A16W8 prequant GEMM (bf16 activations quantized to FP8 per 1x128
    group inside the GEMM, e4m3fn weights with fp32 128x128 block scales,
    fp32 output), C argument order."""
    _check(lib().gemm_a16w8_prequant(_ptr(a), int(lda), _ptr(w), _ptr(w_scale), int(w_layout), int(M), int(N),
                                     int(K), _ptr(out), int(ldc),
                                     _stream(stream, a.device if a is not None else None)))


def gemm_afp4wfp4(a_q, a_scale, a_scale_layout, w, w_scale, w_layout, M, N, K, out, ldc, stream=None) -> None:
    """The GEMM of MXFP4 activations as the group quantization writes them
    (codes and e8m0 scales in any of its layouts) with MXFP4 weights, fp32
    output, C argument order."""
    _check(lib().gemm_afp4wfp4(_ptr(a_q), _ptr(a_scale), int(a_scale_layout), _ptr(w), _ptr(w_scale), int(w_layout),
                               int(M), int(N), int(K), _ptr(out), int(ldc),
                               _stream(stream, a_q.device if a_q is not None else None)))


def gemm_a8w8_blockscale(a_q, a_scale, a_scale_layout, w, w_scale, w_layout, M, N, K, out, ldc,
                         stream=None) -> None:
    """The GEMM of FP8 activations as the group quantization writes them
    (e4m3fn codes, fp32 1x128 scales row- or column-major) with e4m3fn weights
    and fp32 128x128 block scales, fp32 output, C argument order."""
    _check(lib().gemm_a8w8_blockscale(_ptr(a_q), _ptr(a_scale), int(a_scale_layout), _ptr(w), _ptr(w_scale),
                                      int(w_layout), int(M), int(N), int(K), _ptr(out), int(ldc),
                                      _stream(stream, a_q.device if a_q is not None else None)))


def fp8_weight_preshuffle(w, N, K, w_out, stream=None) -> None:
    """Row-major e4m3fn weights to the A16W8 GEMM's preshuffled layout."""
    _check(lib().fp8_weight_preshuffle(_ptr(w), int(N), int(K), _ptr(w_out),
                                       _stream(stream, w.device if w is not None else None)))


def rmsq_device_supported(device: int = 0) -> bool:
    return bool(lib().rmsq_device_supported(int(device)))


def rmsq_scale_bytes(M, N, group, fmt, scale_layout=SCALE_ROW_MAJOR) -> int:
    return int(lib().rmsq_scale_bytes(int(M), int(N), int(group), int(fmt), int(scale_layout)))


def rmsq_query_shape(N: int, rows: int):
    """(J, W): chunks per lane and waves per row the library picks."""
    j, w = C.c_int32(), C.c_int32()
    _check(lib().rmsq_query_shape(int(N), int(rows), C.byref(j), C.byref(w)))
    return j.value, w.value


# -------------------------------------------------------- convenience --
def alloc_outputs(M, N, fmt, scale_layout=SCALE_ROW_MAJOR, keep_bf16=False, device="cuda"):
    import torch
    q = torch.empty((M, N if fmt == FMT_FP8_E4M3FN else N // 2), dtype=torch.uint8, device=device)
    G = N // _GROUP[fmt]
    dt = torch.float32 if fmt == FMT_FP8_E4M3FN else torch.uint8
    if scale_layout == SCALE_TILED32:
        scale = torch.empty((((M + 31) // 32) * 32 * G,), dtype=dt, device=device)
    elif scale_layout == SCALE_COL_MAJOR:
        scale = torch.empty((G, M), dtype=dt, device=device)
    else:
        scale = torch.empty((M, G), dtype=dt, device=device)
    yb = torch.empty((M, N), dtype=torch.bfloat16, device=device) if keep_bf16 else None
    return q, scale, yb


def fused_rmsnorm_quant(x, gamma, eps=1e-6, residual=None, fmt="fp8", keep_bf16=False,
                        scale_layout="row", inplace_residual=False, stream=None):
    """Allocate outputs and run one fused call.

    Returns ``((q, scale), residual_out)`` or ``((bf16, q, scale), residual_out)``
    (``residual_out`` is None without a residual; it is ``residual`` itself
    when ``inplace_residual``). FP8 codes are returned as ``uint8`` (view them
    with ``.view(torch.float8_e4m3fn)``), MXFP4 codes as packed ``uint8``.
    """
    import torch
    f = _FMT[fmt] if isinstance(fmt, str) else int(fmt)
    lay = _LAYOUT[scale_layout] if isinstance(scale_layout, str) else int(scale_layout)
    M, N = x.shape
    q, scale, yb = alloc_outputs(M, N, f, lay, keep_bf16, x.device)
    res_out = None
    if residual is not None:
        # the library writes residual_out with residual's row stride
        res_out = residual if inplace_residual else torch.empty_strided(
            residual.shape, residual.stride(), dtype=residual.dtype, device=residual.device)
    p = make_problem(x, gamma, eps, q, scale, residual_in=residual, residual_out=res_out,
                     out_bf16=yb, fmt=f, scale_layout=lay)
    rmsnorm_quant_group_multi([p], stream)
    return ((yb, q, scale) if keep_bf16 else (q, scale)), res_out


def preshuffle_weights(w, w_scale, fmt="mxfp4", stream=None):
    """The prequant GEMM's faster weight layout, made once per weight matrix.

    ``fmt="mxfp4"``: ``w`` [N, K/2] uint8 e2m1 codes and ``w_scale`` [N, K/32]
    uint8 e8m0 bytes; returns both rearranged. ``fmt="fp8"``: ``w`` [N, K]
    uint8 e4m3fn codes (``w_scale``, the [ceil(N/128), K/128] fp32 block
    scales, keeps its layout and is returned as is)."""
    import torch
    N = w.shape[0]
    if fmt == "mxfp4":
        K = w.shape[1] * 2
        sw, sws = torch.empty_like(w), torch.empty_like(w_scale)
        mxfp4_weight_preshuffle(w, w_scale, N, K, sw, sws, stream)
        return sw, sws
    if fmt == "fp8":
        K = w.shape[1]
        sw = torch.empty_like(w)
        fp8_weight_preshuffle(w, N, K, sw, stream)
        return sw, w_scale
    raise ValueError(f"unknown weight format {fmt!r}")


def prequant_gemm(a, w, w_scale, fmt="mxfp4", preshuffled=False, out=None, stream=None):
    """out = a @ w^T with the bf16 activations ``a`` [M, K] quantized inside the
    GEMM: ``fmt="mxfp4"`` (1x32 MXFP4 groups; ``w`` [N, K/2] e2m1 codes,
    ``w_scale`` [N, K/32] e8m0 bytes) or ``fmt="fp8"`` (1x128 FP8 groups;
    ``w`` [N, K] e4m3fn codes, ``w_scale`` [ceil(N/128), K/128] fp32 block
    scales). ``preshuffled``: the weights come from ``preshuffle_weights``.
    Returns the fp32 [M, N] output (``out`` if given)."""
    import torch
    if a.dtype != torch.bfloat16 or a.dim() != 2 or a.stride(1) != 1:
        raise ValueError("a must be a 2-D bf16 tensor with unit column stride")
    if w.dtype != torch.uint8 or not w.is_contiguous() or not w_scale.is_contiguous():
        raise ValueError("w must be contiguous uint8 codes and w_scale contiguous")
    M, K = a.shape
    N = w.shape[0]
    if fmt == "mxfp4":
        if w.shape != (N, K // 2) or w_scale.dtype != torch.uint8 or w_scale.numel() != N * (K // 32):
            raise ValueError("MXFP4 weights: w [N, K/2] uint8 and w_scale [N, K/32] uint8")
        call = gemm_a16wfp4_prequant
    elif fmt == "fp8":
        if w.shape != (N, K) or w_scale.dtype != torch.float32 or w_scale.numel() != -(-N // 128) * (K // 128):
            raise ValueError("FP8 weights: w [N, K] uint8 and w_scale [ceil(N/128), K/128] float32")
        call = gemm_a16w8_prequant
    else:
        raise ValueError(f"unknown weight format {fmt!r}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    elif out.dtype != torch.float32 or out.shape != (M, N) or out.stride(1) != 1:
        raise ValueError("out must be a float32 [M, N] tensor with unit column stride")
    # strides of a single row are never applied: pass the dense ones
    call(a, a.stride(0) if M > 1 else K, w, w_scale, W_PRESHUFFLED if preshuffled else W_ROW_MAJOR, M, N, K, out,
         out.stride(0) if M > 1 else N, stream)
    return out


def quantized_gemm(a_q, a_scale, w, w_scale, fmt="mxfp4", scale_layout=SCALE_ROW_MAJOR, preshuffled=False, out=None,
                   stream=None):
    """out = dq(a) @ dq(w)^T for activations already quantized by
    ``fused_rmsnorm_quant`` or the standalone group quantization:
    ``fmt="mxfp4"``: ``a_q`` [M, K/2] uint8 codes, ``a_scale`` its e8m0 bytes in
    ``scale_layout`` (row-major, 32-row tiled or column-major), weights as for
    ``prequant_gemm``; ``fmt="fp8"``: ``a_q`` [M, K] uint8 e4m3fn codes,
    ``a_scale`` its fp32 scales (row- or column-major). Returns the fp32
    [M, N] output (``out`` if given)."""
    import torch
    if a_q.dtype != torch.uint8 or a_q.dim() != 2 or not a_q.is_contiguous() or not a_scale.is_contiguous():
        raise ValueError("a_q must be contiguous 2-D uint8 codes and a_scale contiguous")
    if w.dtype != torch.uint8 or not w.is_contiguous() or not w_scale.is_contiguous():
        raise ValueError("w must be contiguous uint8 codes and w_scale contiguous")
    M, N = a_q.shape[0], w.shape[0]
    if fmt == "mxfp4":
        K = a_q.shape[1] * 2
        if w.shape != (N, K // 2) or w_scale.dtype != torch.uint8 or w_scale.numel() != N * (K // 32):
            raise ValueError("MXFP4 weights: w [N, K/2] uint8 and w_scale [N, K/32] uint8")
        if a_scale.dtype != torch.uint8 or a_scale.numel() < rmsq_scale_bytes(M, K, 32, FMT_MXFP4_E2M1, scale_layout):
            raise ValueError("a_scale: the e8m0 scale bytes of a_q in scale_layout")
        call = gemm_afp4wfp4
    elif fmt == "fp8":
        K = a_q.shape[1]
        if w.shape != (N, K) or w_scale.dtype != torch.float32 or w_scale.numel() != -(-N // 128) * (K // 128):
            raise ValueError("FP8 weights: w [N, K] uint8 and w_scale [ceil(N/128), K/128] float32")
        if a_scale.dtype != torch.float32 or a_scale.numel() < M * (K // 128):
            raise ValueError("a_scale: the fp32 scales of a_q in scale_layout")
        call = gemm_a8w8_blockscale
    else:
        raise ValueError(f"unknown weight format {fmt!r}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a_q.device)
    elif out.dtype != torch.float32 or out.shape != (M, N) or out.stride(1) != 1:
        raise ValueError("out must be a float32 [M, N] tensor with unit column stride")
    call(a_q, a_scale, scale_layout, w, w_scale, W_PRESHUFFLED if preshuffled else W_ROW_MAJOR, M, N, K, out,
         out.stride(0) if M > 1 else N, stream)
    return out
