"""CPU oracle for residual-add + RMSNorm + per-group FP8 / MXFP4 quantization.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product library
(``fp4_quant_amd``) never imports it, and the two share no code.

Thin ctypes wrapper over ``liboracle.so`` (plain C, double precision; see
``rmsq_oracle.c`` for the arithmetic and the passages it follows). bf16
tensors are numpy ``uint16`` arrays of bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
FMT_FP8 = 0
FMT_MXFP4 = 1
LAYOUT_ROW = 0
LAYOUT_TILED32 = 1
LAYOUT_COL = 2

_p = C.c_void_p
_i64 = C.c_int64
_i32 = C.c_int32


def _bind(L):
    L.oracle_bf16_from_double.restype = C.c_uint16
    L.oracle_bf16_from_double.argtypes = [C.c_double]
    L.oracle_bf16_to_double.restype = C.c_double
    L.oracle_bf16_to_double.argtypes = [C.c_uint16]
    L.oracle_e4m3fn_encode.restype = C.c_uint8
    L.oracle_e4m3fn_encode.argtypes = [C.c_double]
    L.oracle_e4m3fn_decode.restype = C.c_double
    L.oracle_e4m3fn_decode.argtypes = [C.c_uint8]
    L.oracle_e2m1_encode.restype = C.c_uint8
    L.oracle_e2m1_encode.argtypes = [C.c_double]
    L.oracle_e2m1_decode.restype = C.c_double
    L.oracle_e2m1_decode.argtypes = [C.c_uint8]
    L.oracle_mx_scale_exponent.restype = C.c_int
    L.oracle_mx_scale_exponent.argtypes = [C.c_double]
    for name in ("oracle_bf16_from_double_n", "oracle_e4m3fn_encode_n", "oracle_e2m1_encode_n"):
        f = getattr(L, name)
        f.restype = None
        f.argtypes = [_p, _p, _i64]
    L.oracle_add_rmsnorm.restype = None
    L.oracle_add_rmsnorm.argtypes = [_p, _i64, _p, _i64, _p, C.c_float, _i64, _i64, _p, _i64, _p, _i64]
    L.oracle_group_quant.restype = None
    L.oracle_group_quant.argtypes = [_p, _i64, _i64, _i64, _i32, _i32, _i32, _p, _p]
    L.oracle_rmsnorm_quant_group.restype = C.c_int
    L.oracle_rmsnorm_quant_group.argtypes = [_p, _i64, _p, _i64, _p, C.c_float, _i64, _i64,
                                             _i32, _i32, _i32, _p, _p, _p, _p, _i64]
    L.oracle_gemm_a16wfp4_prequant.restype = C.c_int
    L.oracle_gemm_a16wfp4_prequant.argtypes = [_p, _i64, _p, _p, _i64, _i64, _i64, _p, _i64]
    L.oracle_gemm_a16w8_prequant.restype = C.c_int
    L.oracle_gemm_a16w8_prequant.argtypes = [_p, _i64, _p, _p, _i64, _i64, _i64, _p, _i64]
    for name in ("oracle_gemm_afp4wfp4", "oracle_gemm_a8w8_blockscale"):
        f = getattr(L, name)
        f.restype = C.c_int
        f.argtypes = [_p, _p, _i32, _p, _p, _i64, _i64, _i64, _p, _i64]
    L.oracle_num_threads.restype = C.c_int
    L.oracle_num_threads.argtypes = []
    L.oracle_set_num_threads.restype = None
    L.oracle_set_num_threads.argtypes = [C.c_int]
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data


def _scale_shape(M, N, group, fmt, layout):
    G = N // group
    dt = np.float32 if fmt == FMT_FP8 else np.uint8
    if layout == LAYOUT_TILED32:
        return (((M + 31) // 32) * 32 * G,), dt
    if layout == LAYOUT_COL:
        return (G, M), dt
    return (M, G), dt


def bf16_to_double(b) -> np.ndarray:
    """bf16 bit patterns -> float64 (a widening that numpy does exactly)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Oracle:
    """Binding of one build of the oracle library (the default build, or -
    in the pin tests' mutation check - a copy with a planted mistake)."""

    def __init__(self, path: str):
        self._L = _bind(C.CDLL(path))
        self._e4m3 = None
        self._e2m1 = None

    def lib(self):
        return self._L

    def num_threads(self) -> int:
        return self._L.oracle_num_threads()

    def set_num_threads(self, n: int) -> None:
        self._L.oracle_set_num_threads(int(n))

    # ------------------------------------------------------------- codecs --
    def bf16_from_double(self, v) -> np.ndarray:
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, np.uint16)
        self._L.oracle_bf16_from_double_n(_ptr(v), _ptr(out), v.size)
        return out

    bf16_to_double = staticmethod(bf16_to_double)

    def e4m3fn_encode(self, v) -> np.ndarray:
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, np.uint8)
        self._L.oracle_e4m3fn_encode_n(_ptr(v), _ptr(out), v.size)
        return out

    def e2m1_encode(self, v) -> np.ndarray:
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, np.uint8)
        self._L.oracle_e2m1_encode_n(_ptr(v), _ptr(out), v.size)
        return out

    def e4m3fn_table(self) -> np.ndarray:
        """Decoded value of each of the 256 e4m3fn codes (NaN for 0x7F / 0xFF)."""
        if self._e4m3 is None:
            self._e4m3 = np.array([self._L.oracle_e4m3fn_decode(c) for c in range(256)])
        return self._e4m3

    def e2m1_table(self) -> np.ndarray:
        if self._e2m1 is None:
            self._e2m1 = np.array([self._L.oracle_e2m1_decode(c) for c in range(16)])
        return self._e2m1

    def mx_scale_exponent(self, amax: float) -> int:
        return self._L.oracle_mx_scale_exponent(float(amax))

    # ----------------------------------------------------------- pipeline --
    def alloc_outputs(self, M, N, group=128, fmt=FMT_FP8, scale_layout=LAYOUT_ROW, residual=False,
                      keep_bf16=False, ldr=None, scale_fill=0):
        """Output arrays for ``rmsnorm_quant_group(..., out=...)``, written once
        here (so their pages are mapped before any timed call)."""
        out = {"q": np.zeros((M, N if fmt == FMT_FP8 else N // 2), np.uint8)}
        sshape, sdt = _scale_shape(M, N, group, fmt, scale_layout)
        out["scale"] = np.full(sshape, scale_fill, sdt)
        if residual:
            out["residual_out"] = np.zeros((M, ldr or N), np.uint16)[:, :N]   # the input's row stride
        if keep_bf16:
            out["bf16"] = np.zeros((M, N), np.uint16)
        return out

    def rmsnorm_quant_group(self, x, gamma, eps, residual=None, group=128, fmt=FMT_FP8,
                            scale_layout=LAYOUT_ROW, keep_bf16=False, scale_fill=0, out=None):
        """Fused oracle. x, residual: [M, N] uint16 (bf16 bits), row stride may
        exceed N; gamma: [N] uint16. Returns a dict with 'q', 'scale' and, when
        present, 'residual_out' and 'bf16'. Bytes of the tiled scale buffer that
        no row owns keep ``scale_fill``. ``out``: arrays from ``alloc_outputs``
        to write into instead of fresh ones (their unowned scale bytes keep
        what they held)."""
        M, N = x.shape
        assert x.strides[1] == 2 and gamma.dtype == np.uint16
        ldx = x.strides[0] // 2
        gamma = np.ascontiguousarray(gamma)
        ldr = 0
        if residual is not None:
            assert residual.shape == (M, N) and residual.strides[1] == 2
            ldr = residual.strides[0] // 2
        if out is None:
            out = self.alloc_outputs(M, N, group, fmt, scale_layout, residual is not None, keep_bf16, ldr,
                                     scale_fill)
        q, scale = out["q"], out["scale"]
        sshape, sdt = _scale_shape(M, N, group, fmt, scale_layout)
        assert q.shape == (M, N if fmt == FMT_FP8 else N // 2) and q.dtype == np.uint8 and q.flags.c_contiguous
        assert scale.shape == sshape and scale.dtype == sdt and scale.flags.c_contiguous
        res_out = out.get("residual_out") if residual is not None else None
        if residual is not None:
            assert res_out is not None and res_out.shape == (M, N) and res_out.strides == residual.strides
        yb = out.get("bf16") if keep_bf16 else None
        if keep_bf16:
            assert yb is not None and yb.shape == (M, N) and yb.flags.c_contiguous
        rc = self._L.oracle_rmsnorm_quant_group(
            _ptr(x), ldx, _ptr(residual), ldr, _ptr(gamma), float(eps), M, N, group, fmt,
            scale_layout, _ptr(q), _ptr(scale), _ptr(res_out), _ptr(yb), N)
        if rc != 0:
            raise ValueError("oracle: arguments outside the defined operation")
        res = {"q": q, "scale": scale}
        if res_out is not None:
            res["residual_out"] = res_out
        if yb is not None:
            res["bf16"] = yb
        return res

    def add_rmsnorm(self, x, gamma, eps, residual=None):
        """Stage 1 alone: returns (h or None, yb)."""
        M, N = x.shape
        x = np.ascontiguousarray(x)
        h = np.zeros((M, N), np.uint16) if residual is not None else None
        r = np.ascontiguousarray(residual) if residual is not None else None
        yb = np.zeros((M, N), np.uint16)
        self._L.oracle_add_rmsnorm(_ptr(x), N, _ptr(r), N, _ptr(np.ascontiguousarray(gamma)), float(eps),
                                   M, N, _ptr(h), N, _ptr(yb), N)
        return h, yb

    def gemm_a16wfp4_prequant(self, a, w, w_scale):
        """A16WFP4 prequant GEMM: a [M, K] uint16 (bf16 bits, row stride may
        exceed K), w [N, K/2] uint8 e2m1 codes, w_scale [N, K/32] uint8 e8m0.
        Returns C [M, N] float64."""
        M, K = a.shape
        assert a.strides[1] == 2 and a.dtype == np.uint16
        N = w.shape[0]
        assert w.shape == (N, K // 2) and w_scale.shape == (N, K // 32)
        w = np.ascontiguousarray(w, dtype=np.uint8)
        w_scale = np.ascontiguousarray(w_scale, dtype=np.uint8)
        out = np.zeros((M, N), np.float64)
        rc = self._L.oracle_gemm_a16wfp4_prequant(_ptr(a), a.strides[0] // 2, _ptr(w), _ptr(w_scale), M, N, K,
                                                  _ptr(out), N)
        if rc != 0:
            raise ValueError("oracle: arguments outside the defined operation")
        return out

    def gemm_a16w8_prequant(self, a, w, w_scale):
        """A16W8 prequant GEMM: a [M, K] uint16 (bf16 bits, row stride may
        exceed K), w [N, K] uint8 e4m3fn codes, w_scale [ceil(N/128), K/128]
        float32 block scales. Returns C [M, N] float64."""
        M, K = a.shape
        assert a.strides[1] == 2 and a.dtype == np.uint16
        N = w.shape[0]
        assert w.shape == (N, K) and w_scale.shape == (-(-N // 128), K // 128)
        w = np.ascontiguousarray(w, dtype=np.uint8)
        w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
        out = np.zeros((M, N), np.float64)
        rc = self._L.oracle_gemm_a16w8_prequant(_ptr(a), a.strides[0] // 2, _ptr(w), _ptr(w_scale), M, N, K,
                                                _ptr(out), N)
        if rc != 0:
            raise ValueError("oracle: arguments outside the defined operation")
        return out

    def gemm_afp4wfp4(self, a_q, a_scale, w, w_scale, scale_layout=LAYOUT_ROW):
        """GEMM of MXFP4 activations as the group quantization writes them
        (a_q [M, K/2] uint8 codes, a_scale its e8m0 scale array in
        scale_layout) with MXFP4 weights w [N, K/2], w_scale [N, K/32].
        Returns C [M, N] float64."""
        a_q = np.ascontiguousarray(a_q, dtype=np.uint8)
        M, K = a_q.shape[0], a_q.shape[1] * 2
        N = w.shape[0]
        assert w.shape == (N, K // 2) and w_scale.shape == (N, K // 32)
        sshape, _ = _scale_shape(M, K, 32, FMT_MXFP4, scale_layout)
        a_scale = np.ascontiguousarray(a_scale, dtype=np.uint8)
        assert a_scale.size >= int(np.prod(sshape))
        w = np.ascontiguousarray(w, dtype=np.uint8)
        w_scale = np.ascontiguousarray(w_scale, dtype=np.uint8)
        out = np.zeros((M, N), np.float64)
        rc = self._L.oracle_gemm_afp4wfp4(_ptr(a_q), _ptr(a_scale), scale_layout, _ptr(w), _ptr(w_scale), M, N, K,
                                          _ptr(out), N)
        if rc != 0:
            raise ValueError("oracle: arguments outside the defined operation")
        return out

    def gemm_a8w8_blockscale(self, a_q, a_scale, w, w_scale, scale_layout=LAYOUT_ROW):
        """GEMM of FP8 activations as the group quantization writes them
        (a_q [M, K] uint8 e4m3fn codes, a_scale its fp32 scale array in
        scale_layout, row- or column-major) with FP8 weights w [N, K] and
        fp32 block scales w_scale [ceil(N/128), K/128]. Returns C [M, N]
        float64."""
        a_q = np.ascontiguousarray(a_q, dtype=np.uint8)
        M, K = a_q.shape
        N = w.shape[0]
        assert w.shape == (N, K) and w_scale.shape == (-(-N // 128), K // 128)
        sshape, _ = _scale_shape(M, K, 128, FMT_FP8, scale_layout)
        a_scale = np.ascontiguousarray(a_scale, dtype=np.float32)
        assert a_scale.size >= int(np.prod(sshape))
        w = np.ascontiguousarray(w, dtype=np.uint8)
        w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
        out = np.zeros((M, N), np.float64)
        rc = self._L.oracle_gemm_a8w8_blockscale(_ptr(a_q), _ptr(a_scale), scale_layout, _ptr(w), _ptr(w_scale),
                                                 M, N, K, _ptr(out), N)
        if rc != 0:
            raise ValueError("oracle: arguments outside the defined operation")
        return out

    def group_quant(self, yb, group=128, fmt=FMT_FP8, scale_layout=LAYOUT_ROW, scale_fill=0):
        """Stage 2 alone on bf16 rows: returns (q, scale)."""
        yb = np.ascontiguousarray(yb, dtype=np.uint16)
        M, N = yb.shape
        q = np.zeros((M, N if fmt == FMT_FP8 else N // 2), np.uint8)
        sshape, sdt = _scale_shape(M, N, group, fmt, scale_layout)
        scale = np.full(sshape, scale_fill, sdt)
        self._L.oracle_group_quant(_ptr(yb), N, M, N, group, fmt, scale_layout, _ptr(q), _ptr(scale))
        return q, scale


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _default = Oracle(_LIB_PATH)
    return _default


_serial = None


def serial() -> Oracle:
    """The same oracle built without OpenMP: one thread, whatever the host's
    OpenMP runtime is told (for a single-core timing)."""
    global _serial
    if _serial is None:
        from . import build as _b
        if not os.path.exists(_b.LIB_SERIAL):
            _b.build()
        _serial = Oracle(_b.LIB_SERIAL)
    return _serial


# Module-level API: the default build.
def lib():
    return default().lib()


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


def bf16_from_double(v):
    return default().bf16_from_double(v)


def e4m3fn_encode(v):
    return default().e4m3fn_encode(v)


def e2m1_encode(v):
    return default().e2m1_encode(v)


def e4m3fn_table():
    return default().e4m3fn_table()


def e2m1_table():
    return default().e2m1_table()


def mx_scale_exponent(amax):
    return default().mx_scale_exponent(amax)


def rmsnorm_quant_group(*a, **k):
    return default().rmsnorm_quant_group(*a, **k)


def alloc_outputs(*a, **k):
    return default().alloc_outputs(*a, **k)


def add_rmsnorm(*a, **k):
    return default().add_rmsnorm(*a, **k)


def gemm_a16wfp4_prequant(*a, **k):
    return default().gemm_a16wfp4_prequant(*a, **k)


def gemm_a16w8_prequant(*a, **k):
    return default().gemm_a16w8_prequant(*a, **k)


def gemm_afp4wfp4(*a, **k):
    return default().gemm_afp4wfp4(*a, **k)


def gemm_a8w8_blockscale(*a, **k):
    return default().gemm_a8w8_blockscale(*a, **k)


def group_quant(*a, **k):
    return default().group_quant(*a, **k)
