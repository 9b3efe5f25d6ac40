"""ctypes front-end of the plain C NVFP4 oracle -- TEST INFRASTRUCTURE ONLY.

Marshals numpy arrays into liboracle.so (built from nvfp4_oracle.c by
build_oracle.py) and back.  All arithmetic of the method lives in the C file;
this module only allocates outputs and loops over MoE groups.

Layout / rounding integers follow the public ABI numbering:
  layouts ROW_1D=0, COL_1D=1, ROW_COL_1D=2, BLK_2D=3; rounding RNE=0, SR=1;
  dtypes F32=0, BF16=1 (BF16 passed as uint16 bit patterns);
  scale modes 1D=0, 2D=1.
"""
import ctypes
import os

import numpy as np

from . import build_oracle

F32, BF16 = 0, 1
ROW_1D, COL_1D, ROW_COL_1D, BLK_2D = 0, 1, 2, 3
RNE, SR = 0, 1
SCALE_1D, SCALE_2D = 0, 1
STREAM_ROW, STREAM_COL, STREAM_2D, STREAM_RHT = 0, 1, 2, 3
MX_FP8, MX_FP4 = 0, 1
STREAM_MX_ROW, STREAM_MX_COL = 4, 5

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = build_oracle.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(build_oracle.SRC):
            build_oracle.build()
        L = ctypes.CDLL(path)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        L.orc_philox4x32_10.argtypes = [u32p, u32p, u32p]
        L.orc_philox4x32_10.restype = None
        L.orc_draw16.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64]
        L.orc_draw16.restype = ctypes.c_uint32
        L.orc_e2m1_value.argtypes = [ctypes.c_uint32]
        L.orc_e2m1_value.restype = ctypes.c_float
        L.orc_e4m3_value.argtypes = [ctypes.c_uint32]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode.restype = ctypes.c_uint32
        L.orc_e2m1_rne.argtypes = [ctypes.c_float]
        L.orc_e2m1_rne.restype = ctypes.c_uint32
        L.orc_e2m1_sr.argtypes = [ctypes.c_float, ctypes.c_uint32]
        L.orc_e2m1_sr.restype = ctypes.c_uint32
        L.orc_tensor_scale.argtypes = [ctypes.c_float]
        L.orc_tensor_scale.restype = ctypes.c_float
        L.orc_rht_sign_mask.argtypes = [ctypes.c_uint64]
        L.orc_rht_sign_mask.restype = ctypes.c_uint32
        L.orc_rht16.argtypes = [f32p, ctypes.c_uint32, f32p]
        L.orc_rht16.restype = None
        L.orc_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                   ctypes.c_int, ctypes.c_uint64, f32p, ctypes.c_uint64,
                                   u8p, u8p, f32p, u8p, u8p, f32p]
        L.orc_quantize.restype = ctypes.c_int
        L.orc_amax.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                               ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_uint64]
        L.orc_amax.restype = ctypes.c_float
        L.orc_dequantize.argtypes = [u8p, u8p, ctypes.c_float, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        L.orc_dequantize.restype = None
        L.orc_dequantize_f64.argtypes = [u8p, u8p, ctypes.c_double, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int, f64p]
        L.orc_dequantize_f64.restype = None
        L.orc_gemm.argtypes = [u8p, u8p, ctypes.c_double, ctypes.c_int,
                               u8p, u8p, ctypes.c_double, ctypes.c_int,
                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                               i64p, i64p, ctypes.c_int64, f64p, f64p]
        L.orc_gemm.restype = None
        L.orc_swiglu.argtypes = [ctypes.c_double, ctypes.c_double]
        L.orc_swiglu.restype = ctypes.c_double
        L.orc_mx_scale_exp.argtypes = [ctypes.c_float, ctypes.c_int]
        L.orc_mx_scale_exp.restype = ctypes.c_int
        L.orc_e4m3_sr.argtypes = [ctypes.c_float, ctypes.c_uint32]
        L.orc_e4m3_sr.restype = ctypes.c_uint32
        L.orc_mx_elem_value.argtypes = [ctypes.c_uint32, ctypes.c_int]
        L.orc_mx_elem_value.restype = ctypes.c_double
        L.orc_mx_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_uint64, ctypes.c_uint64, u8p, u8p]
        L.orc_mx_quantize.restype = ctypes.c_int
        L.orc_mx_dequantize.argtypes = [u8p, u8p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_int]
        L.orc_mx_dequantize.restype = None
        L.orc_mx_gemm.argtypes = [u8p, u8p, ctypes.c_int, u8p, u8p, ctypes.c_int,
                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                  i64p, i64p, ctypes.c_int64, f64p, f64p]
        L.orc_mx_gemm.restype = None
        _lib = L
    return _lib


def _p(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ---------------------------------------------------------------- primitives
def philox4x32_10(counter, key):
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_p(c, ctypes.c_uint32), _p(k, ctypes.c_uint32), _p(out, ctypes.c_uint32))
    return out


def draw16(seed, stream, index):
    return int(lib().orc_draw16(seed, stream, index))


def e2m1_value(code):
    return float(lib().orc_e2m1_value(code))


def e4m3_value(byte):
    return float(lib().orc_e4m3_value(byte))


def e4m3_encode(u):
    return int(lib().orc_e4m3_encode(float(u)))


def e2m1_rne(y):
    return int(lib().orc_e2m1_rne(float(y)))


def e2m1_sr(y, r16):
    return int(lib().orc_e2m1_sr(float(y), int(r16)))


def tensor_scale(amax):
    return float(lib().orc_tensor_scale(float(amax)))


def rht_sign_mask(seed):
    return int(lib().orc_rht_sign_mask(seed))


def rht16(x, sign_mask):
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape == (16,)
    out = np.zeros(16, dtype=np.float32)
    lib().orc_rht16(_p(x, ctypes.c_float), sign_mask, _p(out, ctypes.c_float))
    return out


# ---------------------------------------------------------------- quantize
class QTensor:
    """codes [R x C/2] u8, scales u8, tensor scale (python float, binary32)."""

    def __init__(self, codes, scales, ts, rows, cols, scale_mode):
        self.codes, self.scales, self.ts = codes, scales, ts
        self.rows, self.cols, self.scale_mode = rows, cols, scale_mode


def quantize(x, dtype, layout, rnd=RNE, sr_seed=0, hadamard=False, hadamard_seed=0,
             amax_in=None, ld=None, index_base=0):
    """x: numpy float32 [rows x cols] (dtype F32) or uint16 bf16 bits (BF16).

    index_base offsets every element's random-draw index (a band of a larger
    tensor).  Returns one QTensor, or (row, col) for ROW_COL_1D."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    if ld is None:
        ld = cols
    if dtype == BF16:
        assert x.dtype == np.uint16
    else:
        assert x.dtype == np.float32

    def alloc(r, c, mode):
        codes = np.zeros((r, c // 2), dtype=np.uint8)
        if mode == SCALE_2D:
            scales = np.zeros((r // 16, c // 16), dtype=np.uint8)
        else:
            scales = np.zeros((r, c // 16), dtype=np.uint8)
        return codes, scales, np.zeros(1, dtype=np.float32)

    if layout == COL_1D:
        r1, c1, m1 = cols, rows, SCALE_1D
    elif layout == BLK_2D:
        r1, c1, m1 = rows, cols, SCALE_2D
    else:
        r1, c1, m1 = rows, cols, SCALE_1D
    codes, scales, ts = alloc(r1, c1, m1)
    if layout == ROW_COL_1D:
        codes2, scales2, ts2 = alloc(cols, rows, SCALE_1D)
    else:
        codes2 = scales2 = None
        ts2 = None
    # one A_t, or (ROW_COL_1D with the transform) a pair: row output, column output
    amax_arr = None if amax_in is None else np.array(np.atleast_1d(amax_in), dtype=np.float32)
    nul8 = ctypes.POINTER(ctypes.c_uint8)()
    nulf = ctypes.POINTER(ctypes.c_float)()
    rc = lib().orc_quantize(
        x.ctypes.data_as(ctypes.c_void_p), dtype, rows, cols, ld, layout, rnd,
        ctypes.c_uint64(sr_seed), int(bool(hadamard)), ctypes.c_uint64(hadamard_seed),
        _p(amax_arr, ctypes.c_float) if amax_arr is not None else nulf,
        ctypes.c_uint64(index_base), _p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8), _p(ts, ctypes.c_float),
        _p(codes2, ctypes.c_uint8) if codes2 is not None else nul8,
        _p(scales2, ctypes.c_uint8) if scales2 is not None else nul8,
        _p(ts2, ctypes.c_float) if ts2 is not None else nulf)
    if rc != 0:
        raise ValueError(f"oracle quantize rejected the request (code {rc})")
    q = QTensor(codes, scales, float(ts[0]), r1, c1, m1)
    if layout == ROW_COL_1D:
        return q, QTensor(codes2, scales2, float(ts2[0]), cols, rows, SCALE_1D)
    return q


def amax(x, dtype, layout, hadamard=False, hadamard_seed=0):
    """A_t of the tensor `layout` quantizes (after the optional transform)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    return float(lib().orc_amax(x.ctypes.data_as(ctypes.c_void_p), dtype, rows, cols, cols, layout,
                                int(bool(hadamard)), ctypes.c_uint64(hadamard_seed)))


def dequantize(q, out_dtype=F32):
    out = np.zeros((q.rows, q.cols), dtype=np.uint16 if out_dtype == BF16 else np.float32)
    lib().orc_dequantize(_p(q.codes, ctypes.c_uint8), _p(q.scales, ctypes.c_uint8),
                         ctypes.c_float(q.ts), q.rows, q.cols, q.scale_mode,
                         out.ctypes.data_as(ctypes.c_void_p), out_dtype)
    return out


def requantize(q, rnd=RNE, sr_seed=0, hadamard=False, hadamard_seed=0, amax_in=None, index_base=0):
    """Re-quantization of a row-blocked QTensor along columns: the backward
    pass forms column blocks from the stored forward tensor ("Thinking
    Machines ускорила обучение Inkling 2 Small 4-битными числами", iitak.ru,
    section "Как это работает").  It is the COL_1D quantization of the
    binary32 dequantization, written as exactly that composition (no
    arithmetic of its own)."""
    assert q.scale_mode == SCALE_1D
    x = dequantize(q, F32)
    return quantize(x, F32, COL_1D, rnd, sr_seed=sr_seed, hadamard=hadamard,
                    hadamard_seed=hadamard_seed, amax_in=amax_in, index_base=index_base)


def dequantize_f64(q):
    out = np.zeros((q.rows, q.cols), dtype=np.float64)
    lib().orc_dequantize_f64(_p(q.codes, ctypes.c_uint8), _p(q.scales, ctypes.c_uint8),
                             float(np.float32(q.ts)), q.rows, q.cols, q.scale_mode,
                             _p(out, ctypes.c_double))
    return out


# ---------------------------------------------------------------- GEMM
def gemm(A, B, entries=None):
    """C = A B^T over exactly dequantized operands in float64.

    A: QTensor [M x K], B: QTensor [N x K].  Returns (C, W) with W = sum |a b|.
    With entries = (m_idx, n_idx) only those outputs are computed (1-D arrays)."""
    assert A.cols == B.cols
    M, N, K = A.rows, B.rows, A.cols
    if entries is None:
        C = np.zeros((M, N), dtype=np.float64)
        W = np.zeros((M, N), dtype=np.float64)
        em = en = ctypes.POINTER(ctypes.c_int64)()
        ne = -1
    else:
        mi = np.ascontiguousarray(entries[0], dtype=np.int64)
        ni = np.ascontiguousarray(entries[1], dtype=np.int64)
        ne = mi.size
        C = np.zeros(ne, dtype=np.float64)
        W = np.zeros(ne, dtype=np.float64)
        em, en = _p(mi, ctypes.c_int64), _p(ni, ctypes.c_int64)
    lib().orc_gemm(_p(A.codes, ctypes.c_uint8), _p(A.scales, ctypes.c_uint8),
                   float(np.float32(A.ts)), A.scale_mode,
                   _p(B.codes, ctypes.c_uint8), _p(B.scales, ctypes.c_uint8),
                   float(np.float32(B.ts)), B.scale_mode,
                   M, N, K, em, en, ne, _p(C, ctypes.c_double), _p(W, ctypes.c_double))
    return C, W


def row_slice(q, r0, r1):
    """Rows [r0, r1) of a 1D-scaled (or 16-aligned 2D-scaled) QTensor."""
    if q.scale_mode == SCALE_2D:
        assert r0 % 16 == 0 and r1 % 16 == 0
        sc = q.scales[r0 // 16:r1 // 16]
    else:
        sc = q.scales[r0:r1]
    return QTensor(np.ascontiguousarray(q.codes[r0:r1]), np.ascontiguousarray(sc), q.ts,
                   r1 - r0, q.cols, q.scale_mode)


def grouped_gemm(A, offsets, B_groups, entries=None):
    """Per group g: C[rows of g] = A[rows of g] B_g^T.  B_groups: list of QTensor.

    entries: optional (m_idx, n_idx) over the stacked output; returns (C, W)."""
    G = len(B_groups)
    N = B_groups[0].rows
    if entries is None:
        C = np.zeros((A.rows, N), dtype=np.float64)
        W = np.zeros((A.rows, N), dtype=np.float64)
        for g in range(G):
            r0, r1 = int(offsets[g]), int(offsets[g + 1])
            if r1 > r0:
                c, w = gemm(row_slice(A, r0, r1), B_groups[g])
                C[r0:r1], W[r0:r1] = c, w
        return C, W
    mi = np.asarray(entries[0], dtype=np.int64)
    ni = np.asarray(entries[1], dtype=np.int64)
    C = np.zeros(mi.size, dtype=np.float64)
    W = np.zeros(mi.size, dtype=np.float64)
    grp = np.searchsorted(np.asarray(offsets), mi, side="right") - 1
    for g in np.unique(grp):
        sel = np.nonzero(grp == g)[0]
        c, w = gemm(A, B_groups[g], entries=(mi[sel], ni[sel]))
        C[sel], W[sel] = c, w
    return C, W


def swiglu(g, u):
    f = lib().orc_swiglu
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    out = np.empty(np.broadcast(g, u).shape, dtype=np.float64)
    for i, (a, b) in enumerate(zip(g.ravel(), u.ravel())):
        out.flat[i] = f(float(a), float(b))
    return out


# ---------------------------------------------------------------- MX formats
class MXTensor:
    """MX tensor: codes (FP8: rows x cols bytes; FP4: rows x cols/2), E8M0
    scales rows x cols/32, element format elem (MX_FP8 or MX_FP4)."""

    def __init__(self, codes, scales, rows, cols, elem):
        self.codes, self.scales = codes, scales
        self.rows, self.cols, self.elem = rows, cols, elem


def mx_quantize(x, dtype, layout, elem, rnd=RNE, seed=0, index_base=0):
    """OCP-MX quantization (E8M0 scale per 32 along the block dimension) of
    x (numpy float32, or uint16 bf16 bits); layout ROW_1D or COL_1D (the
    result describes the transpose)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    assert x.dtype == (np.uint16 if dtype == BF16 else np.float32)
    r, c = (cols, rows) if layout == COL_1D else (rows, cols)
    codes = np.zeros((r, c if elem == MX_FP8 else c // 2), dtype=np.uint8)
    scales = np.zeros((r, c // 32), dtype=np.uint8)
    rc = lib().orc_mx_quantize(x.ctypes.data_as(ctypes.c_void_p), dtype, rows, cols, cols, layout,
                               elem, rnd, ctypes.c_uint64(seed), ctypes.c_uint64(index_base),
                               _p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8))
    if rc != 0:
        raise ValueError(f"oracle mx_quantize rejected the request (code {rc})")
    return MXTensor(codes, scales, r, c, elem)


def mx_dequantize(q, out_dtype=F32):
    """out_dtype F32, BF16 (uint16 bits) or 2 (float64, exact)."""
    dt = {F32: np.float32, BF16: np.uint16, 2: np.float64}[out_dtype]
    out = np.zeros((q.rows, q.cols), dtype=dt)
    lib().orc_mx_dequantize(_p(q.codes, ctypes.c_uint8), _p(q.scales, ctypes.c_uint8), q.elem,
                            q.rows, q.cols, out.ctypes.data_as(ctypes.c_void_p), out_dtype)
    return out


def mx_gemm(A, B, entries=None):
    """C = A B^T over exactly dequantized MX operands in float64; (C, W) as gemm."""
    assert A.cols == B.cols
    M, N, K = A.rows, B.rows, A.cols
    if entries is None:
        C = np.zeros((M, N), dtype=np.float64)
        W = np.zeros((M, N), dtype=np.float64)
        em = en = ctypes.POINTER(ctypes.c_int64)()
        ne = -1
    else:
        mi = np.ascontiguousarray(entries[0], dtype=np.int64)
        ni = np.ascontiguousarray(entries[1], dtype=np.int64)
        ne = mi.size
        C = np.zeros(ne, dtype=np.float64)
        W = np.zeros(ne, dtype=np.float64)
        em, en = _p(mi, ctypes.c_int64), _p(ni, ctypes.c_int64)
    lib().orc_mx_gemm(_p(A.codes, ctypes.c_uint8), _p(A.scales, ctypes.c_uint8), A.elem,
                      _p(B.codes, ctypes.c_uint8), _p(B.scales, ctypes.c_uint8), B.elem,
                      M, N, K, em, en, ne, _p(C, ctypes.c_double), _p(W, ctypes.c_double))
    return C, W

