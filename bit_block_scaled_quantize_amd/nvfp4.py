"""Thin ctypes binding of libnvfp4.so (include/nvfp4.h).

Argument marshalling only: every step of quantize / dequantize / GEMM runs in
the HIP kernels behind the C ABI.  PyTorch supplies device memory (output
tensors are allocated with torch) and the current HIP stream.  If the built
library is missing, importing this module raises -- there is no fallback.
"""
import contextlib
import ctypes
import functools
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

# enums (include/nvfp4.h)
NVFP4_OK = 0
NVFP4_F32, NVFP4_BF16 = 0, 1
NVFP4_ROW_1D, NVFP4_COL_1D, NVFP4_ROW_COL_1D, NVFP4_BLK_2D = 0, 1, 2, 3
NVFP4_RNE, NVFP4_SR = 0, 1
NVFP4_EPI_NONE, NVFP4_EPI_SWIGLU = 0, 1
NVFP4_SCALE_1D, NVFP4_SCALE_2D = 0, 1
NVFP4_MX_E4M3, NVFP4_MX_E2M1 = 0, 1
NVFP4_MX_ACC_NATIVE, NVFP4_MX_ACC_EXACT = 0, 1

EXPORTED = ["nvfp4_quantize_workspace_size", "nvfp4_quantize", "nvfp4_quantize_noalloc", "nvfp4_requantize",
            "nvfp4_dequantize",
            "nvfp4_gemm", "nvfp4_gemm_workspace_size", "nvfp4_grouped_gemm", "nvfp4_mx_quantize", "nvfp4_mx_dequantize", "nvfp4_mx_gemm",
            "nvfp4_mx_gemm_workspace_size",
            "nvfp4_status_string", "nvfp4_version"]


class CTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("scale_mode", ctypes.c_int32)]


class CMXTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("elem", ctypes.c_int32)]


class CQuantOpts(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("round", ctypes.c_int32), ("sr_seed", ctypes.c_uint64),
                ("hadamard", ctypes.c_int32), ("hadamard_seed", ctypes.c_uint64),
                ("amax_in", ctypes.c_void_p), ("amax_out", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run bit_block_scaled_quantize_amd/build.py "
                          "(there is no non-HIP fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.nvfp4_quantize_workspace_size.argtypes = [i64, i64, ctypes.POINTER(CQuantOpts)]
    L.nvfp4_quantize_workspace_size.restype = sz
    L.nvfp4_quantize.argtypes = [vp, i32, i64, i64, i64, ctypes.POINTER(CQuantOpts),
                                 ctypes.POINTER(CTensor), vp, sz, vp]
    L.nvfp4_quantize.restype = i32
    L.nvfp4_quantize_noalloc.argtypes = [vp, i32, i64, i64, i64, ctypes.POINTER(CQuantOpts),
                                         ctypes.POINTER(CTensor), vp]
    L.nvfp4_quantize_noalloc.restype = i32
    L.nvfp4_dequantize.argtypes = [ctypes.POINTER(CTensor), vp, i32, i64, vp]
    L.nvfp4_dequantize.restype = i32
    L.nvfp4_requantize.argtypes = [ctypes.POINTER(CTensor), ctypes.POINTER(CQuantOpts),
                                   ctypes.POINTER(CTensor), vp, sz, vp]
    L.nvfp4_requantize.restype = i32
    L.nvfp4_gemm.argtypes = [ctypes.POINTER(CTensor), ctypes.POINTER(CTensor), vp, i32, i64, i32, vp, sz, vp]
    L.nvfp4_gemm.restype = i32
    L.nvfp4_gemm_workspace_size.argtypes = [ctypes.POINTER(CTensor), ctypes.POINTER(CTensor), i32, i32]
    L.nvfp4_gemm_workspace_size.restype = sz
    L.nvfp4_grouped_gemm.argtypes = [i32, ctypes.POINTER(CTensor), vp, ctypes.POINTER(CTensor), vp,
                                     i32, i64, i32, vp, vp, sz, vp]
    L.nvfp4_grouped_gemm.restype = i32
    L.nvfp4_mx_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, ctypes.c_uint64,
                                    ctypes.POINTER(CMXTensor), vp]
    L.nvfp4_mx_quantize.restype = i32
    L.nvfp4_mx_dequantize.argtypes = [ctypes.POINTER(CMXTensor), vp, i32, i64, vp]
    L.nvfp4_mx_dequantize.restype = i32
    L.nvfp4_mx_gemm.argtypes = [ctypes.POINTER(CMXTensor), ctypes.POINTER(CMXTensor), vp, i32, i64, i32, vp, sz, vp]
    L.nvfp4_mx_gemm.restype = i32
    L.nvfp4_mx_gemm_workspace_size.argtypes = [ctypes.POINTER(CMXTensor), ctypes.POINTER(CMXTensor), i32, i32]
    L.nvfp4_mx_gemm_workspace_size.restype = sz
    L.nvfp4_status_string.argtypes = [i32]
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_version.argtypes = []
    L.nvfp4_version.restype = i32
    return L


lib = _load()


class NVFP4Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({lib.nvfp4_status_string(status).decode()})")


def _check(fn, status):
    if status != NVFP4_OK:
        raise NVFP4Error(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context in which a call's outputs and workspace are allocated: the
    stream the kernels run on.  torch's caching allocator hands a freed block
    back only to later allocations on the stream it was allocated on, so a
    workspace released when the call returns cannot be reused by other work
    while the kernels on `stream` still read it."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _launches_on_stream(fn):
    """Run the binding function fn with `stream` (keyword) as torch's current
    stream, so that everything it allocates belongs to that stream."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        with _on(stream):
            return fn(*args, stream=stream, **kw)
    return call


def _dtype_code(dt):
    if dt == torch.float32:
        return NVFP4_F32
    if dt == torch.bfloat16:
        return NVFP4_BF16
    raise TypeError(f"unsupported dtype {dt}")


@dataclass
class NVFP4Tensor:
    """codes [rows, cols/2] uint8, scales uint8 ([rows, cols/16] or
    [rows/16, cols/16]), tensor_scale float32 [1] (or [G] for grouped
    weights) -- all device tensors."""
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor
    rows: int
    cols: int
    scale_mode: int = NVFP4_SCALE_1D

    def c(self):
        return CTensor(self.codes.data_ptr(), self.scales.data_ptr(), self.tensor_scale.data_ptr(),
                       self.rows, self.cols, self.scale_mode)

    @staticmethod
    def empty(rows, cols, scale_mode=NVFP4_SCALE_1D, device="cuda", n_scales=1):
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        if scale_mode == NVFP4_SCALE_2D:
            scales = torch.empty((rows // 16, cols // 16), dtype=torch.uint8, device=device)
        else:
            scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=device)
        ts = torch.empty((n_scales,), dtype=torch.float32, device=device)
        return NVFP4Tensor(codes, scales, ts, rows, cols, scale_mode)


def nvfp4_quantize_workspace_size(rows, cols, amax_in=None):
    o = CQuantOpts(0, 0, 0, 0, 0, None if amax_in is None else amax_in.data_ptr(), None)
    return int(lib.nvfp4_quantize_workspace_size(rows, cols, ctypes.byref(o)))


@_launches_on_stream
def nvfp4_quantize(x, layout=NVFP4_ROW_1D, round=NVFP4_RNE, sr_seed=0, hadamard=False,
                   hadamard_seed=0, amax_in=None, out=None, workspace=None, amax_out=None,
                   stream=None):
    """Quantize a 2-D device tensor (float32 or bfloat16, unit column stride).

    Returns an NVFP4Tensor, or (row, col) for NVFP4_ROW_COL_1D.  `out` may
    pass preallocated outputs (one NVFP4Tensor, or a pair for ROW_COL);
    `amax_out` (float32 device tensor) receives the tensor amax used."""
    assert x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else max(cols, x.stride(0))
    dev = x.device
    if out is None:
        if layout == NVFP4_COL_1D:
            outs = [NVFP4Tensor.empty(cols, rows, NVFP4_SCALE_1D, dev)]
        elif layout == NVFP4_BLK_2D:
            outs = [NVFP4Tensor.empty(rows, cols, NVFP4_SCALE_2D, dev)]
        elif layout == NVFP4_ROW_COL_1D:
            outs = [NVFP4Tensor.empty(rows, cols, NVFP4_SCALE_1D, dev),
                    NVFP4Tensor.empty(cols, rows, NVFP4_SCALE_1D, dev)]
        else:
            outs = [NVFP4Tensor.empty(rows, cols, NVFP4_SCALE_1D, dev)]
    else:
        outs = list(out) if isinstance(out, (list, tuple)) else [out]
    arr = (CTensor * 2)()
    for i, t in enumerate(outs):
        arr[i] = t.c()
    opts = CQuantOpts(layout, round, sr_seed, int(bool(hadamard)), hadamard_seed,
                      None if amax_in is None else amax_in.data_ptr(),
                      None if amax_out is None else amax_out.data_ptr())
    need = int(lib.nvfp4_quantize_workspace_size(rows, cols, ctypes.byref(opts)))
    if workspace is None and need:
        workspace = torch.empty((need + 15) // 16 * 4, dtype=torch.float32, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.nvfp4_quantize(ctypes.c_void_p(x.data_ptr()), _dtype_code(x.dtype), rows, cols, ld,
                            ctypes.byref(opts), arr, _ptr(workspace), ws_bytes, _stream(stream))
    _check("nvfp4_quantize", st)
    return tuple(outs) if layout == NVFP4_ROW_COL_1D else outs[0]


def nvfp4_quantize_noalloc(x, out, layout=NVFP4_ROW_1D, round=NVFP4_RNE, sr_seed=0, hadamard=False,
                           hadamard_seed=0, amax_in=None, amax_out=None, stream=None):
    """nvfp4_quantize into preallocated outputs (`out`: one NVFP4Tensor, or a
    pair for NVFP4_ROW_COL_1D) with no workspace: the library's static
    device scratch holds the amax partials, so neither the library nor this
    wrapper allocates anything."""
    assert x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else max(cols, x.stride(0))
    outs = list(out) if isinstance(out, (list, tuple)) else [out]
    arr = (CTensor * 2)()
    for i, t in enumerate(outs):
        arr[i] = t.c()
    opts = CQuantOpts(layout, round, sr_seed, int(bool(hadamard)), hadamard_seed,
                      None if amax_in is None else amax_in.data_ptr(),
                      None if amax_out is None else amax_out.data_ptr())
    st = lib.nvfp4_quantize_noalloc(ctypes.c_void_p(x.data_ptr()), _dtype_code(x.dtype), rows, cols, ld,
                                    ctypes.byref(opts), arr, _stream(stream))
    _check("nvfp4_quantize_noalloc", st)
    return tuple(outs) if layout == NVFP4_ROW_COL_1D else outs[0]


@_launches_on_stream
def nvfp4_requantize(q, round=NVFP4_RNE, sr_seed=0, hadamard=False, hadamard_seed=0, amax_in=None,
                     out=None, workspace=None, amax_out=None, stream=None):
    """COL_1D re-quantization of a row-blocked NVFP4Tensor q (rows x cols):
    returns the cols x rows NVFP4Tensor that quantizing q's binary32
    dequantization along columns gives."""
    dev = q.codes.device
    if out is None:
        out = NVFP4Tensor.empty(q.cols, q.rows, NVFP4_SCALE_1D, dev)
    opts = CQuantOpts(NVFP4_COL_1D, round, sr_seed, int(bool(hadamard)), hadamard_seed,
                      None if amax_in is None else amax_in.data_ptr(),
                      None if amax_out is None else amax_out.data_ptr())
    need = int(lib.nvfp4_quantize_workspace_size(q.rows, q.cols, ctypes.byref(opts)))
    if workspace is None and need:
        workspace = torch.empty((need + 15) // 16 * 4, dtype=torch.float32, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ci, co = q.c(), out.c()
    st = lib.nvfp4_requantize(ctypes.byref(ci), ctypes.byref(opts), ctypes.byref(co), _ptr(workspace),
                              ws_bytes, _stream(stream))
    _check("nvfp4_requantize", st)
    return out


@_launches_on_stream
def nvfp4_dequantize(q, dtype=torch.float32, out=None, stream=None):
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=dtype, device=q.codes.device)
    assert out.stride(1) == 1
    ld = out.stride(0) if q.rows > 1 else max(q.cols, out.stride(0))
    ct = q.c()
    st = lib.nvfp4_dequantize(ctypes.byref(ct), ctypes.c_void_p(out.data_ptr()), _dtype_code(out.dtype),
                              ld, _stream(stream))
    _check("nvfp4_dequantize", st)
    return out


def nvfp4_gemm_workspace_size(A, B, out_dtype=torch.float32, epilogue=NVFP4_EPI_NONE):
    """Bytes of workspace with which nvfp4_gemm splits a last partial round
    of tiles on the current device (0: no split)."""
    ca, cb = A.c(), B.c()
    return int(lib.nvfp4_gemm_workspace_size(ctypes.byref(ca), ctypes.byref(cb), _dtype_code(out_dtype),
                                             epilogue))


@_launches_on_stream
def nvfp4_gemm(A, B, out_dtype=torch.float32, out=None, epilogue=NVFP4_EPI_NONE, workspace=None,
               stream=None):
    """C = A B^T (A: M x K, B: N x K NVFP4 tensors); with NVFP4_EPI_SWIGLU
    (N = 2F, bfloat16 output) C = gate * sigmoid(gate) * up, M x F.
    workspace: None allocates what nvfp4_gemm_workspace_size asks for (a
    split of a last partial round of tiles; often nothing); False passes
    none; a device tensor is passed as is."""
    ncols = B.rows // 2 if epilogue == NVFP4_EPI_SWIGLU else B.rows
    if out is None:
        out = torch.empty((A.rows, ncols), dtype=out_dtype, device=A.codes.device)
    assert out.stride(1) == 1
    ldc = out.stride(0) if A.rows > 1 else max(ncols, out.stride(0))
    ca, cb = A.c(), B.c()
    if workspace is None:
        need = int(lib.nvfp4_gemm_workspace_size(ctypes.byref(ca), ctypes.byref(cb), _dtype_code(out.dtype),
                                                 epilogue))
        workspace = torch.empty((need + 15) // 16 * 4, dtype=torch.float32, device=out.device) if need else False
    if workspace is False:
        workspace = None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.nvfp4_gemm(ctypes.byref(ca), ctypes.byref(cb), ctypes.c_void_p(out.data_ptr()),
                        _dtype_code(out.dtype), ldc, epilogue, _ptr(workspace), ws_bytes, _stream(stream))
    _check("nvfp4_gemm", st)
    return out


@_launches_on_stream
def nvfp4_grouped_gemm(A, offsets, B, groups, epilogue=NVFP4_EPI_NONE, out_dtype=torch.bfloat16,
                       out=None, amax_out=None, stream=None):
    """Per group g: rows offsets[g]..offsets[g+1]-1 of A times B_g^T (B stacks
    `groups` weight matrices).  offsets: int64 device tensor [groups+1]."""
    assert offsets.dtype == torch.int64 and offsets.is_cuda
    ng = B.rows // groups
    ncols = ng // 2 if epilogue == NVFP4_EPI_SWIGLU else ng
    if out is None:
        out = torch.empty((A.rows, ncols), dtype=out_dtype, device=A.codes.device)
    assert out.stride(1) == 1
    ldc = out.stride(0) if A.rows > 1 else max(ncols, out.stride(0))
    ca, cb = A.c(), B.c()
    st = lib.nvfp4_grouped_gemm(groups, ctypes.byref(ca), ctypes.c_void_p(offsets.data_ptr()),
                                ctypes.byref(cb), ctypes.c_void_p(out.data_ptr()),
                                _dtype_code(out.dtype), ldc, epilogue, _ptr(amax_out), None, 0,
                                _stream(stream))
    _check("nvfp4_grouped_gemm", st)
    return out


# ---------------------------------------------------------------- MX formats
@dataclass
class MXTensor:
    """codes uint8 ([rows, cols] for E4M3, [rows, cols/2] for E2M1) and E8M0
    scales uint8 [rows, cols/32] -- device tensors."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    cols: int
    elem: int = NVFP4_MX_E4M3

    def c(self):
        return CMXTensor(self.codes.data_ptr(), self.scales.data_ptr(), self.rows, self.cols, self.elem)

    @staticmethod
    def empty(rows, cols, elem=NVFP4_MX_E4M3, device="cuda"):
        codes = torch.empty((rows, cols if elem == NVFP4_MX_E4M3 else cols // 2), dtype=torch.uint8,
                            device=device)
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=device)
        return MXTensor(codes, scales, rows, cols, elem)


@_launches_on_stream
def nvfp4_mx_quantize(x, layout=NVFP4_ROW_1D, elem=NVFP4_MX_E4M3, round=NVFP4_RNE, sr_seed=0, out=None,
                      stream=None):
    """MX-quantize a 2-D device tensor (float32 or bfloat16, unit column
    stride) along rows (ROW_1D) or columns (COL_1D; the result describes the
    transpose)."""
    assert x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else max(cols, x.stride(0))
    if out is None:
        r, c = (cols, rows) if layout == NVFP4_COL_1D else (rows, cols)
        out = MXTensor.empty(r, c, elem, x.device)
    ct = out.c()
    st = lib.nvfp4_mx_quantize(ctypes.c_void_p(x.data_ptr()), _dtype_code(x.dtype), rows, cols, ld, layout,
                               round, sr_seed, ctypes.byref(ct), _stream(stream))
    _check("nvfp4_mx_quantize", st)
    return out


@_launches_on_stream
def nvfp4_mx_dequantize(q, dtype=torch.float32, out=None, stream=None):
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=dtype, device=q.codes.device)
    assert out.stride(1) == 1
    ld = out.stride(0) if q.rows > 1 else max(q.cols, out.stride(0))
    ct = q.c()
    st = lib.nvfp4_mx_dequantize(ctypes.byref(ct), ctypes.c_void_p(out.data_ptr()), _dtype_code(out.dtype), ld,
                                 _stream(stream))
    _check("nvfp4_mx_dequantize", st)
    return out


def nvfp4_mx_gemm_workspace_size(A, B, out_dtype=torch.float32, accum=NVFP4_MX_ACC_NATIVE):
    """Bytes of workspace with which nvfp4_mx_gemm splits a last partial
    round of tiles on the current device (0: no split)."""
    ca, cb = A.c(), B.c()
    return int(lib.nvfp4_mx_gemm_workspace_size(ctypes.byref(ca), ctypes.byref(cb), _dtype_code(out_dtype),
                                                accum))


@_launches_on_stream
def nvfp4_mx_gemm(A, B, out_dtype=torch.float32, out=None, accum=NVFP4_MX_ACC_NATIVE, workspace=None,
                  stream=None):
    """C = A B^T (A: M x K, B: N x K MX tensors of one element format);
    accum NVFP4_MX_ACC_NATIVE (scaled matrix cores) or NVFP4_MX_ACC_EXACT
    (exact products, binary32 sums).  workspace as for nvfp4_gemm."""
    if out is None:
        out = torch.empty((A.rows, B.rows), dtype=out_dtype, device=A.codes.device)
    assert out.stride(1) == 1
    ldc = out.stride(0) if A.rows > 1 else max(B.rows, out.stride(0))
    ca, cb = A.c(), B.c()
    if workspace is None:
        need = int(lib.nvfp4_mx_gemm_workspace_size(ctypes.byref(ca), ctypes.byref(cb), _dtype_code(out.dtype),
                                                    accum))
        workspace = torch.empty((need + 15) // 16 * 4, dtype=torch.float32, device=out.device) if need else False
    if workspace is False:
        workspace = None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.nvfp4_mx_gemm(ctypes.byref(ca), ctypes.byref(cb), ctypes.c_void_p(out.data_ptr()),
                           _dtype_code(out.dtype), ldc, accum, _ptr(workspace), ws_bytes, _stream(stream))
    _check("nvfp4_mx_gemm", st)
    return out
