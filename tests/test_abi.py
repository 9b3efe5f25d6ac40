"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/nvfp4.h, and rejects invalid arguments on the host
before anything is launched (those paths make no HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


@pytest.fixture(scope="module")
def nv():
    import bit_block_scaled_quantize_amd.nvfp4 as nv
    return nv


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_four_operations():
    fns = declared_functions()
    for f in ["nvfp4_quantize", "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_grouped_gemm"]:
        assert f in fns


def test_library_exports_every_declared_symbol(nv):
    lib = ctypes.CDLL(nv.LIB_PATH)
    for f in declared_functions():
        assert hasattr(lib, f), f
    assert sorted(nv.EXPORTED) == declared_functions()


def test_status_strings_and_version(nv):
    for s in range(8):
        assert nv.lib.nvfp4_status_string(s)
    assert nv.lib.nvfp4_version() >= 100


def test_workspace_size(nv):
    assert nv.nvfp4_quantize_workspace_size(8192, 8192) > 0
    o = nv.CQuantOpts(0, 0, 0, 0, 0, 1234, None)
    assert nv.lib.nvfp4_quantize_workspace_size(8192, 8192, ctypes.byref(o)) == 0


def _t(rows, cols, mode=0, codes=4096, scales=8192, ts=16384):
    import bit_block_scaled_quantize_amd.nvfp4 as nv
    return nv.CTensor(codes, scales, ts, rows, cols, mode)


def _quant(nv, x=65536, dt=1, rows=32, cols=32, ld=32, layout=0, rnd=0, had=0, outs=None,
           ws=1 << 20, ws_bytes=1 << 20, amax=None):
    o = nv.CQuantOpts(layout, rnd, 1, had, 2, amax, None)
    arr = (nv.CTensor * 2)()
    if outs is None:
        outs = [_t(rows, cols)]
    for i, t in enumerate(outs):
        arr[i] = t
    return nv.lib.nvfp4_quantize(x, dt, rows, cols, ld, ctypes.byref(o), arr, ws, ws_bytes, None)


def test_quantize_rejects_bad_arguments(nv):
    E = dict(NULL=1, ENUM=2, SHAPE=3, ALIGN=4, UNSUP=5, WS=6)
    assert _quant(nv, x=None) == E["NULL"]
    assert _quant(nv, dt=7) == E["ENUM"]
    assert _quant(nv, layout=9) == E["ENUM"]
    assert _quant(nv, rnd=5) == E["ENUM"]
    assert _quant(nv, cols=24, ld=32, outs=[_t(32, 24)]) == E["SHAPE"]        # cols % 16
    assert _quant(nv, rows=24, layout=1, outs=[_t(32, 24)]) == E["SHAPE"]     # rows % 16 (COL)
    assert _quant(nv, ld=16) == E["SHAPE"]                                     # ld < cols
    assert _quant(nv, ld=36) == E["ALIGN"]                                     # 72 bytes
    assert _quant(nv, x=65536 + 2) == E["ALIGN"]
    assert _quant(nv, layout=3, had=1, outs=[_t(32, 32, 1)]) == E["UNSUP"]
    # ROW_COL_1D with the transform is supported; its outputs are still checked
    assert _quant(nv, layout=2, had=1, outs=[_t(32, 32), _t(16, 32)]) == E["SHAPE"]
    assert _quant(nv, outs=[_t(32, 32, 1)]) == E["SHAPE"]                     # wrong scale mode
    assert _quant(nv, layout=1, outs=[_t(32, 64)]) == E["SHAPE"]              # COL output shape
    assert _quant(nv, outs=[_t(32, 32, codes=None)]) == E["NULL"]
    assert _quant(nv, outs=[_t(32, 32, codes=4100)]) == E["ALIGN"]
    assert _quant(nv, ws=None) == E["WS"]
    assert _quant(nv, ws_bytes=16) == E["WS"]


def test_dequantize_rejects_bad_arguments(nv):
    q = _t(32, 32)
    assert nv.lib.nvfp4_dequantize(None, 65536, 0, 32, None) == 1
    assert nv.lib.nvfp4_dequantize(ctypes.byref(q), None, 0, 32, None) == 1
    assert nv.lib.nvfp4_dequantize(ctypes.byref(q), 65536, 3, 32, None) == 2
    assert nv.lib.nvfp4_dequantize(ctypes.byref(q), 65536, 0, 16, None) == 3
    assert nv.lib.nvfp4_dequantize(ctypes.byref(q), 65540, 0, 32, None) == 4
    bad = _t(32, 24)
    assert nv.lib.nvfp4_dequantize(ctypes.byref(bad), 65536, 0, 32, None) == 3
    bad2 = _t(24, 32, 1)
    assert nv.lib.nvfp4_dequantize(ctypes.byref(bad2), 65536, 0, 32, None) == 3


def test_requantize_rejects_bad_arguments(nv):
    def call(q, layout=1, rnd=0, out=None, ws=1 << 20, ws_bytes=1 << 20, amax=None):
        o = nv.CQuantOpts(layout, rnd, 1, 0, 2, amax, None)
        out = _t(q.cols, q.rows) if out is None else out
        return nv.lib.nvfp4_requantize(ctypes.byref(q), ctypes.byref(o), ctypes.byref(out), ws, ws_bytes,
                                       None)

    q = _t(64, 32)
    o = nv.CQuantOpts(1, 0, 1, 0, 2, None, None)
    assert nv.lib.nvfp4_requantize(None, ctypes.byref(o), ctypes.byref(_t(32, 64)), 1 << 20, 1 << 20,
                                   None) == 1
    assert call(q, layout=7) == 2
    assert call(q, rnd=5) == 2
    assert call(q, layout=0) == 5                     # only COL_1D re-quantization
    assert call(_t(64, 32, 1)) == 5                   # input must carry row-block scales
    assert call(_t(40, 32)) == 3                      # rows % 16
    assert call(q, out=_t(64, 32)) == 3               # output is cols x rows
    assert call(q, out=_t(32, 64, codes=4100)) == 4
    assert call(q, ws=None) == 6
    assert call(q, ws_bytes=16) == 6


def test_gemm_rejects_bad_arguments(nv):
    a, b = _t(64, 64), _t(32, 64)
    g = nv.lib.nvfp4_gemm
    assert g(None, ctypes.byref(b), 65536, 0, 32, 0, None, 0, None) == 1
    assert g(ctypes.byref(a), ctypes.byref(b), 65536, 9, 32, 0, None, 0, None) == 2
    assert g(ctypes.byref(a), ctypes.byref(b), 65536, 0, 32, 1, None, 0, None) == 5     # SwiGLU: BF16 output only
    assert g(ctypes.byref(a), ctypes.byref(b), 65536, 1, 15, 1, None, 0, None) == 3     # SwiGLU: ldc < F = 16
    b48 = _t(48, 64)
    assert g(ctypes.byref(a), ctypes.byref(b48), 65536, 1, 24, 1, None, 0, None) == 3   # SwiGLU: F = 24 not % 16
    b2 = _t(32, 48)
    assert g(ctypes.byref(a), ctypes.byref(b2), 65536, 0, 32, 0, None, 0, None) == 3    # K mismatch
    assert g(ctypes.byref(a), ctypes.byref(b), 65536, 0, 16, 0, None, 0, None) == 3     # ldc < N
    assert g(ctypes.byref(a), ctypes.byref(b), None, 0, 32, 0, None, 0, None) == 1
    a3 = _t(64, 40)
    b3 = _t(32, 40)
    assert g(ctypes.byref(a3), ctypes.byref(b3), 65536, 0, 32, 0, None, 0, None) == 3   # K % 16
    assert g(ctypes.byref(a), ctypes.byref(b), 65536, 0, 32, 0, 4100, 1 << 20, None) == 4   # ws misaligned
    s = nv.lib.nvfp4_gemm_workspace_size
    assert s(ctypes.byref(a), ctypes.byref(b), 9, 0) == 0      # invalid dtype
    assert s(ctypes.byref(a), ctypes.byref(b48), 1, 1) == 0    # SwiGLU: no split
    assert s(None, ctypes.byref(b), 0, 0) == 0


def test_grouped_gemm_rejects_bad_arguments(nv):
    a, b = _t(100, 64), _t(4 * 32, 64, 1)
    g = nv.lib.nvfp4_grouped_gemm
    args = lambda **k: dict(dict(G=4, A=ctypes.byref(a), off=65536, B=ctypes.byref(b), C=65536,
                                 dt=1, ldc=32, ep=0, amax=None), **k)

    def call(d):
        return g(d["G"], d["A"], d["off"], d["B"], d["C"], d["dt"], d["ldc"], d["ep"], d["amax"],
                 None, 0, None)

    assert call(args(off=None)) == 1
    assert call(args(G=0)) == 3
    assert call(args(G=3)) == 3                      # B rows not divisible by G
    assert call(args(ep=1, dt=0, ldc=16)) == 5       # SwiGLU needs bf16 output
    assert call(args(ep=1, ldc=8)) == 3              # ldc < F
    assert call(args(amax=65536)) == 5               # amax only with SwiGLU
    a2 = _t(100, 64, 1)
    assert call(args(A=ctypes.byref(a2))) == 3 or call(args(A=ctypes.byref(a2))) == 5


def test_mx_rejects_bad_arguments(nv):
    E = dict(NULL=1, ENUM=2, SHAPE=3, ALIGN=4, UNSUP=5)

    def q(x=65536, dt=1, rows=64, cols=64, ld=64, layout=0, rnd=0, out=(64, 64), elem=0, codes=4096):
        t = nv.CMXTensor(codes, 8192, out[0], out[1], elem) if out is not None else None
        return nv.lib.nvfp4_mx_quantize(x, dt, rows, cols, ld, layout, rnd, 1,
                                        ctypes.byref(t) if t is not None else None, None)

    assert q(out=None) == E["NULL"]
    assert q(x=None) == E["NULL"]
    assert q(dt=3) == E["ENUM"]
    assert q(layout=7) == E["ENUM"]
    assert q(rnd=2) == E["ENUM"]
    assert q(elem=2) == E["ENUM"]
    assert q(layout=2) == E["UNSUP"]                       # ROW_COL is not offered for MX
    assert q(layout=3) == E["UNSUP"]
    assert q(cols=48, ld=48, out=(64, 48)) == E["SHAPE"]   # cols % 32 (ROW)
    assert q(rows=48, layout=1, out=(64, 48)) == E["SHAPE"]  # rows % 32 (COL)
    assert q(layout=1, rows=64, cols=96, ld=96, out=(64, 96)) == E["SHAPE"]  # COL output is the transpose
    assert q(ld=32) == E["SHAPE"]
    assert q(ld=68) == E["ALIGN"]                          # 136 bytes
    assert q(codes=4096 + 8) == E["ALIGN"]
    assert q(rows=0, x=None, codes=None, out=(0, 64)) == 0  # empty: a no-op

    def dq(rows=64, cols=64, elem=0, y=65536, dt=0, ld=64):
        t = nv.CMXTensor(4096, 8192, rows, cols, elem)
        return nv.lib.nvfp4_mx_dequantize(ctypes.byref(t), y, dt, ld, None)

    assert nv.lib.nvfp4_mx_dequantize(None, 65536, 0, 64, None) == E["NULL"]
    assert dq(elem=5) == E["ENUM"]
    assert dq(dt=9) == E["ENUM"]
    assert dq(cols=48, ld=48) == E["SHAPE"]
    assert dq(ld=32) == E["SHAPE"]
    assert dq(y=None) == E["NULL"]
    assert dq(y=65536 + 4) == E["ALIGN"]
    assert dq(ld=66) == E["ALIGN"]                          # 264 bytes (fp32)


def test_mx_gemm_rejects_bad_arguments(nv):
    E = dict(NULL=1, ENUM=2, SHAPE=3, ALIGN=4, UNSUP=5)

    def g(ma=(64, 128, 0), mb=(32, 128, 0), C=65536, dt=0, ldc=32, ac=4096, asc=8192, acc=0):
        a = nv.CMXTensor(ac, asc, ma[0], ma[1], ma[2])
        b = nv.CMXTensor(4096, 8192, mb[0], mb[1], mb[2])
        return nv.lib.nvfp4_mx_gemm(ctypes.byref(a), ctypes.byref(b), C, dt, ldc, acc, None, 0, None)

    assert nv.lib.nvfp4_mx_gemm(None, None, 65536, 0, 32, 0, None, 0, None) == E["NULL"]
    assert g(dt=4) == E["ENUM"]
    assert g(acc=2) == E["ENUM"]
    assert g(acc=-1) == E["ENUM"]
    assert g(ma=(64, 128, 3)) == E["ENUM"]
    assert g(ma=(64, 96, 0), mb=(32, 96, 0)) == E["UNSUP"]       # K % 64 == 32
    assert g(ma=(64, 80, 0), mb=(32, 80, 0)) == E["SHAPE"]       # K % 32
    assert g(mb=(32, 192, 0)) == E["SHAPE"]                      # K mismatch
    assert g(mb=(32, 128, 1)) == E["UNSUP"]                      # mixed element formats
    assert g(ldc=16) == E["SHAPE"]
    assert g(C=None) == E["NULL"]
    assert g(C=65536 + 2) == E["ALIGN"]
    assert g(ac=4096 + 4) == E["ALIGN"]
    assert g(asc=8192 + 1) == E["ALIGN"]
    assert g(ma=(-1, 128, 0)) == E["SHAPE"]
    # per-lane 32-bit byte offsets inside a 256-row tile: code rows below 2^24 bytes
    K4 = 1 << 24                                                 # E4M3: 2^24 bytes per row
    assert g(ma=(64, K4, 0), mb=(32, K4, 0)) == E["UNSUP"]
    assert g(ma=(64, 2 * K4, 1), mb=(32, 2 * K4, 1)) == E["UNSUP"]   # E2M1: K/2 bytes per row
    assert g(ma=(64, K4, 0), mb=(32, K4, 0), acc=1) == E["UNSUP"]     # the exact path shares the limit


def test_quantize_noalloc_rejects_bad_arguments(nv):
    """The allocation-free variant validates like nvfp4_quantize (before it
    looks anything up on a device)."""
    E = dict(NULL=1, ENUM=2, SHAPE=3, ALIGN=4, UNSUP=5)

    def q(x=65536, dt=1, rows=32, cols=32, ld=32, layout=0, had=0, outs=None):
        o = nv.CQuantOpts(layout, 0, 1, had, 2, None, None)
        arr = (nv.CTensor * 2)()
        for i, t in enumerate(outs or [_t(rows, cols)]):
            arr[i] = t
        return nv.lib.nvfp4_quantize_noalloc(x, dt, rows, cols, ld, ctypes.byref(o), arr, None)

    assert nv.lib.nvfp4_quantize_noalloc(65536, 1, 32, 32, 32, None, None, None) == E["NULL"]
    assert q(x=None) == E["NULL"]
    assert q(dt=5) == E["ENUM"]
    assert q(cols=24, ld=32, outs=[_t(32, 24)]) == E["SHAPE"]
    assert q(ld=36) == E["ALIGN"]
    assert q(layout=3, had=1, outs=[_t(32, 32, 1)]) == E["UNSUP"]
    assert q(outs=[_t(32, 32, 1)]) == E["SHAPE"]
