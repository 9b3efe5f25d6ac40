"""Band-parallel driver of the C oracle -- TEST INFRASTRUCTURE ONLY.

Runs the unchanged oracle functions of nvfp4_oracle.c on independent bands of
a tensor, one plain oracle call per band, in a pool of threads (a ctypes call
releases the GIL, so the calls run on separate cores).  The bands are the
ones the format makes independent once the tensor amax A_t is fixed:
  - rows of a row-blocked output (ROW_1D), 16-row bands of a 16x16-blocked one
    (BLK_2D): input rows [r0, r1);
  - rows of a column-blocked output (COL_1D), i.e. input columns [c0, c1);
and the Hadamard transform never crosses them (it runs along the block
dimension).  Each band gets, through the oracle's index_base, the random-draw
indices its elements have in the whole output tensor, so the assembled result
is byte for byte the single call's (tests/test_oracle_banded.py checks that).
A_t itself is the maximum of the bands' maxima (orc_amax per band).
ROW_COL_1D is the ROW_1D and COL_1D outputs, which is how the oracle defines
it.  The GEMM references split their output rows (or listed entries) the same
way: every output entry is its own oracle dot product.  Nothing here does any
of the method's arithmetic.
"""
import concurrent.futures
import ctypes
import os

import numpy as np

from . import oracle as O

_U8P = ctypes.POINTER(ctypes.c_uint8)
_F32P = ctypes.POINTER(ctypes.c_float)


def default_threads():
    """Cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def bands(n, parts, align=1):
    """[0, n) as at most `parts` contiguous ranges whose starts are multiples
    of `align`."""
    if n <= 0:
        return []
    units = -(-n // align)
    per = -(-units // max(1, parts))
    out = []
    for u0 in range(0, units, per):
        out.append((u0 * align, min(n, (u0 + per) * align)))
    return out


def _run(fn, jobs, threads):
    if threads <= 1 or len(jobs) <= 1:
        return [fn(*j) for j in jobs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda j: fn(*j), jobs))


def _at(a, byte_offset, ctype=ctypes.c_uint8):
    return ctypes.cast(a.ctypes.data + byte_offset, ctypes.POINTER(ctype))


def amax(x, dtype, layout, hadamard=False, hadamard_seed=0, threads=None):
    """A_t of the tensor `layout` quantizes: the largest of the bands'
    oracle amaxes (ROW_1D / BLK_2D: row bands; COL_1D: column bands)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    threads = threads or default_threads()
    es = x.dtype.itemsize
    lib = O.lib()
    if layout == O.COL_1D:
        jobs = [(c0, c1) for c0, c1 in bands(cols, 4 * threads)]

        def one(c0, c1):
            return lib.orc_amax(ctypes.c_void_p(x.ctypes.data + c0 * es), dtype, rows, c1 - c0, cols,
                                layout, int(bool(hadamard)), ctypes.c_uint64(hadamard_seed))
    else:
        jobs = [(r0, r1) for r0, r1 in bands(rows, 4 * threads, 16 if layout == O.BLK_2D else 1)]

        def one(r0, r1):
            return lib.orc_amax(ctypes.c_void_p(x.ctypes.data + r0 * cols * es), dtype, r1 - r0, cols, cols,
                                layout, int(bool(hadamard)), ctypes.c_uint64(hadamard_seed))
    vals = _run(one, jobs, threads)
    return float(max(vals)) if vals else 0.0


def quantize(x, dtype, layout, rnd=O.RNE, sr_seed=0, hadamard=False, hadamard_seed=0, amax_in=None,
             threads=None):
    """O.quantize computed band by band in threads; the same result.
    Returns one QTensor, or (row, col) for ROW_COL_1D."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    threads = threads or default_threads()
    if layout == O.ROW_COL_1D:
        if amax_in is None:
            a_row = amax(x, dtype, O.ROW_1D, hadamard, hadamard_seed, threads)
            a_col = amax(x, dtype, O.COL_1D, hadamard, hadamard_seed, threads) if hadamard else a_row
        else:
            pair = np.atleast_1d(np.asarray(amax_in, dtype=np.float32))
            a_row = float(pair[0])
            a_col = float(pair[1]) if hadamard else a_row
        r = quantize(x, dtype, O.ROW_1D, rnd, sr_seed, hadamard, hadamard_seed, a_row, threads)
        c = quantize(x, dtype, O.COL_1D, rnd, sr_seed, hadamard, hadamard_seed, a_col, threads)
        return r, c
    a = amax(x, dtype, layout, hadamard, hadamard_seed, threads) if amax_in is None else float(amax_in)
    a_arr = np.array([a], dtype=np.float32)
    es = x.dtype.itemsize
    lib = O.lib()
    col = layout == O.COL_1D
    R, C = (cols, rows) if col else (rows, cols)
    codes = np.zeros((R, C // 2), dtype=np.uint8)
    if layout == O.BLK_2D:
        scales = np.zeros((R // 16, C // 16), dtype=np.uint8)
    else:
        scales = np.zeros((R, C // 16), dtype=np.uint8)
    nul8 = _U8P()
    nulf = _F32P()
    if col:
        jobs = bands(cols, 4 * threads)
    else:
        jobs = bands(rows, 4 * threads, 16 if layout == O.BLK_2D else 1)

    def one(o0, o1):
        # band of the output rows [o0, o1): input columns (COL_1D) or input rows
        ts = np.zeros(1, dtype=np.float32)
        if col:
            xp, br, bc, base = x.ctypes.data + o0 * es, rows, o1 - o0, o0 * rows
        else:
            xp, br, bc, base = x.ctypes.data + o0 * cols * es, o1 - o0, cols, o0 * cols
        srow = o0 // 16 if layout == O.BLK_2D else o0
        rc = lib.orc_quantize(ctypes.c_void_p(xp), dtype, br, bc, cols, layout, rnd, ctypes.c_uint64(sr_seed),
                              int(bool(hadamard)), ctypes.c_uint64(hadamard_seed),
                              a_arr.ctypes.data_as(_F32P), ctypes.c_uint64(base),
                              _at(codes, o0 * codes.shape[1]), _at(scales, srow * scales.shape[1]),
                              ts.ctypes.data_as(_F32P), nul8, nul8, nulf)
        if rc != 0:
            raise ValueError(f"oracle quantize rejected a band (code {rc})")
        return float(ts[0])

    ts_all = _run(one, jobs, threads)
    ts = ts_all[0] if ts_all else O.tensor_scale(a)
    return O.QTensor(codes, scales, ts, R, C, O.SCALE_2D if layout == O.BLK_2D else O.SCALE_1D)


def dequantize(q, out_dtype=O.F32, threads=None):
    """O.dequantize computed over row bands of the stored tensor in threads."""
    threads = threads or default_threads()
    out = np.zeros((q.rows, q.cols), dtype=np.uint16 if out_dtype == O.BF16 else np.float32)
    lib = O.lib()
    two_d = q.scale_mode == O.SCALE_2D
    codes, scales = np.ascontiguousarray(q.codes), np.ascontiguousarray(q.scales)

    def one(r0, r1):
        srow = r0 // 16 if two_d else r0
        lib.orc_dequantize(_at(codes, r0 * codes.shape[1]), _at(scales, srow * scales.shape[1]),
                           ctypes.c_float(q.ts), r1 - r0, q.cols, q.scale_mode,
                           ctypes.c_void_p(out.ctypes.data + r0 * q.cols * out.itemsize), out_dtype)

    _run(one, bands(q.rows, 4 * threads, 16 if two_d else 1), threads)
    return out


def gemm_entries(A, B, m_idx, n_idx, threads=None):
    """O.gemm on the listed output entries, the list split over threads;
    returns (C, W) as O.gemm does."""
    threads = threads or default_threads()
    mi = np.ascontiguousarray(m_idx, dtype=np.int64)
    ni = np.ascontiguousarray(n_idx, dtype=np.int64)
    C = np.zeros(mi.size, dtype=np.float64)
    Wt = np.zeros(mi.size, dtype=np.float64)

    def one(e0, e1):
        c, w = O.gemm(A, B, entries=(mi[e0:e1], ni[e0:e1]))
        C[e0:e1], Wt[e0:e1] = c, w

    _run(one, bands(mi.size, 4 * threads), threads)
    return C, Wt


def _row_slice_mx(q, r0, r1):
    return O.MXTensor(np.ascontiguousarray(q.codes[r0:r1]), np.ascontiguousarray(q.scales[r0:r1]),
                      r1 - r0, q.cols, q.elem)


def _gemm_rows(gemm, slice_rows, A, B, entries, threads):
    threads = threads or default_threads()
    if entries is not None:
        mi = np.ascontiguousarray(entries[0], dtype=np.int64)
        ni = np.ascontiguousarray(entries[1], dtype=np.int64)
        C = np.zeros(mi.size, dtype=np.float64)
        Wt = np.zeros(mi.size, dtype=np.float64)

        def one(e0, e1):
            C[e0:e1], Wt[e0:e1] = gemm(A, B, entries=(mi[e0:e1], ni[e0:e1]))

        _run(one, bands(mi.size, 4 * threads), threads)
        return C, Wt
    C = np.zeros((A.rows, B.rows), dtype=np.float64)
    Wt = np.zeros((A.rows, B.rows), dtype=np.float64)

    def one(r0, r1):
        C[r0:r1], Wt[r0:r1] = gemm(slice_rows(A, r0, r1), B)

    _run(one, bands(A.rows, 4 * threads, 16), threads)
    return C, Wt


def gemm(A, B, entries=None, threads=None):
    """O.gemm with the output rows (or the listed entries) split over
    threads; the same (C, W).  For the whole output A must be row-blocked
    (SCALE_1D) or split on 16-row bands (SCALE_2D)."""
    def rows_of(q, r0, r1):
        if q.scale_mode == O.SCALE_2D:
            assert r0 % 16 == 0 and (r1 % 16 == 0 or r1 == q.rows)
        return O.row_slice(q, r0, r1)
    return _gemm_rows(O.gemm, rows_of, A, B, entries, threads)


def mx_gemm(A, B, entries=None, threads=None):
    """O.mx_gemm with the output rows (or the listed entries) split over
    threads; the same (C, W)."""
    return _gemm_rows(O.mx_gemm, _row_slice_mx, A, B, entries, threads)


def mx_quantize(x, dtype, elem, rnd=O.RNE, seed=0, threads=None):
    """O.mx_quantize (ROW_1D) band by band over rows, each band with the
    random-draw index base of its first row; the same result."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    threads = threads or default_threads()
    out = O.MXTensor(np.zeros((rows, cols if elem == O.MX_FP8 else cols // 2), dtype=np.uint8),
                     np.zeros((rows, cols // 32), dtype=np.uint8), rows, cols, elem)

    def one(r0, r1):
        q = O.mx_quantize(x[r0:r1], dtype, O.ROW_1D, elem, rnd, seed=seed, index_base=r0 * cols)
        out.codes[r0:r1], out.scales[r0:r1] = q.codes, q.scales

    _run(one, bands(rows, 4 * threads), threads)
    return out
