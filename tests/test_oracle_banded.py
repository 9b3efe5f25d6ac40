"""The band-parallel oracle driver (oracle/banded.py) gives the single
oracle call's result byte for byte: codes, scale bytes, tensor scale and
amax, for every layout, rounding, input type and the Hadamard transform, with
bands that do not divide the tensor evenly; dequantization and sampled GEMM
entries too.  The GPU parity tests at the workloads' full sizes use it."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from oracle import banded as B


def _x(rows, cols, dtype, seed):
    x = W.with_spikes(W.student_t((rows, cols), 3.0, seed=seed), 2e-3, 60.0, seed=seed + 1)
    x[:16, :16] = 0.0
    return W.f32_to_bf16_bits(x) if dtype == O.BF16 else x


def _same(a, b, what):
    assert a.ts == b.ts, what
    assert a.rows == b.rows and a.cols == b.cols and a.scale_mode == b.scale_mode, what
    assert np.array_equal(a.codes, b.codes), what
    assert np.array_equal(a.scales, b.scales), what


def test_bands_cover_the_range():
    for n, parts, align in [(100, 7, 1), (208, 5, 16), (16, 8, 16), (5, 9, 1), (0, 3, 1)]:
        bs = B.bands(n, parts, align)
        assert len(bs) <= max(parts, 0) or n == 0
        covered = [i for a, b in bs for i in range(a, b)]
        assert covered == list(range(n))
        assert all(a % align == 0 for a, _ in bs)


@pytest.mark.parametrize("dtype", [O.BF16, O.F32])
@pytest.mark.parametrize("rnd", [O.RNE, O.SR])
@pytest.mark.parametrize("layout,had", [(O.ROW_1D, False), (O.ROW_1D, True), (O.COL_1D, False),
                                        (O.COL_1D, True), (O.ROW_COL_1D, False), (O.ROW_COL_1D, True),
                                        (O.BLK_2D, False)])
def test_banded_quantize_equals_single_call(dtype, rnd, layout, had):
    x = _x(208, 176, dtype, seed=3 + layout)
    ref = O.quantize(x, dtype, layout, rnd, sr_seed=41, hadamard=had, hadamard_seed=42)
    got = B.quantize(x, dtype, layout, rnd, sr_seed=41, hadamard=had, hadamard_seed=42, threads=5)
    refs = ref if isinstance(ref, tuple) else (ref,)
    gots = got if isinstance(got, tuple) else (got,)
    for g, r in zip(gots, refs):
        _same(g, r, f"layout {layout} rnd {rnd} had {had}")
    # a given amax (a pair for the two transformed tensors of ROW_COL_1D)
    a = (7.0, 11.0) if (layout == O.ROW_COL_1D and had) else 7.0
    ref = O.quantize(x, dtype, layout, rnd, sr_seed=41, hadamard=had, hadamard_seed=42, amax_in=a)
    got = B.quantize(x, dtype, layout, rnd, sr_seed=41, hadamard=had, hadamard_seed=42, amax_in=a, threads=3)
    refs = ref if isinstance(ref, tuple) else (ref,)
    gots = got if isinstance(got, tuple) else (got,)
    for g, r in zip(gots, refs):
        _same(g, r, f"given amax: layout {layout} rnd {rnd} had {had}")


@pytest.mark.parametrize("layout,had", [(O.ROW_1D, False), (O.ROW_1D, True), (O.COL_1D, True), (O.BLK_2D, False)])
def test_banded_amax(layout, had):
    x = _x(160, 96, O.BF16, seed=9)
    assert B.amax(x, O.BF16, layout, had, 5, threads=6) == O.amax(x, O.BF16, layout, had, 5)


@pytest.mark.parametrize("layout", [O.ROW_1D, O.BLK_2D])
@pytest.mark.parametrize("out", [O.F32, O.BF16])
def test_banded_dequantize(layout, out):
    x = _x(96, 128, O.F32, seed=12)
    q = O.quantize(x, O.F32, layout, O.SR, sr_seed=3)
    assert np.array_equal(B.dequantize(q, out, threads=4), O.dequantize(q, out))


def test_banded_gemm_entries():
    A = O.quantize(_x(64, 96, O.F32, seed=21), O.F32, O.ROW_1D)
    Bq = O.quantize(W.normal((48, 96), 0.02, seed=22), O.F32, O.BLK_2D)
    g = W.rng(23)
    mi, ni = g.integers(0, 64, 101), g.integers(0, 48, 101)
    c, w = B.gemm_entries(A, Bq, mi, ni, threads=4)
    c1, w1 = O.gemm(A, Bq, entries=(mi, ni))
    assert np.array_equal(c, c1) and np.array_equal(w, w1)


def test_banded_gemms_and_mx_quantize():
    A = O.quantize(_x(70, 96, O.F32, seed=31), O.F32, O.ROW_1D)
    Bq = O.quantize(W.normal((48, 96), 0.02, seed=32), O.F32, O.BLK_2D)
    for got, ref in zip(B.gemm(A, Bq, threads=3), O.gemm(A, Bq)):
        assert np.array_equal(got, ref)
    x = _x(96, 128, O.F32, seed=33)
    for elem in (O.MX_FP8, O.MX_FP4):
        for rnd in (O.RNE, O.SR):
            q = B.mx_quantize(x, O.F32, elem, rnd, seed=34, threads=5)
            r = O.mx_quantize(x, O.F32, O.ROW_1D, elem, rnd, seed=34)
            assert np.array_equal(q.codes, r.codes) and np.array_equal(q.scales, r.scales)
        qb = O.mx_quantize(_x(40, 128, O.F32, seed=35), O.F32, O.ROW_1D, elem)
        for got, ref in zip(B.mx_gemm(r, qb, threads=4), O.mx_gemm(r, qb)):
            assert np.array_equal(got, ref)
        mi, ni = np.array([0, 5, 95, 3]), np.array([1, 39, 0, 7])
        for got, ref in zip(B.mx_gemm(r, qb, entries=(mi, ni), threads=2), O.mx_gemm(r, qb, entries=(mi, ni))):
            assert np.array_equal(got, ref)
