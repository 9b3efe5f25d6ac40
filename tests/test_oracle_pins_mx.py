"""CPU pins of the oracle's MX formats (OCP Microscaling: the reading for the
MXFP8 / MXFP4 formats the pages name, and for the 8.25-bit transit format of
"Thinking Machines ускорила обучение Inkling 2 Small 4-битными числами",
iitak.ru, section "Но"): each check compares the oracle with something other
than itself -- closed forms, torch's float8_e4m3fn conversion, exhaustive
draw counts, exact rational arithmetic."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


def test_scale_exponent_closed_forms():
    f = O.lib().orc_mx_scale_exp
    assert f(1.0, O.MX_FP8) == -8 and f(1.0, O.MX_FP4) == -2
    assert f(448.0, O.MX_FP8) == 0 and f(511.0, O.MX_FP8) == 0 and f(512.0, O.MX_FP8) == 1
    assert f(6.0, O.MX_FP4) == 0 and f(7.9, O.MX_FP4) == 0 and f(8.0, O.MX_FP4) == 1
    assert f(0.0, O.MX_FP8) == -127
    assert f(2.0 ** -140, O.MX_FP8) == -127                 # clamped at the E8M0 minimum
    assert f(3.0e38, O.MX_FP4) == 125                      # floor(log2(3e38)) = 127
    assert f(np.float32(1.4e-45), O.MX_FP4) == -127


def test_block_layout_saturation_and_bits_per_number():
    """One block whose largest magnitude is 500: scale 2^(8-8) = 1 (byte 127),
    500 clamps to 448; 8-bit codes plus an 8-bit scale per 32 is 8.25 bits."""
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 3] = 500.0
    x[0, 5] = -1.0
    q = O.mx_quantize(x, O.F32, O.ROW_1D, O.MX_FP8)
    assert q.scales[0, 0] == 127
    assert q.codes[0, 3] == 0x7E and q.codes[0, 5] == 0xB8    # 448 and -1.0
    bits = (q.codes.nbytes + q.scales.nbytes) * 8 / x.size
    assert bits == 8.25


def test_fp8_rne_elements_match_torch_float8_e4m3fn():
    x = W.student_t((64, 256), 3.0, seed=11)
    q = O.mx_quantize(x, O.F32, O.ROW_1D, O.MX_FP8, O.RNE)
    s = q.scales.astype(np.int64) - 127
    y = x * np.repeat(np.ldexp(1.0, -s), 32, axis=1).astype(np.float32)
    y = np.clip(y, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q.codes, ref)


def test_fp4_elements_are_the_nvfp4_e2m1_rounding():
    x = W.student_t((32, 128), 3.0, seed=12)
    for rnd in (O.RNE, O.SR):
        q = O.mx_quantize(x, O.F32, O.ROW_1D, O.MX_FP4, rnd, seed=5)
        s = q.scales.astype(np.int64) - 127
        for r in range(0, 32, 7):
            for c in range(0, 128, 5):
                y = np.float32(abs(x[r, c])) * np.float32(np.ldexp(1.0, -s[r, c // 32]))
                draw = O.lib().orc_draw16(5, O.STREAM_MX_ROW, r * 128 + c)
                mag = O.lib().orc_e2m1_sr(y, draw) if rnd == O.SR else O.lib().orc_e2m1_rne(y)
                code = (q.codes[r, c // 2] >> (4 * (c % 2))) & 15
                assert code == ((8 if np.signbit(x[r, c]) else 0) | mag)


@pytest.mark.parametrize("y,lo,hi", [(1.0625, 0x38, 0x39), (0.0029296875, 0x01, 0x02),
                                     (416.5, 0x7D, 0x7E), (0.001, 0x00, 0x01)])
def test_e4m3_stochastic_rounding_counts(y, lo, hi):
    """Exhaustive over all 2^16 draws: the count of round-ups is ceil(f 2^16),
    f the exact position of y between its neighbours."""
    f = O.lib().orc_e4m3_sr
    codes = np.array([f(y, r) for r in range(65536)])
    assert set(np.unique(codes)) <= {lo, hi}
    vlo, vhi = O.lib().orc_e4m3_value(lo), O.lib().orc_e4m3_value(hi)
    frac = (Fraction(float(np.float32(y))) - Fraction(vlo)) / (Fraction(vhi) - Fraction(vlo))
    ups = int((codes == hi).sum())
    assert ups == -((-frac * 65536).numerator // (frac * 65536).denominator)


def test_e4m3_sr_saturates_and_keeps_exact_values():
    f = O.lib().orc_e4m3_sr
    assert all(f(448.0, r) == 0x7E for r in (0, 1, 65535))
    assert all(f(1000.0, r) == 0x7E for r in (0, 65535))
    assert all(f(1.125, r) == 0x39 for r in (0, 65535))
    assert f(0.0, 0) == 0


@pytest.mark.parametrize("elem", [O.MX_FP8, O.MX_FP4])
def test_dequantize_of_quantize_is_a_fixed_point(elem):
    """MX values are exactly representable, and a block's largest magnitude
    keeps its power-of-two range, so quantizing the dequantized tensor
    reproduces codes and scales."""
    x = W.student_t((64, 128), 3.0, seed=13)
    q = O.mx_quantize(x, O.F32, O.ROW_1D, elem)
    d = O.mx_dequantize(q, O.F32)
    q2 = O.mx_quantize(d, O.F32, O.ROW_1D, elem)
    assert np.array_equal(q.codes, q2.codes) and np.array_equal(q.scales, q2.scales)


def test_column_layout_is_row_layout_of_the_transpose():
    x = W.student_t((64, 96), 3.0, seed=14)
    for elem in (O.MX_FP8, O.MX_FP4):
        a = O.mx_quantize(x, O.F32, O.COL_1D, elem, O.RNE)
        b = O.mx_quantize(np.ascontiguousarray(x.T), O.F32, O.ROW_1D, elem, O.RNE)
        assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales)


def _exact(q):
    out = []
    for r in range(q.rows):
        row = []
        for c in range(q.cols):
            code = int(q.codes[r, c]) if q.elem == O.MX_FP8 else int(q.codes[r, c // 2] >> (4 * (c % 2))) & 15
            v = Fraction(O.lib().orc_mx_elem_value(code, q.elem))
            row.append(v * Fraction(2) ** (int(q.scales[r, c // 32]) - 127))
        out.append(row)
    return out


@pytest.mark.parametrize("ea,eb", [(O.MX_FP8, O.MX_FP8), (O.MX_FP4, O.MX_FP4), (O.MX_FP8, O.MX_FP4)])
def test_mx_gemm_against_rational_brute_force(ea, eb):
    a = W.with_spikes(W.normal((5, 64), 1.0, seed=15), 0.05, 40.0, seed=16)
    b = W.normal((4, 64), 0.02, seed=17)
    A, B = O.mx_quantize(a, O.F32, O.ROW_1D, ea), O.mx_quantize(b, O.F32, O.ROW_1D, eb)
    C, Wt = O.mx_gemm(A, B)
    ea_, eb_ = _exact(A), _exact(B)
    for m in range(5):
        for n in range(4):
            s = sum(x * y for x, y in zip(ea_[m], eb_[n]))
            w = sum(abs(x * y) for x, y in zip(ea_[m], eb_[n]))
            assert abs(Fraction(C[m, n]) - s) <= Fraction(w) * Fraction(1, 2 ** 50)
            assert abs(Fraction(Wt[m, n]) - w) <= Fraction(w) * Fraction(1, 2 ** 50)
