"""Pins of the CPU oracle against what the NVFP4 pages and mathematics fix.

None of these tests re-types an oracle formula: each compares the oracle with
a value printed on the pages (tests/golden/page_examples.json), a closed form,
an invariant, a brute-force search, or an independent library routine
(rocRAND's Philox4x32-10 engine, torch's float8_e4m3fn and bfloat16
conversions, scipy's Sylvester Hadamard matrix).
"""
import json
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle as O
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "page_examples.json")))
MAGS = [Fraction(v).limit_denominator(4) for v in GOLD["e2m1_magnitudes"]["values"]]


# ------------------------------------------------------------------ E2M1
def test_e2m1_value_set_matches_pages():
    g = GOLD["e2m1_magnitudes"]
    vals = [O.e2m1_value(c) for c in range(16)]
    assert len(vals) == g["n_codes"]
    assert sorted(set(abs(v) for v in vals)) == sorted(float(v) for v in g["values"])
    assert min(vals) == g["min"] and max(vals) == g["max"]
    for v in g["not_representable"]:
        assert v not in vals and -v not in vals
    # sign bit is bit 3; code 8 is negative zero
    assert np.signbit(vals[8]) and vals[8] == 0.0
    for c in range(8):
        assert vals[c + 8] == -vals[c]
    # 1 sign + 2 exponent + 1 mantissa bits = 4 bits per code
    b = GOLD["e2m1_bits"]
    assert b["sign"] + b["exponent"] + b["mantissa"] == 4


def _brute_rne_code(y):
    """Nearest magnitude by exact rational distance; ties to the even index."""
    y = Fraction(y)
    if y >= 6:
        return 7
    best = None
    for i, m in enumerate(MAGS):
        d = abs(y - m)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def test_e2m1_rne_ties_and_saturation():
    assert O.e2m1_value(O.e2m1_rne(5.0)) == 4.0        # 5 is not representable; tie -> even code
    assert O.e2m1_value(O.e2m1_rne(4.9)) == 4.0
    assert O.e2m1_value(O.e2m1_rne(5.1)) == 6.0
    assert O.e2m1_value(O.e2m1_rne(0.25)) == 0.0       # tie 0 / 0.5 -> code 0
    assert O.e2m1_value(O.e2m1_rne(0.75)) == 1.0       # tie 0.5 / 1 -> code 2
    assert O.e2m1_value(O.e2m1_rne(2.5)) == 2.0        # tie 2 / 3 -> code 4
    assert O.e2m1_value(O.e2m1_rne(1e9)) == 6.0        # saturate
    for v in GOLD["e2m1_magnitudes"]["values"]:
        assert O.e2m1_value(O.e2m1_rne(v)) == v


def test_e2m1_rne_brute_force_dense_grid():
    grid = [i / 256 for i in range(0, 7 * 256)]
    rs = W.uniform((4000,), 0.0, 7.0, seed=11)
    for y in list(grid) + [float(v) for v in rs]:
        y32 = float(np.float32(y))
        assert O.e2m1_rne(y32) == _brute_rne_code(y32), y32


# ------------------------------------------------------------------ E4M3
def test_e4m3_decode_matches_torch_float8():
    b = torch.arange(0, 127, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([O.e4m3_value(i) for i in range(127)])
    assert np.array_equal(got, ref)
    assert O.e4m3_value(0x7E) == 448.0


def test_e4m3_encode_matches_torch_below_saturation():
    vals = [O.e4m3_value(i) for i in range(127)]
    mids = [(vals[i] + vals[i + 1]) / 2 for i in range(126)]          # exact ties
    near = [np.nextafter(np.float32(m), np.float32(0)) for m in mids] + \
           [np.nextafter(np.float32(m), np.float32(1e9)) for m in mids]
    rnd = np.exp(W.uniform((5000,), np.log(1e-4), np.log(463.0), seed=3)).astype(np.float32)
    xs = np.array(vals + mids + near + list(rnd) + [0.0, 2.0 ** -10, 2.0 ** -11],
                  dtype=np.float32)
    xs = xs[xs < 464.0]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_encode(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    for u in [448.0, 449.0, 463.99, 464.0, 465.0, 1e6, 3.0e38]:
        assert O.e4m3_encode(u) == 0x7E


# ------------------------------------------------------------------ Philox
@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand"):
        pytest.skip("rocRAND headers / hipcc not available for the Philox known-answer pin")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    subprocess.run([hipcc, "-O1", "-o", exe, os.path.join(HERE, "philox_rocrand_ref.cpp")],
                   check=True, capture_output=True)

    def run(triples):
        inp = "\n".join(f"{s} {q} {o}" for s, q, o in triples) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [list(map(int, line.split())) for line in out.strip().splitlines()]

    return run


def test_philox_matches_rocrand(rocrand_philox):
    r = W.rng(5)
    cases = []
    for _ in range(64):
        seed = int(r.integers(0, 2 ** 64, dtype=np.uint64))
        q = int(r.integers(0, 2 ** 62, dtype=np.uint64))
        sub = int(r.integers(0, 2 ** 32, dtype=np.uint64))
        cases.append((seed, sub, q))
    cases += [(0, 0, 0), (2 ** 64 - 1, 2 ** 32 - 1, 2 ** 62 - 1), (1, 3, 0)]
    ref = rocrand_philox([(s, sub, 4 * q) for s, sub, q in cases])
    for (seed, sub, q), words in zip(cases, ref):
        ctr = [q & 0xFFFFFFFF, q >> 32, sub & 0xFFFFFFFF, sub >> 32]
        key = [seed & 0xFFFFFFFF, seed >> 32]
        assert list(O.philox4x32_10(ctr, key)) == words


def test_draw16_and_sign_mask_mapping(rocrand_philox):
    r = W.rng(6)
    idx = [0, 1, 7, 8, 15, 16, 12345, 2 ** 33 + 5] + [int(v) for v in r.integers(0, 2 ** 40, 40)]
    for stream in (O.STREAM_ROW, O.STREAM_COL, O.STREAM_2D):
        seed = 0x1234_5678_9ABC_DEF0 + stream
        ref = rocrand_philox([(seed, stream, 4 * (i >> 3)) for i in idx])
        for i, words in zip(idx, ref):
            j = i & 7
            expect = (words[j >> 1] >> (16 * (j & 1))) & 0xFFFF
            assert O.draw16(seed, stream, i) == expect
    for seed in (0, 1, 99, 2 ** 63 + 7):
        words = rocrand_philox([(seed, O.STREAM_RHT, 0)])[0]
        assert O.rht_sign_mask(seed) == words[0] & 0xFFFF


# ------------------------------------------------------------------ SR
def test_sr_page_example_exact_probability():
    """2.25 becomes 2 in three cases of four and 3 in one."""
    g = GOLD["stochastic_rounding_example"]
    codes = np.array([O.e2m1_sr(g["value"], r) for r in range(65536)])
    vals = np.array([O.e2m1_value(c) for c in codes])
    assert set(vals) == {g["down"], g["up"]}
    assert np.mean(vals == g["up"]) == g["p_up"]
    assert np.mean(vals == g["down"]) == g["p_down"]
    assert np.mean(vals) == g["mean"]


def test_sr_exhaustive_counts_are_ceil_f():
    ys = list(W.uniform((300,), 0.0, 6.0, seed=8)) + [0.0, 0.1, 0.5, 1.9999999, 4.0, 5.999999]
    for y in ys:
        y = float(np.float32(y))
        yf = Fraction(y)
        lo = max(i for i, m in enumerate(MAGS) if m <= yf)
        f = (yf - MAGS[lo]) / (MAGS[lo + 1] - MAGS[lo])
        k = sum(O.e2m1_sr(y, r) == lo + 1 for r in range(0, 65536, 1))
        expect = -((-f * 65536) // 1)         # ceil(f * 2^16)
        assert k == expect, y
        # unbiased to within one draw's resolution
        mean = MAGS[lo] + Fraction(k, 65536) * (MAGS[lo + 1] - MAGS[lo])
        assert abs(mean - yf) <= (MAGS[lo + 1] - MAGS[lo]) / 65536


def test_sr_quantize_statistics_on_page_example():
    """Tensor-level check: blocks [48, 18, 18, ...] with s_t = 1 put 18 at
    y = 2.25 (block multiplier 8); about a quarter of them become 3*8."""
    rows, cols = 256, 256
    x = np.full((rows, cols), 18.0, dtype=np.float32)
    x[:, ::16] = 48.0
    q = O.quantize(x, O.F32, O.ROW_1D, O.SR, sr_seed=77, amax_in=2688.0)
    assert q.ts == 1.0
    assert np.all(q.scales == O.e4m3_encode(8.0))
    deq = O.dequantize(q)
    mask = np.ones_like(x, dtype=bool)
    mask[:, ::16] = False
    d = deq[mask]
    assert set(np.unique(d)) == {16.0, 24.0}
    n = d.size
    p = np.mean(d == 24.0)
    assert abs(p - 0.25) < 5 * np.sqrt(0.25 * 0.75 / n)
    assert abs(d.mean() - 18.0) < 5 * 8 * np.sqrt(0.25 * 0.75 / n)


# ------------------------------------------------------------------ page example -54
def test_minus54_one_level():
    """A block whose largest magnitude is -54 becomes -6 with multiplier 9
    (tensor scale 1: a second block holds the tensor maximum 6 * 448)."""
    g = GOLD["block_max_example"]
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :16] = W.uniform((16,), -5.0, 5.0, seed=1)
    x[0, 3] = g["block_max"]
    x[0, 16] = 2688.0
    q = O.quantize(x, O.F32, O.ROW_1D)
    assert q.ts == 1.0
    assert O.e4m3_value(int(q.scales[0, 0])) == g["multiplier"]
    code = (q.codes[0, 1] >> 4) & 0xF
    assert O.e2m1_value(code) == g["becomes"]
    assert O.dequantize(q)[0, 3] == g["block_max"]


def test_minus54_two_level():
    """Same example through both scale levels: one block, tensor maximum 54.
    The block multiplier S = e4m3(u) * s_t comes out as exactly 9."""
    g = GOLD["block_max_example"]
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, :] = W.uniform((16,), -5.0, 5.0, seed=2)
    x[0, 0] = g["block_max"]
    q = O.quantize(x, O.F32, O.ROW_1D)
    S = np.float32(O.e4m3_value(int(q.scales[0, 0]))) * np.float32(q.ts)
    assert float(S) == g["multiplier"]
    assert O.e2m1_value(q.codes[0, 0] & 0xF) == g["becomes"]
    assert O.dequantize(q)[0, 0] == g["block_max"]


# ------------------------------------------------------------------ scales
def test_tensor_scale_closed_form_and_max_block():
    x = W.student_t((64, 128), seed=4)
    q = O.quantize(x, O.F32, O.ROW_1D)
    amax = np.float32(np.abs(x).max())
    assert q.ts == float(np.float32(amax / np.float32(6 * 448)))
    r, c = np.unravel_index(np.abs(x).argmax(), x.shape)
    assert q.scales[r, c // 16] == 0x7E
    # every block's scale: its largest element lands on 6 or 4 (RNE of ~6*(1 +- 2^-4))
    deq = O.dequantize(q)
    blocks = np.abs(x).reshape(64, 8, 16).max(-1)
    dmax = np.abs(deq).reshape(64, 8, 16).max(-1)
    assert np.all(np.abs(dmax - blocks) <= blocks * (1 / 16 + 1e-6) + 1e-30)


def test_zero_tensor():
    x = np.zeros((16, 32), dtype=np.float32)
    x[3, 5] = -0.0
    for layout in (O.ROW_1D, O.COL_1D, O.BLK_2D):
        q = O.quantize(x, O.F32, layout)
        assert q.ts == 1.0
        assert np.all(q.scales == 0)
        assert np.all((q.codes & 0x77) == 0)      # magnitudes 0, sign copied
    q = O.quantize(x, O.F32, O.ROW_1D)
    assert (q.codes[3, 2] >> 4) == 0x8


def test_bits_per_element():
    x = W.student_t((128, 256), seed=5)
    q = O.quantize(x, O.F32, O.ROW_1D)
    nbits = 8 * (q.codes.nbytes + q.scales.nbytes)
    assert nbits == 4.5 * x.size
    assert round(16 / 4.5, 1) == GOLD["bits_vs_bf16"]["ratio"]


# ------------------------------------------------------------------ RNE error bound / values
def test_rne_is_nearest_grid_point():
    x = W.with_spikes(W.student_t((96, 160), seed=6), 0.01, 50.0, seed=7)
    q = O.quantize(x, O.F32, O.ROW_1D)
    st = np.float32(q.ts)
    for r in range(0, 96, 7):
        for b in range(160 // 16):
            S = np.float32(np.float32(O.e4m3_value(int(q.scales[r, b]))) * st)
            grid = [Fraction(float(S)) * m for m in MAGS]
            for c in range(16 * b, 16 * b + 16):
                code = (q.codes[r, c // 2] >> (4 * (c & 1))) & 0xF
                v = Fraction(float(S)) * MAGS[code & 7]
                t = Fraction(float(abs(x[r, c])))
                # no other grid point is strictly closer (ties allowed)
                assert all(abs(t - v) <= abs(t - gp) + Fraction(float(S)) * Fraction(1, 2 ** 20)
                           for gp in grid if gp <= 6 * Fraction(float(S))) or code & 7 == 7


def test_every_code_decodes_into_value_set():
    x = W.with_spikes(W.student_t((64, 64), seed=9), 0.001, 50.0, seed=10)
    allowed = set(float(v) for v in GOLD["e2m1_magnitudes"]["values"])
    for layout in (O.ROW_1D, O.COL_1D, O.BLK_2D):
        for rnd in (O.RNE, O.SR):
            q = O.quantize(x, O.F32, layout, rnd, sr_seed=3)
            lo = q.codes & 0xF
            hi = q.codes >> 4
            for c in np.unique(np.concatenate([lo.ravel(), hi.ravel()])):
                assert abs(O.e2m1_value(int(c))) in allowed


# ------------------------------------------------------------------ invariants
def test_idempotence_rne():
    x = W.with_spikes(W.student_t((64, 192), seed=12), 0.001, 50.0, seed=13)
    for layout in (O.ROW_1D, O.COL_1D, O.BLK_2D):
        q = O.quantize(x, O.F32, layout)
        amax = np.float32(np.abs(x).max())
        deq = O.dequantize(q)
        x2 = deq.T.copy() if layout == O.COL_1D else deq
        q2 = O.quantize(x2, O.F32, layout, amax_in=float(amax))
        assert np.array_equal(q2.codes, q.codes)
        assert np.array_equal(q2.scales, q.scales)
        assert q2.ts == q.ts
        q3 = O.quantize(x2, O.F32, layout)          # own amax: s_t within one ulp
        assert abs(q3.ts - q.ts) <= float(np.spacing(np.float32(q.ts)))


def test_col_is_row_of_transpose_and_row_col_fused():
    x = W.student_t((48, 80), seed=14)
    b = W.f32_to_bf16_bits(x)
    qc = O.quantize(b, O.BF16, O.COL_1D)
    qr_t = O.quantize(b.T.copy(), O.BF16, O.ROW_1D)
    assert np.array_equal(qc.codes, qr_t.codes) and np.array_equal(qc.scales, qr_t.scales)
    assert qc.ts == qr_t.ts
    for rnd in (O.RNE, O.SR):
        row, col = O.quantize(b, O.BF16, O.ROW_COL_1D, rnd, sr_seed=21)
        r1 = O.quantize(b, O.BF16, O.ROW_1D, rnd, sr_seed=21)
        c1 = O.quantize(b, O.BF16, O.COL_1D, rnd, sr_seed=21)
        assert np.array_equal(row.codes, r1.codes) and np.array_equal(col.codes, c1.codes)
        assert np.array_equal(row.scales, r1.scales) and np.array_equal(col.scales, c1.scales)


def test_2d_scale_transpose_invariance():
    """One multiplier per 16x16 square does not change under the flip."""
    x = W.normal((64, 96), 0.02, seed=15)
    q = O.quantize(x, O.F32, O.BLK_2D)
    qt = O.quantize(x.T.copy(), O.F32, O.BLK_2D)
    assert np.array_equal(qt.scales, q.scales.T)
    assert np.array_equal(O.dequantize(qt), O.dequantize(q).T)


def test_2d_outlier_zeroes_its_square_but_1d_only_its_block():
    x = W.uniform((32, 32), -1.0, 1.0, seed=16)
    x[5, 9] = 1000.0
    q2 = O.quantize(x, O.F32, O.BLK_2D)
    d2 = O.dequantize(q2)
    sq = d2[:16, :16].copy()
    assert sq[5, 9] == 1000.0 or abs(sq[5, 9] - 1000.0) / 1000.0 < 0.2
    sq[5, 9] = 0.0
    assert np.all(sq == 0.0)                         # the other 255 round to (signed) zero
    assert np.count_nonzero(d2[16:, 16:]) > 0        # other squares unaffected
    q1 = O.quantize(x, O.F32, O.ROW_1D)
    d1 = O.dequantize(q1)
    blk = d1[5, :16].copy()
    blk[9] = 0.0
    assert np.all(blk == 0.0)
    assert np.count_nonzero(d1[6, :16]) > 0 and np.count_nonzero(d1[4, :16]) > 0


# ------------------------------------------------------------------ Hadamard
def test_rht_plain_signs_is_textbook_walsh_hadamard():
    H = scipy.linalg.hadamard(16).astype(np.float64)
    for seed in range(5):
        x = W.normal((16,), 1.0, seed=100 + seed)
        t = O.rht16(x, 0)
        ref = H @ x.astype(np.float64) / 4.0
        assert np.allclose(t, ref, rtol=0, atol=1e-6 * np.abs(x).sum())


def test_rht_signs_inverse_parseval_dot():
    H = scipy.linalg.hadamard(16).astype(np.float64)
    mask = O.rht_sign_mask(1234)
    d = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])
    a = W.normal((16,), 1.0, seed=200)
    b = W.normal((16,), 1.0, seed=201)
    ta, tb = O.rht16(a, mask), O.rht16(b, mask)
    assert np.allclose(ta, H @ (d * a) / 4.0, atol=1e-6 * np.abs(a).sum())
    back = d * (H @ ta.astype(np.float64)) / 4.0
    assert np.allclose(back, a, atol=1e-6 * np.abs(a).sum())
    assert np.isclose(np.dot(ta, ta), np.dot(a, a), rtol=1e-5)
    assert np.isclose(np.dot(ta.astype(np.float64), tb), np.dot(a.astype(np.float64), b),
                      rtol=0, atol=1e-5 * np.abs(a).sum() * np.abs(b).sum() / 16)


def test_rht_applied_along_block_dim_before_quantize():
    x = W.normal((32, 64), 1.0, seed=17)
    mask = O.rht_sign_mask(55)
    H = scipy.linalg.hadamard(16).astype(np.float64)
    d = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])
    # COL layout: chunks of 16 consecutive rows; compare the dequantized
    # result against the fp64 transform of x^T within quantization error.
    q = O.quantize(x, O.F32, O.COL_1D, hadamard=True, hadamard_seed=55)
    t_ref = np.zeros((64, 32))
    for c in range(64):
        for r0 in range(0, 32, 16):
            t_ref[c, r0:r0 + 16] = H @ (d * x[r0:r0 + 16, c]) / 4.0
    amax = np.float32(np.abs(t_ref).max())
    assert abs(q.ts - amax / 2688) <= 1e-6 * amax / 2688
    deq = O.dequantize_f64(q)
    blk = np.abs(t_ref).reshape(64, 2, 16).max(-1, keepdims=True)
    assert np.all(np.abs(deq.reshape(64, 2, 16) - t_ref.reshape(64, 2, 16)) <= blk * (1 / 6 + 1 / 8))


# ------------------------------------------------------------------ dequantize / GEMM
def test_dequantize_bf16_matches_torch_rounding():
    x = W.student_t((32, 64), seed=18)
    q = O.quantize(x, O.F32, O.ROW_1D)
    f = O.dequantize(q, O.F32)
    b = O.dequantize(q, O.BF16)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def _exact_deq(q):
    """Rational dequantization from the page's value set and torch's E4M3."""
    sc = torch.from_numpy(q.scales.copy()).view(torch.float8_e4m3fn).double().numpy()
    ts = Fraction(float(np.float32(q.ts)))
    out = [[None] * q.cols for _ in range(q.rows)]
    for r in range(q.rows):
        for c in range(q.cols):
            code = (int(q.codes[r, c // 2]) >> (4 * (c & 1))) & 0xF
            v = MAGS[code & 7] * (-1 if code & 8 else 1)
            s = sc[r // 16, c // 16] if q.scale_mode == O.SCALE_2D else sc[r, c // 16]
            out[r][c] = v * Fraction(float(s)) * ts
    return out


@pytest.mark.parametrize("layout", [O.ROW_1D, O.BLK_2D])
def test_dequantize_f64_and_f32_equal_rational_value(layout):
    """The float64 dequantization is the exact value code x multiplier x s_t
    (at most 30 significant bits, so float64 holds it), and the binary32 one
    is that exact value rounded once; both checked element by element
    against rational arithmetic on the page's value set and torch's E4M3."""
    x = W.with_spikes(W.student_t((32, 64), 3.0, seed=60), 0.05, 300.0, seed=61)
    x[3, :16] = 0.0                      # an all-zero block: multiplier byte 0
    x[5, 16:32] *= 1e-6                  # a block with a subnormal-range multiplier
    q = O.quantize(x, O.F32, layout, O.SR, sr_seed=62)
    exact = _exact_deq(q)
    d64 = O.dequantize_f64(q)
    d32 = O.dequantize(q, O.F32)
    for r in range(q.rows):
        for c in range(q.cols):
            assert Fraction(float(d64[r, c])) == exact[r][c], (r, c)
            assert d32[r, c] == np.float32(float(exact[r][c])), (r, c)
    assert len({float(v) for row in exact for v in row}) > 40   # many distinct values were checked


@pytest.mark.parametrize("modes", [(O.ROW_1D, O.ROW_1D), (O.ROW_1D, O.BLK_2D), (O.COL_1D, O.COL_1D)])
def test_gemm_brute_force_tiny(modes):
    M, N, K = 16, 16, 48
    xa = W.with_spikes(W.normal((M, K) if modes[0] != O.COL_1D else (K, M), seed=19), 0.02, 50, seed=20)
    xb = W.normal((N, K) if modes[1] != O.COL_1D else (K, N), seed=21)
    A = O.quantize(xa, O.F32, modes[0])
    B = O.quantize(xb, O.F32, modes[1])
    C, Wt = O.gemm(A, B)
    ea, eb = _exact_deq(A), _exact_deq(B)
    for m in range(M):
        for n in range(N):
            exact = sum(ea[m][k] * eb[n][k] for k in range(K))
            wabs = sum(abs(ea[m][k] * eb[n][k]) for k in range(K))
            assert abs(Fraction(C[m, n]) - exact) <= wabs * Fraction(1, 2 ** 50)
            assert abs(Fraction(Wt[m, n]) - wabs) <= wabs * Fraction(1, 2 ** 50)
    # sampled entries agree with the full result
    mi, ni = np.array([0, 3, 15]), np.array([2, 15, 0])
    Ce, We = O.gemm(A, B, entries=(mi, ni))
    assert np.array_equal(Ce, C[mi, ni]) and np.array_equal(We, Wt[mi, ni])


def test_gemm_exact_with_unit_scales():
    """Blocks whose largest magnitude is 6 in a tensor whose maximum is 2688
    (s_t = 1): every block scale is 1 and the products are multiples of 1/4,
    so the float64 result is exact and equals an integer matmul."""
    M, N, K = 32, 24, 64
    r = W.rng(22)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)

    def make(rows):
        x = grid[r.integers(0, 8, size=(rows, K))] * np.where(r.random((rows, K)) < 0.5, -1, 1)
        x = x.astype(np.float32)
        x[:, ::16] = 6.0
        return x

    a, b = make(M), make(N)
    A = O.quantize(a, O.F32, O.ROW_1D, amax_in=2688.0)
    B = O.quantize(b, O.F32, O.ROW_1D, amax_in=2688.0)
    assert A.ts == 1.0 and np.all(A.scales == 0x38) and np.all(B.scales == 0x38)
    C, _ = O.gemm(A, B)
    ref = (np.rint(a * 2).astype(np.int64) @ np.rint(b * 2).astype(np.int64).T) / 4.0
    assert np.array_equal(C, ref)


def test_grouped_gemm_is_per_group_gemm():
    K, N = 64, 32
    counts = [5, 0, 17, 10]
    offs = np.concatenate([[0], np.cumsum(counts)])
    a = W.normal((int(offs[-1]), K), seed=23)
    A = O.quantize(a, O.F32, O.ROW_1D)
    Bs = [O.quantize(W.normal((N, K), 0.02, seed=30 + g), O.F32, O.BLK_2D) for g in range(4)]
    C, _ = O.grouped_gemm(A, offs, Bs)
    deqA = O.dequantize_f64(A)
    for g in range(4):
        r0, r1 = offs[g], offs[g + 1]
        ref = deqA[r0:r1] @ O.dequantize_f64(Bs[g]).T
        assert np.allclose(C[r0:r1], ref, rtol=1e-12, atol=1e-12)
    mi = np.array([0, 4, 5, 21, 31])
    ni = np.array([1, 2, 3, 4, 31])
    Ce, _ = O.grouped_gemm(A, offs, Bs, entries=(mi, ni))
    assert np.array_equal(Ce, C[mi, ni])


def test_swiglu_closed_forms():
    from scipy.special import expit
    g = np.array([-8.0, -1.0, 0.0, 0.5, 3.0, 20.0])
    u = np.array([1.0, 2.0, 5.0, -1.0, 0.25, 1.0])
    ref = g * expit(g) * u
    assert np.allclose(O.swiglu(g, u), ref, rtol=1e-14, atol=0)
    assert O.swiglu(0.0, 7.0) == 0.0


@pytest.mark.parametrize("rnd", [O.RNE, O.SR])
def test_requantize_of_grid_exact_tensor_is_the_transpose(rnd):
    """Re-quantization along columns (iitak.ru page, "Как это работает"):
    for a tensor whose values lie on the E2M1 grid and in which every
    16-element row block and column block holds a +-6, with A_t = 2688 the
    multipliers are all 1 (byte 0x38) and every value is exact, so the row
    quantization stores x exactly, its dequantization gives x back, and the
    column re-quantization must store x transposed: its code nibbles are the
    transpose of the row codes' nibbles.  Stochastic rounding has fraction 0
    everywhere and must agree."""
    rng = np.random.default_rng(7)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    rows, cols = 48, 64
    x = grid[rng.integers(0, 8, size=(rows, cols))] * np.where(rng.random((rows, cols)) < 0.5, -1, 1)
    x = x.astype(np.float32)
    for i in range(rows):                      # a +-6 in every row block and every column block
        for b in range(cols // 16):
            x[i, 16 * b + (i + 5 * b) % 16] = 6.0 if (i + b) % 2 else -6.0
    q = O.quantize(x, O.F32, O.ROW_1D, O.RNE, amax_in=2688.0)
    assert np.all(q.scales == 0x38)
    assert np.array_equal(O.dequantize(q, O.F32), x)
    r = O.requantize(q, rnd, sr_seed=3, amax_in=2688.0)
    assert (r.rows, r.cols) == (cols, rows)
    assert np.all(r.scales == 0x38)

    def nibbles(c):
        n = np.empty((c.shape[0], 2 * c.shape[1]), dtype=np.uint8)
        n[:, 0::2], n[:, 1::2] = c & 15, c >> 4
        return n

    assert np.array_equal(nibbles(r.codes), nibbles(q.codes).T)



def test_rowcol_hadamard_is_row_and_col_of_their_own_transforms():
    """ROW_COL_1D with the Hadamard transform: the row output is ROW_1D of x
    transformed along rows, the column output COL_1D of x transformed along
    columns (both pinned above against scipy's Sylvester matrix), each with
    the A_t of its own transformed tensor; a given pair of A_t is used as
    (row output, column output)."""
    x = W.f32_to_bf16_bits(W.with_spikes(W.student_t((64, 96), 3.0, seed=70), 0.01, 80.0, seed=71))
    for rnd in (O.RNE, O.SR):
        r, c = O.quantize(x, O.BF16, O.ROW_COL_1D, rnd, sr_seed=5, hadamard=True, hadamard_seed=9)
        r1 = O.quantize(x, O.BF16, O.ROW_1D, rnd, sr_seed=5, hadamard=True, hadamard_seed=9)
        c1 = O.quantize(x, O.BF16, O.COL_1D, rnd, sr_seed=5, hadamard=True, hadamard_seed=9)
        for a, b in ((r, r1), (c, c1)):
            assert a.ts == b.ts and np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales)
        assert r.ts == O.tensor_scale(O.amax(x, O.BF16, O.ROW_1D, True, 9))
        assert c.ts == O.tensor_scale(O.amax(x, O.BF16, O.COL_1D, True, 9))
        assert r.ts != c.ts
        r2, c2 = O.quantize(x, O.BF16, O.ROW_COL_1D, rnd, sr_seed=5, hadamard=True, hadamard_seed=9,
                            amax_in=(100.0, 200.0))
        assert r2.ts == O.tensor_scale(100.0) and c2.ts == O.tensor_scale(200.0)
