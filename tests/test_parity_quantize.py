"""GPU parity of quantize / dequantize against the CPU oracle: codes, scale
bytes, tensor scales and stochastic-rounding outputs must match bit for bit;
dequantized values must equal the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_utils import assert_q_equal, bf16_tensor_to_bits, q_to_device, q_to_host, require_gpu, to_device

pytestmark = pytest.mark.gpu

LAYOUT_NAMES = {0: "row", 1: "col", 2: "rowcol", 3: "2d"}


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def make_input(rows, cols, dtype, seed, kind="t3"):
    if kind == "t3":
        x = W.student_t((rows, cols), 3.0, seed=seed)
    elif kind == "spiky":
        x = W.with_spikes(W.normal((rows, cols), 1.0, seed=seed), 1e-3, 100.0, seed=seed + 1)
    elif kind == "w":
        x = W.normal((rows, cols), 0.02, seed=seed)
    else:
        raise ValueError(kind)
    if dtype == O.BF16:
        return W.f32_to_bf16_bits(x)
    return x


def run_both(nv, x, dtype, layout, rnd, seed=7, had=False, hseed=0, amax_in=None, pad=None):
    xd = to_device(x, pad)
    amax_d = None if amax_in is None else torch.tensor([amax_in], dtype=torch.float32, device="cuda")
    got = nv.nvfp4_quantize(xd, layout=layout, round=rnd, sr_seed=seed, hadamard=had,
                            hadamard_seed=hseed, amax_in=amax_d)
    ref = O.quantize(x, dtype, layout, rnd, sr_seed=seed, hadamard=had, hadamard_seed=hseed,
                     amax_in=amax_in)
    if layout == O.ROW_COL_1D:
        return [q_to_host(g) for g in got], list(ref)
    return [q_to_host(got)], [ref]


SHAPES_ROW = [(1, 16), (7, 48), (64, 64), (100, 1040), (333, 2064)]
SHAPES_COL = [(16, 1), (48, 7), (64, 64), (96, 37), (208, 1031), (1040, 100)]
SHAPES_BOTH = [(16, 16), (48, 80), (64, 64), (208, 1040), (1024, 96)]


@pytest.mark.parametrize("dtype", [O.BF16, O.F32])
@pytest.mark.parametrize("rnd", [O.RNE, O.SR])
@pytest.mark.parametrize("had", [False, True])
@pytest.mark.parametrize("shape", SHAPES_ROW)
def test_row(nv, dtype, rnd, had, shape):
    x = make_input(*shape, dtype, seed=shape[0] * 7 + shape[1])
    got, ref = run_both(nv, x, dtype, O.ROW_1D, rnd, seed=99, had=had, hseed=1234)
    assert_q_equal(got[0], ref[0], f"row {shape}")


@pytest.mark.parametrize("dtype", [O.BF16, O.F32])
@pytest.mark.parametrize("rnd", [O.RNE, O.SR])
@pytest.mark.parametrize("had", [False, True])
@pytest.mark.parametrize("shape", SHAPES_COL)
def test_col(nv, dtype, rnd, had, shape):
    x = make_input(*shape, dtype, seed=shape[0] * 5 + shape[1], kind="spiky")
    pad = (shape[1] + 7) // 8 * 8 if dtype == O.BF16 else (shape[1] + 3) // 4 * 4
    got, ref = run_both(nv, x, dtype, O.COL_1D, rnd, seed=5, had=had, hseed=77, pad=pad)
    assert_q_equal(got[0], ref[0], f"col {shape}")


@pytest.mark.parametrize("dtype", [O.BF16, O.F32])
@pytest.mark.parametrize("rnd", [O.RNE, O.SR])
@pytest.mark.parametrize("shape", SHAPES_BOTH)
def test_rowcol_and_2d(nv, dtype, rnd, shape):
    x = make_input(*shape, dtype, seed=shape[0] + shape[1] * 3)
    got, ref = run_both(nv, x, dtype, O.ROW_COL_1D, rnd, seed=11)
    assert_q_equal(got[0], ref[0], f"rowcol/row {shape}")
    assert_q_equal(got[1], ref[1], f"rowcol/col {shape}")
    got, ref = run_both(nv, x, dtype, O.BLK_2D, rnd, seed=12)
    assert_q_equal(got[0], ref[0], f"2d {shape}")


@pytest.mark.parametrize("dtype", [O.BF16, O.F32])
@pytest.mark.parametrize("rnd", [O.RNE, O.SR])
@pytest.mark.parametrize("shape", [(16, 16), (48, 80), (208, 1040), (1040, 96)])
def test_rowcol_hadamard(nv, dtype, rnd, shape):
    """ROW_COL_1D with the Hadamard transform: the row output quantizes x
    transformed along rows, the column output x transformed down columns,
    each with its own A_t (computed, then given as a pair and published
    through amax_out as a pair)."""
    x = make_input(*shape, dtype, seed=shape[0] * 3 + shape[1], kind="spiky")
    got, ref = run_both(nv, x, dtype, O.ROW_COL_1D, rnd, seed=13, had=True, hseed=321)
    assert_q_equal(got[0], ref[0], f"rowcol+had/row {shape}")
    assert_q_equal(got[1], ref[1], f"rowcol+had/col {shape}")
    assert got[0].ts != got[1].ts or shape == (16, 16)
    pair = torch.tensor([3.5, 700.0], dtype=torch.float32, device="cuda")
    out_pair = torch.zeros(2, dtype=torch.float32, device="cuda")
    gr, gc = nv.nvfp4_quantize(to_device(x), layout=nv.NVFP4_ROW_COL_1D, round=rnd, sr_seed=13,
                               hadamard=True, hadamard_seed=321, amax_in=pair, amax_out=out_pair)
    rr, rc = O.quantize(x, dtype, O.ROW_COL_1D, rnd, sr_seed=13, hadamard=True, hadamard_seed=321,
                        amax_in=(3.5, 700.0))
    assert_q_equal(q_to_host(gr), rr, f"rowcol+had given pair/row {shape}")
    assert_q_equal(q_to_host(gc), rc, f"rowcol+had given pair/col {shape}")
    assert out_pair.cpu().tolist() == [3.5, 700.0]


@pytest.mark.parametrize("rnd", [O.RNE, O.SR])
def test_col_hadamard_bf16_multiplier_ranges(nv, rnd):
    """BF16 columns with the Hadamard transform: the kernel folds the
    transform's 1/4 into the block multiplier R where that is exact (and with
    SR takes a single multiply when R >= 2^-14), and otherwise forms t = h / 4
    first.  The inputs put whole waves on each side and mix them: columns of
    ordinary magnitude (R near 1), columns scaled by 2^20 (R below 2^-14), the
    two interleaved, a column block of the smallest BF16 subnormals (R = 0 or
    large), each with the transformed amax computed, given, given 2^40 times
    too large, and given far too small (the saturating path)."""
    base = W.with_spikes(W.normal((208, 96), 1.0, seed=41), 1e-3, 100.0, seed=42)
    big = base * np.float32(2.0 ** 20)
    mixed = base.copy()
    mixed[:, 1::2] *= np.float32(2.0 ** 20)
    for name, xf in (("ordinary", base), ("scaled", big), ("mixed", mixed)):
        x = W.f32_to_bf16_bits(xf)
        x[:16, 5] = np.where(np.arange(16) % 3 == 0, 0x8001, 0x0001).astype(x.dtype)
        true_t = O.amax(x, O.BF16, O.COL_1D, True, 91)
        for amax_in in (None, true_t, true_t * 2.0 ** 40, 1e-30):
            got, ref = run_both(nv, x, O.BF16, O.COL_1D, rnd, seed=43, had=True, hseed=91, amax_in=amax_in, pad=96)
            assert_q_equal(got[0], ref[0], f"col+had {name} amax_in={amax_in}")


@pytest.mark.parametrize("dtype", [O.BF16, O.F32])
@pytest.mark.parametrize("layout,rnd", [(O.COL_1D, O.RNE), (O.COL_1D, O.SR), (O.ROW_COL_1D, O.RNE),
                                        (O.ROW_COL_1D, O.SR)])
def test_col_tiles_xcd_remap_with_partial_block(nv, dtype, layout, rnd):
    """2288 x 2048: a 32 x 9 grid of 256-row column tiles for bf16 (64 x 9 for
    fp32), so whole blocks of 8 x 32 (8 x 64) dispatched workgroups take
    remapped tiles while the last, partial block keeps the dispatch order;
    the last tile row is partial (240 rows)."""
    x = make_input(2288, 2048, dtype, seed=77)
    got, ref = run_both(nv, x, dtype, layout, rnd, seed=78)
    for i, (g, r) in enumerate(zip(got, ref)):
        assert_q_equal(g, r, f"remap {layout}/{rnd}/{i}")


def test_fused_rowcol_equals_separate_calls(nv):
    x = make_input(128, 192, O.BF16, seed=3)
    xd = to_device(x)
    r, c = nv.nvfp4_quantize(xd, layout=nv.NVFP4_ROW_COL_1D, round=nv.NVFP4_SR, sr_seed=4)
    r1 = nv.nvfp4_quantize(xd, layout=nv.NVFP4_ROW_1D, round=nv.NVFP4_SR, sr_seed=4)
    c1 = nv.nvfp4_quantize(xd, layout=nv.NVFP4_COL_1D, round=nv.NVFP4_SR, sr_seed=4)
    assert_q_equal(q_to_host(r), q_to_host(r1), "fused row")
    assert_q_equal(q_to_host(c), q_to_host(c1), "fused col")


@pytest.mark.parametrize("layout", [O.ROW_1D, O.COL_1D, O.BLK_2D])
def test_edge_values(nv, layout):
    """Zeros, signed zeros, one huge outlier, tiny (subnormal-scale) blocks,
    exact ties of the E2M1 grid, and a given amax."""
    x = W.student_t((64, 64), 3.0, seed=1)
    x[0:16, 0:16] = 0.0
    x[3, 5] = -0.0
    x[20, 20] = 3.0e5
    x[32:48, 16:32] *= 1e-7
    x[48, 0:16] = np.array([6, 5, 3.5, 2.5, 1.75, 1.25, .75, .25, -6, -5, -3.5, -2.5, -1.75, -1.25,
                            -.75, -.25], dtype=np.float32)
    for rnd in (O.RNE, O.SR):
        for dt in (O.F32, O.BF16):
            xx = x if dt == O.F32 else W.f32_to_bf16_bits(x)
            got, ref = run_both(nv, xx, dt, layout, rnd, seed=21)
            assert_q_equal(got[0], ref[0], f"edge {layout} {rnd} {dt}")
            got, ref = run_both(nv, xx, dt, layout, rnd, seed=21, amax_in=2688.0)
            assert_q_equal(got[0], ref[0], f"edge amax_in {layout} {rnd} {dt}")


@pytest.mark.parametrize("layout", [O.ROW_1D, O.COL_1D, O.ROW_COL_1D, O.BLK_2D])
def test_understated_amax(nv, layout):
    """A caller-supplied A_t below the true amax: block multipliers clamp at
    448, scaled magnitudes run past 6 (to ~1e33 for A_t = 1e-30) and R
    overflows to inf once s_t is subnormal (A_t = 1e-39); every such element
    saturates, on both sides, under both roundings."""
    x = W.student_t((96, 80), 3.0, seed=5)
    true_amax = float(np.abs(x).max())
    for amax_in in (0.5 * true_amax, 1e-2 * true_amax, 1e-30, 1e-39):
        for rnd in (O.RNE, O.SR):
            for dt in (O.F32, O.BF16):
                xx = x if dt == O.F32 else W.f32_to_bf16_bits(x)
                got, ref = run_both(nv, xx, dt, layout, rnd, seed=31, amax_in=amax_in)
                for i in range(len(ref)):
                    assert_q_equal(got[i], ref[i], f"amax_in={amax_in} {layout}/{i} {rnd} {dt}")


@pytest.mark.parametrize("layout", [O.ROW_1D, O.COL_1D, O.ROW_COL_1D, O.BLK_2D])
def test_sr_large_blocks_with_smallest_subnormals(nv, layout):
    """BF16 stochastic rounding with blocks whose multiplier R is below 2^-17:
    in every other 16x16 square the diagonal holds 1e6 (the tensor amax) and
    the rest the smallest BF16 subnormal 2^-133, so each row, column and 2D
    block of the square mixes the two.  There |t|*R < 2^-150 rounds to 0 and
    the code must be 0 under every draw; computing the scaled value as
    |t|*(R*2^23) instead would round up on a zero draw.  The other squares
    hold ordinary values, so waves mix both kinds of block.  The test first
    counts, with the oracle's own draws, the subnormal elements whose draw is
    0 (at least one per layout), so the case is really exercised."""
    n = 1024
    x = W.normal((n, n), 1.0, seed=4242)
    tiny = np.float32(2.0 ** -133)
    mask = np.zeros((n, n), dtype=bool)
    for bi in range(n // 16):
        for bj in range(n // 16):
            if (bi + bj) % 2:
                continue
            sq = x[16 * bi:16 * bi + 16, 16 * bj:16 * bj + 16]
            sq[:] = tiny
            np.fill_diagonal(sq, 1.0e6)
            m = mask[16 * bi:16 * bi + 16, 16 * bj:16 * bj + 16]
            m[:] = True
            np.fill_diagonal(m, False)
    xb = W.f32_to_bf16_bits(x)
    assert np.all(xb[mask] == 0x0001)
    seed = 61
    rr, cc = np.nonzero(mask)
    # output index and random stream of each layout: row blocks 0, column blocks 1, squares 2
    spec = {O.ROW_1D: [(0, rr * n + cc)], O.COL_1D: [(1, cc * n + rr)],
            O.ROW_COL_1D: [(0, rr * n + cc), (1, cc * n + rr)], O.BLK_2D: [(2, rr * n + cc)]}[layout]
    for stream, idx in spec:
        zero_draws = sum(1 for i in idx.tolist() if O.draw16(seed, stream, i) == 0)
        assert zero_draws >= 1, f"stream {stream}: no subnormal element draws 0"
    got, ref = run_both(nv, xb, O.BF16, layout, O.SR, seed=seed)
    for i in range(len(ref)):
        assert_q_equal(got[i], ref[i], f"large blocks {layout}/{i}")


def test_zero_and_empty_tensors(nv):
    x = np.zeros((32, 32), dtype=np.float32)
    got, ref = run_both(nv, x, O.F32, O.ROW_1D, O.SR)
    assert_q_equal(got[0], ref[0], "zeros")
    e = torch.zeros((0, 32), dtype=torch.bfloat16, device="cuda")
    q = nv.nvfp4_quantize(e)
    torch.cuda.synchronize()
    assert q.tensor_scale.item() == 1.0


@pytest.mark.parametrize("layout", [O.ROW_1D, O.COL_1D, O.BLK_2D])
@pytest.mark.parametrize("out_dt", [O.F32, O.BF16])
def test_dequantize(nv, layout, out_dt):
    x = make_input(96, 160, O.BF16, seed=8, kind="spiky")
    ref_q = O.quantize(x, O.BF16, layout)
    qd = q_to_device(ref_q, nv)
    y = nv.nvfp4_dequantize(qd, dtype=torch.bfloat16 if out_dt == O.BF16 else torch.float32)
    ref = O.dequantize(ref_q, out_dt)
    got = bf16_tensor_to_bits(y) if out_dt == O.BF16 else y.cpu().numpy()
    assert np.array_equal(got.view(np.uint32 if out_dt == O.F32 else np.uint16),
                          ref.view(np.uint32 if out_dt == O.F32 else np.uint16))


@pytest.mark.parametrize("had", [False, True])
def test_amax_out_chaining(nv, had):
    """amax_out publishes the A_t a call used; passing it as amax_in to the
    next call on the same tensor gives the same result as computing it."""
    x = make_input(256, 320, O.BF16, seed=41, kind="spiky")
    xd = to_device(x)
    lay = nv.NVFP4_COL_1D if had else nv.NVFP4_ROW_1D
    a = torch.zeros(1, dtype=torch.float32, device="cuda")
    q1 = nv.nvfp4_quantize(xd, layout=lay, round=nv.NVFP4_SR, sr_seed=3, hadamard=had,
                           hadamard_seed=9, amax_out=a)
    torch.cuda.synchronize()
    assert a.item() == O.amax(x, O.BF16, lay, hadamard=had, hadamard_seed=9)
    q2 = nv.nvfp4_quantize(xd, layout=lay, round=nv.NVFP4_SR, sr_seed=3, hadamard=had,
                           hadamard_seed=9, amax_in=a)
    assert_q_equal(q_to_host(q2), q_to_host(q1), "chained")
    if not had:
        r, c = nv.nvfp4_quantize(xd, layout=nv.NVFP4_ROW_COL_1D, amax_in=a)
        ref_r, ref_c = O.quantize(x, O.BF16, O.ROW_COL_1D)
        assert_q_equal(q_to_host(r), ref_r, "chained rowcol row")
        assert_q_equal(q_to_host(c), ref_c, "chained rowcol col")


def test_gpu_idempotence(nv):
    x = make_input(128, 256, O.F32, seed=31)
    xd = to_device(x)
    q = nv.nvfp4_quantize(xd)
    y = nv.nvfp4_dequantize(q, dtype=torch.float32)
    amax = torch.tensor([float(np.abs(x).max())], device="cuda")
    q2 = nv.nvfp4_quantize(y, amax_in=amax)
    assert_q_equal(q_to_host(q2), q_to_host(q), "idempotence")
