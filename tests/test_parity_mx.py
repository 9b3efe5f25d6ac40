"""GPU parity of the MX (OCP Microscaling) quantize and dequantize kernels
against the oracle: E8M0 scale bytes and E4M3 / E2M1 codes bit for bit, for
both block directions, both roundings and both input types; dequantized
values bit for bit.  MXFP8 and MXFP4 are named on "Thinking Machines ускорила
обучение Inkling 2 Small 4-битными числами" (iitak.ru, sections "Как это
работает" and "Но") and "Nvidia добивается успеха с 4-битным форматом NVFP4"
(asector.ru, "Перспективы и дальнейшие направления исследований"); the
format details are the
OCP reading both sides implement."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_utils import bf16_tensor_to_bits, require_gpu, to_device

pytestmark = pytest.mark.gpu

ELEMS = [O.MX_FP8, O.MX_FP4]


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def edge_input(shape, seed):
    """Student-t(3) data with 32 x 32 tiles overwritten by the cases the
    format treats specially: all zeros, negative zeros, binary32 subnormals,
    magnitudes near the binary32 maximum, tiny normals, one huge value among
    tiny ones (the rest underflow to signed zero codes), and block maxima just
    below a power of two (scaled values in (448, 512) or (6, 8) saturate)."""
    x = W.student_t(shape, 3.0, seed=seed)
    g = W.rng(seed + 1)
    R, C = shape
    tiles = [(i, j) for i in range(0, R - 31, 32) for j in range(0, C - 31, 32)]
    for n, (i, j) in enumerate(tiles[1::3]):
        k = n % 8
        t = x[i:i + 32, j:j + 32]
        sgn = np.where(g.random((32, 32)) < 0.5, -1.0, 1.0).astype(np.float32)
        if k == 0:
            t[:] = 0.0
        elif k == 1:
            t[:] = -0.0
            t[::3, ::5] = 0.0
        elif k == 2:
            t[:] = sgn * g.uniform(1e-44, 1e-38, (32, 32)).astype(np.float32)
        elif k == 3:
            t[:] = sgn * g.uniform(1e37, 3.3e38, (32, 32)).astype(np.float32)
        elif k == 4:
            t[:] = sgn * g.uniform(1e-35, 1e-30, (32, 32)).astype(np.float32)
        elif k == 5:
            t[:] = sgn * g.uniform(1e-30, 1e-28, (32, 32)).astype(np.float32)
            t[::4, ::4] = 1e30
        elif k == 6:
            t[:] = sgn * np.float32(1.999) * np.float32(2.0) ** g.integers(-20, 20, (32, 32)).astype(np.float32)
        else:
            t[:] = sgn * g.uniform(0.0, 1.0, (32, 32)).astype(np.float32)
            t[::2, ::2] = np.float32(7.99)
    return x


def gpu_mx(nv, x, dtype, layout, elem, rnd, seed):
    # row stride rounded up to 8 elements (16-byte rows for bf16 and fp32)
    pad = -(-x.shape[1] // 8) * 8
    q = nv.nvfp4_mx_quantize(to_device(x, pad_to=pad), layout=layout, elem=elem, round=rnd, sr_seed=seed)
    torch.cuda.synchronize()
    return q, q.codes.cpu().numpy(), q.scales.cpu().numpy()


def assert_mx_equal(codes, scales, ref, what):
    if not np.array_equal(scales, ref.scales):
        bad = np.argwhere(scales != ref.scales)
        raise AssertionError(f"{what}: {len(bad)} scale bytes differ, first at {bad[0].tolist()} "
                             f"gpu={scales[tuple(bad[0])]} oracle={ref.scales[tuple(bad[0])]}")
    if not np.array_equal(codes, ref.codes):
        bad = np.argwhere(codes != ref.codes)
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first at {bad[0].tolist()} "
                             f"gpu={codes[tuple(bad[0])]:#04x} oracle={ref.codes[tuple(bad[0])]:#04x}")


ROW_SHAPES = [(1, 32), (3, 64), (17, 544), (64, 1056), (130, 2080)]
COL_SHAPES = [(32, 1), (64, 70), (288, 100), (544, 40), (96, 2056)]


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("rnd", [O.RNE, O.SR])
@pytest.mark.parametrize("dtype", [O.BF16, O.F32])
@pytest.mark.parametrize("layout,shape", [(O.ROW_1D, s) for s in ROW_SHAPES] +
                         [(O.COL_1D, s) for s in COL_SHAPES])
def test_mx_quantize_matches_oracle(nv, elem, rnd, dtype, layout, shape):
    seed = shape[0] * 7 + shape[1]
    x = edge_input(shape, seed) if min(shape) >= 32 else W.student_t(shape, 3.0, seed=seed)
    xin = W.f32_to_bf16_bits(x) if dtype == O.BF16 else x
    _, codes, scales = gpu_mx(nv, xin, dtype, layout, elem, rnd, seed + 5)
    ref = O.mx_quantize(xin, dtype, layout, elem, rnd, seed=seed + 5)
    assert_mx_equal(codes, scales, ref, f"mx {shape} layout={layout} elem={elem} rnd={rnd} dtype={dtype}")


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("rnd", [O.RNE, O.SR])
@pytest.mark.parametrize("dtype", [O.BF16, O.F32])
def test_mx_col_tiles_xcd_remap_with_partial_block(nv, elem, rnd, dtype):
    """2304 x 2048 along columns: a 32 x 9 grid of 256-row tiles for bf16
    (64 x 9 for fp32); with nearest-even rounding whole blocks of 8 x 32
    (8 x 64) dispatched workgroups take remapped tiles and the last, partial
    block keeps the dispatch order."""
    x = W.student_t((2304, 2048), 3.0, seed=91)
    xin = W.f32_to_bf16_bits(x) if dtype == O.BF16 else x
    _, codes, scales = gpu_mx(nv, xin, dtype, O.COL_1D, elem, rnd, 92)
    ref = O.mx_quantize(xin, dtype, O.COL_1D, elem, rnd, seed=92)
    assert_mx_equal(codes, scales, ref, f"mx remap elem={elem} rnd={rnd} dtype={dtype}")


@pytest.mark.parametrize("elem", ELEMS)
def test_mx_quantize_strided_input(nv, elem):
    """A row stride wider than the row (a column slice of a wider tensor)."""
    x = W.f32_to_bf16_bits(W.normal((64, 96), 1.0, seed=3))
    for layout in (O.ROW_1D, O.COL_1D):
        q = nv.nvfp4_mx_quantize(to_device(x, pad_to=136), layout=layout, elem=elem, round=O.SR, sr_seed=4)
        torch.cuda.synchronize()
        ref = O.mx_quantize(x, O.BF16, layout, elem, O.SR, seed=4)
        assert_mx_equal(q.codes.cpu().numpy(), q.scales.cpu().numpy(), ref, f"strided layout={layout}")


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("layout", [O.ROW_1D, O.COL_1D])
def test_mx_sr_large_blocks_with_smallest_subnormals(nv, elem, layout):
    """BF16 stochastic rounding with block scales 2^s, s = 17: in every other
    32 x 32 square the diagonal holds 2^25 (E4M3) or 2^19 (E2M1) and the rest
    the smallest BF16 subnormal 2^-133, so every row and column block mixes
    the two.  Then |v| * 2^-s = 2^-150 rounds to 0 and the code must be 0
    under every draw; one multiply by 2^-s times 2^29 (or 2^23) would round up
    on a zero draw.  Other squares hold ordinary values, so waves mix both
    kinds of block.  The test first counts, with the oracle's draws, the
    subnormal elements whose draw is 0 (at least one), so the case is really
    exercised."""
    n = 1024
    x = W.normal((n, n), 1.0, seed=4343)
    big = np.float32(2.0 ** 25 if elem == O.MX_FP8 else 2.0 ** 19)
    tiny = np.float32(2.0 ** -133)
    mask = np.zeros((n, n), dtype=bool)
    for bi in range(n // 32):
        for bj in range(n // 32):
            if (bi + bj) % 2:
                continue
            sq = x[32 * bi:32 * bi + 32, 32 * bj:32 * bj + 32]
            sq[:] = tiny
            np.fill_diagonal(sq, big)
            m = mask[32 * bi:32 * bi + 32, 32 * bj:32 * bj + 32]
            m[:] = True
            np.fill_diagonal(m, False)
    xb = W.f32_to_bf16_bits(x)
    assert np.all(xb[mask] == 0x0001)
    seed = 62
    rr, cc = np.nonzero(mask)
    # random streams of the MX layouts: 4 row blocks, 5 column blocks; index in the output tensor
    stream, idx = (4, rr * n + cc) if layout == O.ROW_1D else (5, cc * n + rr)
    zero_draws = sum(1 for i in idx.tolist() if O.draw16(seed, stream, i) == 0)
    assert zero_draws >= 1, "no subnormal element draws 0"
    _, codes, scales = gpu_mx(nv, xb, O.BF16, layout, elem, O.SR, seed)
    ref = O.mx_quantize(xb, O.BF16, layout, elem, O.SR, seed=seed)
    assert_mx_equal(codes, scales, ref, f"large blocks {layout} elem={elem}")


def test_mx_empty(nv):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q = nv.nvfp4_mx_quantize(x)
    y = nv.nvfp4_mx_dequantize(q)
    torch.cuda.synchronize()
    assert q.codes.numel() == 0 and y.shape == (0, 64)


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("out", [O.F32, O.BF16])
def test_mx_dequantize_matches_oracle(nv, elem, out):
    """Dequantization of (a) a quantized edge-case tensor and (b) arbitrary
    code and scale bytes over the whole E8M0 range (results that overflow to
    infinity or land among binary32 subnormals included)."""
    x = edge_input((96, 320), 11)
    q = O.mx_quantize(x, O.F32, O.ROW_1D, elem, O.RNE)
    g = W.rng(12)
    nbytes = 320 if elem == O.MX_FP8 else 160
    codes = g.integers(0, 256, (96, nbytes), dtype=np.uint8)
    if elem == O.MX_FP8:
        codes[(codes & 0x7F) == 0x7F] = 0x3C  # E4M3 NaN encodings are not values
    scales = g.integers(0, 255, (96, 10), dtype=np.uint8)
    rnd = O.MXTensor(codes, scales, 96, 320, elem)
    for qh in (q, rnd):
        qd = nv.MXTensor(torch.from_numpy(qh.codes).cuda(), torch.from_numpy(qh.scales).cuda(), qh.rows, qh.cols,
                         elem)
        y = nv.nvfp4_mx_dequantize(qd, dtype=torch.bfloat16 if out == O.BF16 else torch.float32)
        ref = O.mx_dequantize(qh, out)
        got = bf16_tensor_to_bits(y) if out == O.BF16 else y.cpu().numpy()
        assert np.array_equal(got.view(np.uint16 if out == O.BF16 else np.uint32),
                              ref.view(np.uint16 if out == O.BF16 else np.uint32)), "dequantize"


@pytest.mark.parametrize("elem", ELEMS)
def test_mx_round_trip_of_grid_values(nv, elem):
    """A block whose values all lie on the element grid times 2^s, with its
    largest magnitude in [2^emax, 2^(emax+1)), comes back unchanged under
    both roundings (no draw can move an exact grid value)."""
    g = W.rng(21)
    vals = ([0, .5, 1, 1.5, 2, 3, 4, 6] if elem == O.MX_FP4 else
            [O.e4m3_value(b) for b in range(0x7F)])
    v = np.array(vals, dtype=np.float32)
    top = 6.0 if elem == O.MX_FP4 else 448.0
    x = g.choice(v, size=(64, 256)).astype(np.float32) * np.where(g.random((64, 256)) < 0.5, -1, 1).astype(np.float32)
    x[:, ::32] = top
    x *= np.float32(2.0) ** g.integers(-30, 30, (64, 1)).astype(np.float32)
    for rnd in (O.RNE, O.SR):
        q = nv.nvfp4_mx_quantize(to_device(x), elem=elem, round=rnd, sr_seed=99)
        y = nv.nvfp4_mx_dequantize(q)
        assert np.array_equal(y.cpu().numpy(), x), f"round trip rnd={rnd}"


@pytest.mark.parametrize("layout", [O.ROW_1D, O.COL_1D])
@pytest.mark.parametrize("elem", ELEMS)
def test_mx_8192_sampled(nv, layout, elem):
    """8192 x 8192 BF16 Student-t(3), stochastic rounding, in the benchmarked
    launch configuration: 64-row (ROW) or 64-column (COL) bands of the output
    against the oracle with the band's own draw indices."""
    n = 8192
    xb = W.f32_to_bf16_bits(W.student_t((n, n), 3.0, seed=8100))
    _, codes, scales = gpu_mx(nv, xb, O.BF16, layout, elem, O.SR, 8101)
    for b0 in (0, 4096 + 32, n - 64):
        if layout == O.ROW_1D:
            ref = O.mx_quantize(np.ascontiguousarray(xb[b0:b0 + 64]), O.BF16, layout, elem, O.SR, seed=8101,
                                index_base=b0 * n)
        else:
            ref = O.mx_quantize(np.ascontiguousarray(xb[:, b0:b0 + 64]), O.BF16, layout, elem, O.SR, seed=8101,
                                index_base=b0 * n)
        assert_mx_equal(codes[b0:b0 + 64], scales[b0:b0 + 64], ref, f"band {b0}")
