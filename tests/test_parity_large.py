"""GPU parity past 2^31 elements: a BF16 tensor of 16400 x 131072
(2,149,580,800 elements) quantized along rows (RNE and SR), along rows and
columns at once (SR) and in 16x16 blocks, then dequantized; and a GEMM whose
FP32 output holds 65536 x 32896 (2,155,872,256) elements.  Element offsets,
output offsets and random-draw indices all cross 2^31 in these launches.

The input is a seeded 256-row Student-t(3) block repeated down the rows, each
256-row repetition rotated along the columns by its own amount, so every row
differs from every other; the oracle rebuilds any band of it on the host and
checks bands at the start, the middle and across the 2^31 boundary against
its own quantization with the whole tensor's amax and the band's own
random-draw indices."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import banded as OB
import workloads as W
from parity_utils import assert_q_equal, bf16_tensor_to_bits, gemm_tol, require_gpu

pytestmark = pytest.mark.gpu

ROWS, COLS = 16400, 131072
PERIOD = 256


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def _shift(block):
    return (977 * np.asarray(block, dtype=np.int64)) % COLS


def _rows_host(base, r0, n):
    """Rows r0 .. r0+n-1 of the tensor, on the host."""
    out = np.empty((n, COLS), dtype=np.uint16)
    for i in range(n):
        r = r0 + i
        out[i] = np.roll(base[r % PERIOD], int(_shift(r // PERIOD)))
    return out


def _cols_host(base, c0, n):
    """Columns c0 .. c0+n-1 of the tensor (all rows), on the host."""
    r = np.arange(ROWS)
    idx = (c0 + np.arange(n)[None, :] - _shift(r // PERIOD)[:, None]) % COLS
    return np.ascontiguousarray(base[(r % PERIOD)[:, None], idx])


def _big_input():
    base = W.f32_to_bf16_bits(W.student_t((PERIOD, COLS), 3.0, seed=9000))
    bd = torch.from_numpy(base.view(np.int16)).cuda().view(torch.bfloat16)
    x = torch.empty((ROWS, COLS), dtype=torch.bfloat16, device="cuda")
    for j in range((ROWS + PERIOD - 1) // PERIOD):
        r0 = PERIOD * j
        n = min(PERIOD, ROWS - r0)
        x[r0:r0 + n] = torch.roll(bd[:n], shifts=int(_shift(j)), dims=1)
    return base, x


def _host_rows(q, r0, n, scale_2d=False):
    torch.cuda.synchronize()
    sc = q.scales[r0 // 16:(r0 + n) // 16] if scale_2d else q.scales[r0:r0 + n]
    return O.QTensor(q.codes[r0:r0 + n].cpu().numpy(), sc.cpu().numpy(), float(q.tensor_scale[0].item()),
                     n, q.cols, O.SCALE_2D if scale_2d else O.SCALE_1D)


# row bands (start, height): the start, the middle, and the last 32 rows,
# whose elements all lie past 2^31 (row 16384 starts at element 2^31)
ROW_BANDS = [(0, 64), (8192, 64), (ROWS - 32, 32)]
# column bands of the transposed output: column 130944 holds output element
# 2^31 (130944 * 16400 + 10112), so the middle band crosses it
COL_BANDS = [(0, 64), (130928, 64), (COLS - 64, 64)]


def test_quantize_dequantize_past_2pow31_elements(nv):
    base, x = _big_input()
    amax = O.amax(base, O.BF16, O.ROW_1D)  # the tensor holds exactly base's values
    ts = O.tensor_scale(amax)
    amax_d = torch.tensor([amax], dtype=torch.float32, device="cuda")

    # row blocks, nearest-even, amax computed by the library; then dequantize
    q = nv.nvfp4_quantize(x)
    torch.cuda.synchronize()
    assert float(q.tensor_scale[0].item()) == ts
    y = nv.nvfp4_dequantize(q, dtype=torch.bfloat16)
    for r0, n in ROW_BANDS:
        ref = O.quantize(_rows_host(base, r0, n), O.BF16, O.ROW_1D, amax_in=amax)
        assert_q_equal(_host_rows(q, r0, n), ref, f"row RNE band {r0}")
        got = bf16_tensor_to_bits(y[r0:r0 + n])
        assert np.array_equal(got, O.dequantize(ref, O.BF16)), f"dequantize band {r0}"
    del q, y
    torch.cuda.empty_cache()

    # row blocks, stochastic rounding: draw indices past 2^31
    q = nv.nvfp4_quantize(x, round=nv.NVFP4_SR, sr_seed=9100, amax_in=amax_d)
    for r0, n in ROW_BANDS:
        ref = O.quantize(_rows_host(base, r0, n), O.BF16, O.ROW_1D, O.SR, sr_seed=9100, amax_in=amax,
                         index_base=r0 * COLS)
        assert_q_equal(_host_rows(q, r0, n), ref, f"row SR band {r0}")
    del q
    torch.cuda.empty_cache()

    # rows and columns from one read, stochastic rounding
    r, c = nv.nvfp4_quantize(x, layout=nv.NVFP4_ROW_COL_1D, round=nv.NVFP4_SR, sr_seed=9200, amax_in=amax_d)
    for r0, n in ROW_BANDS:
        ref = O.quantize(_rows_host(base, r0, n), O.BF16, O.ROW_1D, O.SR, sr_seed=9200, amax_in=amax,
                         index_base=r0 * COLS)
        assert_q_equal(_host_rows(r, r0, n), ref, f"fused row band {r0}")
    for c0, n in COL_BANDS:
        ref = O.quantize(_cols_host(base, c0, n), O.BF16, O.COL_1D, O.SR, sr_seed=9200, amax_in=amax,
                         index_base=c0 * ROWS)
        assert_q_equal(_host_rows(c, c0, n), ref, f"fused column band {c0}")
    del r, c
    torch.cuda.empty_cache()

    # 16 x 16 blocks, nearest-even
    q = nv.nvfp4_quantize(x, layout=nv.NVFP4_BLK_2D, amax_in=amax_d)
    for r0, n in ROW_BANDS:
        ref = O.quantize(_rows_host(base, r0, n), O.BF16, O.BLK_2D, amax_in=amax)
        assert_q_equal(_host_rows(q, r0, n, scale_2d=True), ref, f"2D band {r0}")
    del q, x
    torch.cuda.empty_cache()


def test_gemm_output_past_2pow31_elements(nv):
    """C = A B^T with M = 65536, N = 32896 (a ragged last column tile),
    K = 512, FP32 out: entries near the end of C, past element 2^31."""
    M, N, K = 65536, 32896, 512
    a = W.f32_to_bf16_bits(W.student_t((M, K), 3.0, seed=9300))
    b = W.f32_to_bf16_bits(W.normal((N, K), 0.02, seed=9301))
    da = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    db = torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)
    Aq = nv.nvfp4_quantize(da)
    Bq = nv.nvfp4_quantize(db, layout=nv.NVFP4_BLK_2D)
    C = nv.nvfp4_gemm(Aq, Bq, out_dtype=torch.float32)
    g = W.rng(9302)
    mi = np.concatenate([g.integers(65281, M, 512), g.integers(0, M, 64), [0, M - 1, M - 1, 65281]])
    ni = np.concatenate([g.integers(0, N, 576), [0, 0, N - 1, 32768]])
    got = C[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy().astype(np.float64)
    # the oracle quantizes the rows it needs (rows of A and 16-row bands of
    # B are independent given the tensor amax) and checks the GPU's equal
    mu, ml = np.unique(mi, return_inverse=True)
    Ar = O.quantize(np.ascontiguousarray(a[mu]), O.BF16, O.ROW_1D, amax_in=O.amax(a, O.BF16, O.ROW_1D))
    bands = np.unique(ni // 16)
    Br = O.quantize(np.concatenate([b[16 * k:16 * k + 16] for k in bands]), O.BF16, O.BLK_2D,
                    amax_in=O.amax(b, O.BF16, O.BLK_2D))
    nl = np.searchsorted(bands, ni // 16) * 16 + ni % 16
    torch.cuda.synchronize()
    ia = torch.from_numpy(mu).cuda()
    assert_q_equal(O.QTensor(Aq.codes.index_select(0, ia).cpu().numpy(), Aq.scales.index_select(0, ia).cpu().numpy(),
                             float(Aq.tensor_scale[0].item()), mu.size, K, O.SCALE_1D), Ar, "A rows")
    rb = torch.from_numpy((16 * bands[:, None] + np.arange(16)[None, :]).reshape(-1)).cuda()
    assert_q_equal(O.QTensor(Bq.codes.index_select(0, rb).cpu().numpy(),
                             Bq.scales.index_select(0, torch.from_numpy(bands).cuda()).cpu().numpy(),
                             float(Bq.tensor_scale[0].item()), 16 * bands.size, K, O.SCALE_2D), Br, "B bands")
    Cref, Wref = OB.gemm(Ar, Br, entries=(ml, nl))
    tol = gemm_tol(Cref, Wref, False)
    bad = np.abs(got - Cref) > tol
    assert not bad.any(), f"{bad.sum()} entries out of tolerance, first at {(mi[bad][0], ni[bad][0])}"
