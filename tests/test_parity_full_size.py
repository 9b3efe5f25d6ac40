"""Whole-output GPU parity at the workloads' full sizes, in the launch
configurations the benchmark times: every code byte, scale byte and tensor
scale of the 8192 x 8192 activation's row, column, fused row+column and
16x16 quantizations (nearest-even and stochastic rounding) and its
dequantizations, the 20480 x 5120 weight's 16x16 quantization, the weight
gradient operands' Hadamard + column + stochastic quantization (8192 x 20480
and 8192 x 5120), and the MoE activation's row quantization (16384 x 7168),
against the oracle.  The oracle runs band by band on every core
(oracle/banded.py: the unchanged oracle called once per independent band,
byte-identical to single calls), so a whole tensor takes seconds; the amax
is computed on the GPU by the call under test and its tensor scale compared
with the oracle's.  A single wrong code anywhere -- a tile edge in the middle
of the tensor, a 16x16 square holding an outlier (the pages' example of one
large value zeroing the rest of its square, "Thinking Machines ускорила
обучение Inkling 2 Small 4-битными числами", iitak.ru, section "Как это
работает") -- fails the test."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from oracle import banded as OB
from parity_utils import assert_q_equal, bf16_tensor_to_bits, q_to_host, require_gpu, to_device

pytestmark = pytest.mark.gpu

_inputs = {}


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def _act8192():
    """The benchmark step's first input: 8192 x 8192 BF16 Student-t(3), seed 1000."""
    if "act" not in _inputs:
        _inputs["act"] = W.f32_to_bf16_bits(W.student_t((8192, 8192), 3.0, seed=1000))
    return _inputs["act"]


def _free_inputs():
    _inputs.clear()


@pytest.mark.parametrize("layout,rnd", [(O.ROW_1D, O.RNE), (O.ROW_1D, O.SR), (O.COL_1D, O.RNE),
                                        (O.COL_1D, O.SR), (O.BLK_2D, O.RNE), (O.BLK_2D, O.SR)])
def test_activation_8192_whole(nv, layout, rnd):
    x = _act8192()
    print(f"activation 8192^2 layout {layout} round {rnd}", flush=True)
    got = q_to_host(nv.nvfp4_quantize(to_device(x), layout=layout, round=rnd, sr_seed=1100))
    ref = OB.quantize(x, O.BF16, layout, rnd, sr_seed=1100)
    assert_q_equal(got, ref, f"8192^2 layout {layout} round {rnd}")


@pytest.mark.parametrize("rnd", [O.RNE, O.SR])
def test_activation_8192_rowcol_whole(nv, rnd):
    """The fused kernel's two outputs against the oracle's row and column
    quantizations (one shared A_t, random streams 0 and 1)."""
    x = _act8192()
    print(f"activation 8192^2 fused row+col round {rnd}", flush=True)
    r, c = nv.nvfp4_quantize(to_device(x), layout=nv.NVFP4_ROW_COL_1D, round=rnd, sr_seed=1200)
    ref_r, ref_c = OB.quantize(x, O.BF16, O.ROW_COL_1D, rnd, sr_seed=1200)
    assert_q_equal(q_to_host(r), ref_r, f"fused row, round {rnd}")
    assert_q_equal(q_to_host(c), ref_c, f"fused col, round {rnd}")


def test_activation_8192_dequantize_whole(nv):
    """The step's dequantizations: row and column blocks (nearest-even) back
    to BF16, and row blocks to FP32, every element."""
    x = _act8192()
    xd = to_device(x)
    for layout in (O.ROW_1D, O.COL_1D):
        print(f"dequantize 8192^2 layout {layout}", flush=True)
        q = nv.nvfp4_quantize(xd, layout=layout)
        ref_q = OB.quantize(x, O.BF16, layout)
        assert_q_equal(q_to_host(q), ref_q, f"dequantize input, layout {layout}")
        y = bf16_tensor_to_bits(nv.nvfp4_dequantize(q, dtype=torch.bfloat16))
        assert np.array_equal(y, OB.dequantize(ref_q, O.BF16)), f"BF16 dequantize, layout {layout}"
        if layout == O.ROW_1D:
            y32 = nv.nvfp4_dequantize(q, dtype=torch.float32).cpu().numpy()
            assert np.array_equal(y32.view(np.uint32), OB.dequantize(ref_q, O.F32).view(np.uint32))
    _free_inputs()


def test_weight_2d_20480x5120_whole(nv):
    """Weight 20480 x 5120 BF16 N(0, 0.02), 16 x 16 blocks, RNE, and its
    dequantization to BF16."""
    x = W.f32_to_bf16_bits(W.normal((20480, 5120), 0.02, seed=2000))
    q = nv.nvfp4_quantize(to_device(x), layout=nv.NVFP4_BLK_2D)
    ref = OB.quantize(x, O.BF16, O.BLK_2D)
    assert_q_equal(q_to_host(q), ref, "weight 2D")
    y = bf16_tensor_to_bits(nv.nvfp4_dequantize(q, dtype=torch.bfloat16))
    assert np.array_equal(y, OB.dequantize(ref, O.BF16)), "weight 2D dequantize"


@pytest.mark.parametrize("rows,cols,seed", [(8192, 20480, 3000), (8192, 5120, 3010)])
def test_wgrad_hadamard_col_sr_whole(nv, rows, cols, seed):
    """dY 8192 x 20480 and X 8192 x 5120, N(0,1) with 0.01% x100 spikes:
    Hadamard along tokens, column blocks, stochastic rounding; the amax of
    the transformed tensor computed on the GPU."""
    x = W.f32_to_bf16_bits(W.with_spikes(W.normal((rows, cols), 1.0, seed=seed), 1e-4, 100.0,
                                         seed=seed + 1))
    q = nv.nvfp4_quantize(to_device(x), layout=nv.NVFP4_COL_1D, round=nv.NVFP4_SR, sr_seed=seed + 100,
                          hadamard=True, hadamard_seed=seed + 200)
    ref = OB.quantize(x, O.BF16, O.COL_1D, O.SR, sr_seed=seed + 100, hadamard=True, hadamard_seed=seed + 200)
    assert_q_equal(q_to_host(q), ref, f"gradient {rows}x{cols}")


def test_moe_activation_16384x7168_row_whole(nv):
    """The MoE workload's token activations, 16384 x 7168 Student-t(3), row
    blocks, RNE (the grouped GEMM's A before the expert gather)."""
    x = W.f32_to_bf16_bits(W.student_t((16384, 7168), 3.0, seed=6000))
    q = nv.nvfp4_quantize(to_device(x), layout=nv.NVFP4_ROW_1D)
    assert_q_equal(q_to_host(q), OB.quantize(x, O.BF16, O.ROW_1D), "MoE activations")
