"""GPU parity of re-quantization along columns (a row-blocked NVFP4 tensor
re-formed into column blocks, the backward pass's operand: "Thinking Machines
ускорила обучение Inkling 2 Small 4-битными числами", iitak.ru, section "Как
это работает") against the oracle's composition quantize(COL_1D,
dequantize(q)): codes, scale bytes and tensor scales bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_utils import assert_q_equal, q_to_device, q_to_host, require_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def row_quantized(rows, cols, seed, kind="t3"):
    if kind == "t3":
        x = W.student_t((rows, cols), 3.0, seed=seed)
    else:
        x = W.with_spikes(W.normal((rows, cols), 1.0, seed=seed), 1e-3, 100.0, seed=seed + 1)
    return O.quantize(W.f32_to_bf16_bits(x), O.BF16, O.ROW_1D, O.SR, sr_seed=seed + 2)


# cols % 32 == 16 exercises the half-width last tile; rows past a 256-row tile the partial band tile
SHAPES = [(16, 16), (48, 80), (256, 96), (272, 1040), (1040, 48), (64, 2064)]


@pytest.mark.parametrize("rnd", [O.RNE, O.SR])
@pytest.mark.parametrize("had", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_requantize_matches_oracle(nv, rnd, had, shape):
    q = row_quantized(*shape, seed=shape[0] * 3 + shape[1], kind="spiky" if had else "t3")
    got = q_to_host(nv.nvfp4_requantize(q_to_device(q, nv), round=rnd, sr_seed=41, hadamard=had,
                                        hadamard_seed=43))
    ref = O.requantize(q, rnd, sr_seed=41, hadamard=had, hadamard_seed=43)
    assert_q_equal(got, ref, f"requantize {shape} rnd={rnd} had={had}")


def test_requantize_equals_quantize_of_dequantized(nv):
    """The fused kernel against the two-call path on the GPU: F32 dequantize,
    then COL_1D quantize of the result."""
    q = q_to_device(row_quantized(512, 384, seed=5), nv)
    for rnd in (O.RNE, O.SR):
        fused = q_to_host(nv.nvfp4_requantize(q, round=rnd, sr_seed=9))
        x = nv.nvfp4_dequantize(q, dtype=torch.float32)
        two = q_to_host(nv.nvfp4_quantize(x, layout=nv.NVFP4_COL_1D, round=rnd, sr_seed=9))
        assert_q_equal(fused, two, f"fused vs two-call rnd={rnd}")


def test_requantize_amax_in_and_out(nv):
    q = row_quantized(96, 160, seed=11)
    qd = q_to_device(q, nv)
    amax_out = torch.zeros(1, dtype=torch.float32, device="cuda")
    a = nv.nvfp4_requantize(qd, round=O.SR, sr_seed=2, amax_out=amax_out)
    torch.cuda.synchronize()
    xref = O.dequantize(q, O.F32)
    assert amax_out.item() == O.amax(xref, O.F32, O.COL_1D)
    b = nv.nvfp4_requantize(qd, round=O.SR, sr_seed=2, amax_in=amax_out)
    assert_q_equal(q_to_host(b), q_to_host(a), "amax_in chained")
    small = torch.tensor([0.25 * amax_out.item()], dtype=torch.float32, device="cuda")
    c = nv.nvfp4_requantize(qd, round=O.SR, sr_seed=2, amax_in=small)
    assert_q_equal(q_to_host(c), O.requantize(q, O.SR, sr_seed=2, amax_in=0.25 * amax_out.item()),
                   "understated amax")


def test_requantize_empty(nv):
    e = nv.NVFP4Tensor.empty(0, 32)
    r = nv.nvfp4_requantize(e)
    torch.cuda.synchronize()
    assert (r.rows, r.cols) == (32, 0) and r.tensor_scale.item() == 1.0


@pytest.mark.parametrize("had", [False, True])
def test_requantize_8192_sampled(nv, had):
    """8192 x 8192: the forward tensor quantized along rows on the GPU (equal
    to the oracle's row quantization), then re-quantized along columns with
    stochastic rounding (the benchmarked call): the tensor scale against the
    oracle's amax of the whole dequantized tensor, and 64-row bands of the
    output against the oracle with the band's own random-draw indices.  The
    oracle works from its own row quantization."""
    n = 8192
    xb = W.f32_to_bf16_bits(W.student_t((n, n), 3.0, seed=7000))
    qd = nv.nvfp4_quantize(to_device(xb), round=nv.NVFP4_SR, sr_seed=7001)
    r = q_to_host(nv.nvfp4_requantize(qd, round=nv.NVFP4_SR, sr_seed=7002, hadamard=had,
                                      hadamard_seed=7003))
    q = O.quantize(xb, O.BF16, O.ROW_1D, O.SR, sr_seed=7001)
    assert_q_equal(q_to_host(qd), q, "row quantization")
    xd = O.dequantize(q, O.F32)
    amax = O.amax(xd, O.F32, O.COL_1D, hadamard=had, hadamard_seed=7003)
    assert r.ts == O.tensor_scale(amax)
    for b0 in (0, 4096 + 32, n - 64):
        sub = np.ascontiguousarray(xd[:, b0:b0 + 64])
        ref = O.quantize(sub, O.F32, O.COL_1D, O.SR, sr_seed=7002, hadamard=had, hadamard_seed=7003,
                         amax_in=amax, index_base=b0 * n)
        assert np.array_equal(r.codes[b0:b0 + 64], ref.codes), f"codes band {b0}"
        assert np.array_equal(r.scales[b0:b0 + 64], ref.scales), f"scales band {b0}"
