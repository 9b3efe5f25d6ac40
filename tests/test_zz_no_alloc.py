"""The allocation-free quantize entry point (nvfp4_quantize_noalloc), called
through the C ABI, against nvfp4_quantize with a caller workspace: codes,
scale bytes, tensor scales and the published amax must agree bit for bit, on
two calls in a row per case, the second on a smaller input (the static
scratch keeps the first call's partials and must not leak into the second)."""
import numpy as np
import pytest
import torch

import workloads as W
from parity_utils import require_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def _outs(nv, rows, cols, layout):
    if layout == nv.NVFP4_COL_1D:
        return nv.NVFP4Tensor.empty(cols, rows)
    if layout == nv.NVFP4_BLK_2D:
        return nv.NVFP4Tensor.empty(rows, cols, nv.NVFP4_SCALE_2D)
    if layout == nv.NVFP4_ROW_COL_1D:
        return (nv.NVFP4Tensor.empty(rows, cols), nv.NVFP4Tensor.empty(cols, rows))
    return nv.NVFP4Tensor.empty(rows, cols)


def _flat(res):
    res = res if isinstance(res, tuple) else (res,)
    return [t for q in res for t in (q.codes, q.scales, q.tensor_scale)]


CASES = [("row_sr", 0, 1, False), ("col_rne", 1, 0, False), ("rowcol_sr", 2, 1, False),
         ("rowcol_sr_hadamard", 2, 1, True), ("col_sr_hadamard", 1, 1, True), ("2d_rne", 3, 0, False)]


@pytest.mark.parametrize("name,layout,rnd,had", CASES)
def test_noalloc_matches_workspace_entry_point(nv, name, layout, rnd, had):
    # first a large input (many amax partials), then a smaller one (fewer)
    for step, (rows, cols) in enumerate([(4096, 2048), (272, 160)]):
        print(f"noalloc {name}: call {step} on {rows}x{cols}", flush=True)
        x = to_device(W.f32_to_bf16_bits(W.with_spikes(
            W.student_t((rows, cols), 3.0, seed=90 + step), 1e-4, 40.0, seed=91 + step)))
        n_amax = 2 if (layout == nv.NVFP4_ROW_COL_1D and had) else 1
        a_ref = torch.zeros(n_amax, dtype=torch.float32, device="cuda")
        a_got = torch.full((n_amax,), -1.0, dtype=torch.float32, device="cuda")
        ref = nv.nvfp4_quantize(x, layout=layout, round=rnd, sr_seed=17 + step, hadamard=had,
                                hadamard_seed=5, out=_outs(nv, rows, cols, layout), amax_out=a_ref)
        got = nv.nvfp4_quantize_noalloc(x, _outs(nv, rows, cols, layout), layout=layout, round=rnd,
                                        sr_seed=17 + step, hadamard=had, hadamard_seed=5, amax_out=a_got)
        torch.cuda.synchronize()
        for k, (g, r) in enumerate(zip(_flat(got), _flat(ref))):
            assert torch.equal(g.view(torch.uint8), r.view(torch.uint8)), f"{name} call {step}: output {k}"
        assert torch.equal(a_got, a_ref), f"{name} call {step}: amax {a_got.tolist()} != {a_ref.tolist()}"
        # the published amax is the tensor's own
        if not had:
            assert a_got[0].item() == x.float().abs().max().item()
