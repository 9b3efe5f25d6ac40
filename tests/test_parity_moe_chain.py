"""The MoE expert forward as one chain on the GPU, at the workload's full
shape (32 experts, hidden 7168, FFN 2048, 16384 tokens top-4, Zipf(1.1)
expert loads): quantize the tokens (row blocks), gather them by expert,
grouped up-projection with the SwiGLU epilogue and its amax, quantize H with
that amax, grouped down-projection on the GPU-quantized H.  NVFP4 in the
expert layers' forward pass is what the pages describe ("Thinking Machines
ускорила обучение Inkling 2 Small 4-битными числами", iitak.ru, section
"Детали").

The oracle never reads a GPU result.  To follow the chain step for step
anyway, the operands are E2M1 grid values (the pages' value set) with a
largest-magnitude 6 in every 16-element row block of X and every 16x16 square
of the weights, quantized with a given tensor amax of 2688: every block
multiplier and tensor scale is then 1, each GEMM sum is a multiple of 1/4
below 2^18 and exact in binary32, so the GPU's and the oracle's up-projection
agree exactly and H differs only where the two sides' sigmoids differ: in
the last bit, or below binary32's normal range (g < -87, where the GPU's
binary32 sigmoid is 0 and the oracle's float64 one still gives a BF16
subnormal).  On sampled rows:
  - H from the GPU is within the SwiGLU tolerance of the oracle's H (float64
    SwiGLU rounded to BF16) everywhere, and equal to it bit for bit in most
    16-element blocks;
  - the epilogue's amax equals the largest |H| of the GPU's H, and the
    oracle's own H at that position (the GPU gives only the index);
  - the GPU's quantized H equals the oracle's quantization of its own H with
    its own amax in every block whose 16 H values agree;
  - the down-projection of the GPU-quantized H equals the oracle's GEMM of
    the oracle-quantized H on the rows whose quantized H agrees throughout,
    within 1e-5 sum |a b|.
Distribution-faithful operands at the same shape are checked by
test_parity_gemm.py::test_moe_expert_forward_sampled."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from oracle import banded as OB
from parity_utils import assert_q_equal, bf16_tensor_to_bits, gemm_tol, q_to_host, require_gpu, to_device

pytestmark = pytest.mark.gpu

GRID = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -.5, -1, -1.5, -2, -3, -4, -6], dtype=np.float32)


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def grid_rows(shape, seed):
    """E2M1 grid values; element 0 of every 16-element row block is +-6."""
    g = W.rng(seed)
    x = GRID[g.integers(0, GRID.size, shape, dtype=np.int8)]
    x[:, ::16] = np.where(g.integers(0, 2, (shape[0], shape[1] // 16)) == 1, 6.0, -6.0)
    return W.f32_to_bf16_bits(x)


def grid_squares(shape, seed):
    """E2M1 grid values; element (0, 0) of every 16x16 square is 6."""
    g = W.rng(seed)
    x = GRID[g.integers(0, GRID.size, shape, dtype=np.int8)]
    x[::16, ::16] = 6.0
    return W.f32_to_bf16_bits(x)


def _swiglu_tol(G_, U_, Wg, Wu):
    from scipy.special import expit
    s = expit(G_)
    dh_dg = np.abs(s * (1.0 + G_ * (1.0 - s)) * U_)
    dh_du = np.abs(G_ * s)
    h = np.abs(G_ * s * U_)
    # one BF16 rounding: half a spacing, at least the subnormal spacing 2^-133
    e = np.maximum(np.floor(np.log2(np.where(h > 0, h, 1.0))), -126.0)
    ulp = np.where(h > 0, 2.0 ** (e - 7), 2.0 ** -133)
    # a binary32 sigmoid below the normal range (sigma < 2^-126, g < -87.3)
    # is 0 or a subnormal: at most |g u| 2^-126 of absolute error in h
    under = np.abs(G_ * U_) * 2.0 ** -126
    return dh_dg * 1e-5 * Wg + dh_du * 1e-5 * Wu + 1e-6 * h + ulp + under


def test_moe_chain_full_shape(nv):
    E, Hd, F, T = 32, 7168, 2048, 16384
    A_GIVEN = 2688.0  # every block multiplier and tensor scale 1
    counts = W.zipf_expert_counts(E, T, 4, 1.1)
    offs, token = W.moe_routing(counts, T)
    total = int(offs[-1])
    dev = "cuda"
    given = torch.tensor([A_GIVEN], dtype=torch.float32, device=dev)

    print("chain: tokens", flush=True)
    x = grid_rows((T, Hd), seed=8000)
    Xq = nv.nvfp4_quantize(to_device(x), amax_in=given)
    Xref = OB.quantize(x, O.BF16, O.ROW_1D, amax_in=A_GIVEN)
    assert_q_equal(q_to_host(Xq), Xref, "tokens")
    idx = torch.from_numpy(token).to(dev)
    Aperm = nv.NVFP4Tensor(Xq.codes.index_select(0, idx), Xq.scales.index_select(0, idx), Xq.tensor_scale,
                           total, Hd)

    groups = (0, 7, 15, 31)
    print("chain: weights", flush=True)
    W1 = nv.NVFP4Tensor.empty(E * 2 * F, Hd, nv.NVFP4_SCALE_2D, n_scales=E)
    W2 = nv.NVFP4Tensor.empty(E * Hd, F, nv.NVFP4_SCALE_2D, n_scales=E)
    w1ref, w2ref = {}, {}
    for e in range(E):
        for Wt, rows, cols, seed, keep in ((W1, 2 * F, Hd, 8100 + e, w1ref), (W2, Hd, F, 8200 + e, w2ref)):
            w = grid_squares((rows, cols), seed)
            q = nv.nvfp4_quantize(to_device(w), layout=nv.NVFP4_BLK_2D, amax_in=given)
            ref = OB.quantize(w, O.BF16, O.BLK_2D, amax_in=A_GIVEN)
            assert_q_equal(q_to_host(q), ref, f"weights of expert {e}")
            Wt.codes[e * rows:(e + 1) * rows].copy_(q.codes)
            Wt.scales[e * rows // 16:(e + 1) * rows // 16].copy_(q.scales)
            Wt.tensor_scale[e:e + 1].copy_(q.tensor_scale)
            if e in groups:
                keep[e] = ref
    offs_d = torch.from_numpy(offs).to(dev)

    print("chain: GPU up-projection, quantize, down-projection", flush=True)
    hmax = torch.zeros(1, dtype=torch.float32, device=dev)
    H = nv.nvfp4_grouped_gemm(Aperm, offs_d, W1, E, epilogue=nv.NVFP4_EPI_SWIGLU, amax_out=hmax)
    Hq = nv.nvfp4_quantize(H, amax_in=hmax)
    Y = nv.nvfp4_grouped_gemm(Hq, offs_d, W2, E, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()

    # the epilogue's amax is the largest |H| of the GPU's H; the oracle's H at
    # that position (found on the GPU: an index, not a value) is the same number
    habs = H.float().abs()
    flat = int(torch.argmax(habs).item())
    m_star, n_star = divmod(flat, F)
    assert hmax.item() == habs.view(-1)[flat].item()
    g_star = int(np.searchsorted(offs, m_star, side="right") - 1)
    W1g = OB.quantize(grid_squares((2 * F, Hd), 8100 + g_star), O.BF16, O.BLK_2D, amax_in=A_GIVEN)
    a_row = O.row_slice(Xref, int(token[m_star]), int(token[m_star]) + 1)
    cg, _ = O.gemm(a_row, W1g, entries=(np.array([0, 0]), np.array([n_star, F + n_star])))
    h_star = W.bf16_bits_to_f32(W.f32_to_bf16_bits(O.swiglu(cg[0], cg[1]).astype(np.float32).reshape(1)))[0]
    a_ref = float(abs(h_star))
    assert a_ref == hmax.item(), f"amax: oracle |H| {a_ref} at ({m_star}, {n_star}), epilogue {hmax.item()}"

    Hh = bf16_tensor_to_bits(H)
    Hqh = q_to_host(Hq)
    assert Hqh.ts == O.tensor_scale(a_ref)
    Yh = W.bf16_bits_to_f32(bf16_tensor_to_bits(Y)).astype(np.float64)
    rows_same = rows_checked = blocks_same = blocks_checked = 0
    for g_ in groups:
        r0, r1 = int(offs[g_]), int(offs[g_ + 1])
        rows = np.unique(np.linspace(r0, r1 - 1, 8).astype(np.int64))
        print(f"chain: oracle rows of expert {g_}", flush=True)
        Aq = O.QTensor(np.ascontiguousarray(Xref.codes[token[rows]]), np.ascontiguousarray(Xref.scales[token[rows]]),
                       Xref.ts, rows.size, Hd, O.SCALE_1D)
        mi = np.repeat(np.arange(rows.size), 2 * F)
        ni = np.tile(np.arange(2 * F), rows.size)
        c, wabs = OB.gemm_entries(Aq, w1ref[g_], mi, ni)
        c, wabs = c.reshape(rows.size, 2 * F), wabs.reshape(rows.size, 2 * F)
        G_, U_ = c[:, :F], c[:, F:]
        href = O.swiglu(G_, U_)
        got = W.bf16_bits_to_f32(Hh[rows]).astype(np.float64)
        tol = _swiglu_tol(G_, U_, wabs[:, :F], wabs[:, F:])
        assert (np.abs(got - href) <= tol).all(), f"H of expert {g_} out of tolerance"
        hr_bits = W.f32_to_bf16_bits(href.astype(np.float32))
        # the oracle's quantization of its own H rows with its own amax; a
        # 16-element block is fully determined where its 16 H values agree
        Hq_ref = O.quantize(np.ascontiguousarray(hr_bits), O.BF16, O.ROW_1D, amax_in=a_ref)
        blk_same = np.all((Hh[rows] == hr_bits).reshape(rows.size, F // 16, 16), axis=2)
        blocks_checked += blk_same.size
        blocks_same += int(blk_same.sum())
        gc = Hqh.codes[rows].reshape(rows.size, F // 16, 8)
        rc = Hq_ref.codes.reshape(rows.size, F // 16, 8)
        assert np.array_equal(gc[blk_same], rc[blk_same]), f"quantized H codes, expert {g_}"
        assert np.array_equal(Hqh.scales[rows][blk_same], Hq_ref.scales[blk_same]), f"quantized H scales, expert {g_}"
        # down-projection on the rows whose quantized H is the oracle's throughout
        same = np.all(Hqh.codes[rows] == Hq_ref.codes, axis=1) & np.all(Hqh.scales[rows] == Hq_ref.scales, axis=1)
        rows_checked += rows.size
        rows_same += int(same.sum())
        if not same.any():
            continue
        cols = np.arange(5, Hd, 97)
        sel = np.nonzero(same)[0]
        mi = np.repeat(sel, cols.size)
        ni = np.tile(cols, sel.size)
        Cref, Wref = OB.gemm_entries(Hq_ref, w2ref[g_], mi, ni)
        got_y = Yh[rows[mi], ni]
        tol = gemm_tol(Cref, Wref, True)
        assert (np.abs(got_y - Cref) <= tol).all(), f"down-projection of expert {g_} out of tolerance"
    assert blocks_same >= 0.75 * blocks_checked, f"only {blocks_same} of {blocks_checked} H blocks agree bit for bit"
    assert rows_same >= 0.5 * rows_checked, f"only {rows_same} of {rows_checked} quantized H rows agree"
